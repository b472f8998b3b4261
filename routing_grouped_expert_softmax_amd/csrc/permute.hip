// Permute: group the T*k (token, slot) assignments by expert, on the device, with no host
// synchronisation (the sync-free kernels of the technical summary "使用 Megatron Core 大规模
// 训练混合专家模型（MoE）", section 2.4; the routing metadata -- indices and offsets -- of the
// study notes' case 1).
//
//   1. count:  per chunk of kPermChunk assignments, an LDS histogram over experts.
//   2. scan:   per expert, an exclusive scan over chunks (chunk bases) and the totals;
//              offsets = exclusive scan of the totals.
//   3. rank:   one wavefront per chunk walks its assignments in order, 64 at a time; lanes
//              with the same expert are found with log2(E) ballots, so a row is
//              offset + chunk base + running count + rank among equal lanes: a stable,
//              atomic-free counting sort (rows of an expert in ascending token order).
//   4. copy:   row-major x_perm: one wavefront per token reads the x row once and writes it
//              to its k rows (16-byte accesses); in e4m3 mode the row is quantised per
//              1 x 128 block (MXFP8 mode: per 1 x 32 block with an E8M0 scale) in registers
//              first and the codes and scales are written instead.
//              K-blocked x_perm: a gather by destination rows (perm_gather_kblock_kernel),
//              after a token-order e4m3 quantisation in e4m3 mode.
#include <type_traits>

#include "common.h"
#include "kernels.h"

#ifndef MOE_GATHER_SLICES
#define MOE_GATHER_SLICES 8
#endif
#ifndef MOE_GATHER_NT
#define MOE_GATHER_NT 1
#endif

namespace moe {
namespace {

__global__ __launch_bounds__(256) void perm_count_kernel(const int32_t* __restrict__ idx,
                                                         int A, int E,
                                                         int32_t* __restrict__ chunk_counts) {
    extern __shared__ int32_t hist[];
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
    __syncthreads();
    const int a0 = blockIdx.x * kPermChunk;
    for (int a = a0 + threadIdx.x; a < a0 + kPermChunk && a < A; a += blockDim.x)
        atomicAdd(&hist[idx[a]], 1);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        chunk_counts[(size_t)blockIdx.x * E + e] = hist[e];
}

// Single block of 1024 threads (E <= 1024 is validated by the ABI). counts[e] is expert e's
// demand; offsets scan the kept counts min(counts[e], cap), and offsets[E] is their total.
__global__ __launch_bounds__(1024) void perm_scan_kernel(int32_t* __restrict__ chunk_counts,
                                                         int nchunk, int E, int cap,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets) {
    __shared__ int32_t wsum[16];
    const int e = threadIdx.x;
    int run = 0;
    if (e < E) {
        // batches of 32 independent loads, then the running sum over them
        for (int c0 = 0; c0 < nchunk; c0 += 32) {
            int v[32];
#pragma unroll
            for (int u = 0; u < 32; ++u)
                v[u] = c0 + u < nchunk ? chunk_counts[(size_t)(c0 + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < 32; ++u) {
                if (c0 + u < nchunk) chunk_counts[(size_t)(c0 + u) * E + e] = run;
                run += v[u];
            }
        }
        counts[e] = run;
    }
    const int kept = run < cap ? run : cap;
    // exclusive scan of the kept totals over experts: wavefront inclusive scans, then wave sums
    const int lane = e % kWave, wave = e / kWave;
    int v = kept;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int o = __shfl_up(v, off);
        if (lane >= off) v += o;
    }
    if (lane == kWave - 1) wsum[wave] = v;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    int excl = before + v - kept;
    if (e < E) offsets[e] = excl;
    if (e == E - 1) offsets[E] = excl + kept;
}

// One wavefront per chunk. An assignment whose rank among its expert's assignments (token
// order) reaches cap is dropped: pos = -1, and it takes no row.
__global__ __launch_bounds__(64) void perm_rank_kernel(const int32_t* __restrict__ idx,
                                                       const float* __restrict__ gate, int A,
                                                       int E, int k, int nbits, int cap,
                                                       const int32_t* __restrict__ chunk_base,
                                                       const int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ pos,
                                                       int32_t* __restrict__ src,
                                                       float* __restrict__ gate_perm) {
    extern __shared__ int32_t running[];
    const int lane = threadIdx.x;
    for (int e = lane; e < E; e += kWave) running[e] = chunk_base[(size_t)blockIdx.x * E + e];
    __syncthreads();
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int a0 = blockIdx.x * kPermChunk;
    for (int it = 0; it < kPermChunk; it += kWave) {
        const int a = a0 + it + lane;
        const bool active = a < A;
        const int e = active ? idx[a] : 0;
        uint64_t same = __ballot(active);
        for (int b = 0; b < nbits; ++b) {
            uint64_t ones = __ballot(active && ((e >> b) & 1));
            same &= ((e >> b) & 1) ? ones : ~ones;
        }
        int rank = __popcll(same & lt_mask);
        int base = active ? running[e] : 0;
        __builtin_amdgcn_wave_barrier();
        // the highest lane of each expert group advances that expert's running count
        if (active && (same >> lane) == 1ull) running[e] = base + __popcll(same);
        __builtin_amdgcn_wave_barrier();
        if (active) {
            const int rin = base + rank;                  // rank within the expert
            if (rin < cap) {
                const int row = offsets[e] + rin;
                pos[a] = row;
                src[row] = a / k;
                gate_perm[row] = gate[a];
            } else {
                pos[a] = -1;
            }
        }
        if (a0 + it + kWave >= A) break;
    }
}

// Row copy: 4 tokens per 256-thread block, 16-byte chunks. K-blocked x_perm: 16-byte chunk
// c of row r goes to chunk (c / 4) * A * 4 + r * 4 + c % 4 (64-byte K slices).
__global__ __launch_bounds__(256) void perm_copy_kernel(const uint4* __restrict__ x,
                                                        const int32_t* __restrict__ pos,
                                                        int T, int row_chunks, int k, int kblock,
                                                        uint4* __restrict__ x_perm) {
    constexpr int U = 8;            // 16-byte chunks per lane loaded before the stores
    const size_t A = (size_t)T * k;
    const int lane = threadIdx.x % kWave;
    const int t = blockIdx.x * 4 + threadIdx.x / kWave;
    if (t >= T) return;
    int my_pos = lane < k ? pos[(size_t)t * k + lane] : 0;
    const uint4* xr = x + (size_t)t * row_chunks;
    // every lane runs every iteration so that the shuffles read active lanes only
    for (int c0 = 0; c0 < row_chunks; c0 += U * kWave) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * kWave + lane;
            v[u] = c < row_chunks ? xr[c] : make_uint4(0, 0, 0, 0);
        }
        for (int j = 0; j < k; ++j) {
            const int r = __shfl(my_pos, j);
            if (r < 0) continue;                          // dropped by the capacity
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * kWave + lane;
                if (c >= row_chunks) continue;
                const size_t o = kblock ? ((size_t)(c / 4) * A + r) * 4 + c % 4
                                        : (size_t)r * row_chunks + c;
#if MOE_GATHER_NT
                const i32x4_t q = {(int)v[u].x, (int)v[u].y, (int)v[u].z, (int)v[u].w};
                __builtin_nontemporal_store(q, (i32x4_t*)(x_perm + o));
#else
                x_perm[o] = v[u];
#endif
            }
        }
    }
}

// e4m3 row quantise + copy. A wavefront covers 512 columns per step: 16 lanes per
// 128-column block, 8 bf16 values (16 bytes) per lane.
// K-blocked x_perm: 8-byte chunk c of row r goes to chunk (c / 8) * A * 8 + r * 8 + c % 8.
// MX = false: e4m3 with an fp32 scale per 1 x 128 block (16 lanes per block);
// MX = true:  MXFP8, an E8M0 scale per 1 x 32 block (4 lanes per block).
template <bool MX>
__global__ __launch_bounds__(256) void perm_quant_copy_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ pos, int T, int H, int k,
    int kblock, uint2* __restrict__ x_perm, void* __restrict__ x_perm_scales,
    uint2* __restrict__ x_q, void* __restrict__ x_q_scales) {
    using Sc = typename std::conditional<MX, uint8_t, float>::type;
    constexpr int kLanesPerBlk = MX ? 4 : 16;
    const size_t A = (size_t)T * k;
    const int lane = threadIdx.x % kWave;
    const int t = blockIdx.x * 4 + threadIdx.x / kWave;
    if (t >= T) return;
    int my_pos = lane < k ? pos[(size_t)t * k + lane] : 0;
    const int row_chunks = H / 8;
    const int nblk = H / (8 * kLanesPerBlk);
    const uint4* xr = x + (size_t)t * row_chunks;
    // every lane runs every iteration (shuffles read active lanes only); lane groups stay
    // aligned to the blocks because H % 128 == 0
    for (int c0 = 0; c0 < row_chunks; c0 += kWave) {
        const int c = c0 + lane;
        const bool ok = c < row_chunks;
        uint4 v = ok ? xr[c] : make_uint4(0, 0, 0, 0);
        float f[8];
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = bf16_to_f32((uint16_t)(w[i] & 0xFFFFu));
            f[2 * i + 1] = bf16_to_f32((uint16_t)(w[i] >> 16));
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
        for (int off = 1; off < kLanesPerBlk; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
        uint2 packed;
        Sc sc;
        if (MX) {
            const int X = mx_exponent(amax);
            const float inv = exp2_neg(X);
            packed.x = e4m3x4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv);
            packed.y = e4m3x4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv);
            sc = (Sc)(X + 127);
        } else {
            const float s = e4m3_scale(amax);
            packed.x = e4m3x4(f[0] / s, f[1] / s, f[2] / s, f[3] / s);
            packed.y = e4m3x4(f[4] / s, f[5] / s, f[6] / s, f[7] / s);
            sc = (Sc)s;
        }
        const int blk = c / kLanesPerBlk;
        const bool leader = (c % kLanesPerBlk) == 0;
        if (x_q && ok) {
            x_q[(size_t)t * row_chunks + c] = packed;
            if (leader) ((Sc*)x_q_scales)[(size_t)t * nblk + blk] = sc;
        }
        for (int j = 0; j < k; ++j) {
            int r = __shfl(my_pos, j);
            if (ok && r >= 0) {
                const size_t o = kblock ? ((size_t)(c / 8) * A + r) * 8 + c % 8
                                        : (size_t)r * row_chunks + c;
                x_perm[o] = packed;
                if (leader) ((Sc*)x_perm_scales)[(size_t)r * nblk + blk] = sc;
            }
        }
    }
}

// K-blocked x_perm as a gather: one wavefront per (16 consecutive x_perm rows, up to
// kGatherSlices 64-byte K slices); lane l copies 16 bytes (chunk l % 4 of each slice) of row
// r0 + l / 4 from the row of its token src[r], so every store instruction writes one
// contiguous kilobyte of x_perm. Row bytes: H * 2 (bf16) or H (e4m3 codes, with their
// 1 x 128 scales gathered alongside).
constexpr int kGatherSlices = MOE_GATHER_SLICES;
__global__ __launch_bounds__(256) void perm_gather_kblock_kernel(
    const uint8_t* __restrict__ xin, const int32_t* __restrict__ src, int A,
    const int32_t* __restrict__ live_rows, int row_bytes, uint8_t* __restrict__ x_perm,
    const float* __restrict__ in_scales, int nsc, float* __restrict__ out_scales) {
    const int lane = threadIdx.x % kWave;
    const int64_t w = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    const int slices = row_bytes / 64;
    const int sgroups = (slices + kGatherSlices - 1) / kGatherSlices;
    const int64_t rblocks = (A + 15) / 16;
    if (w >= rblocks * sgroups) return;
    const int rb = (int)(w / sgroups), sg = (int)(w % sgroups);
    const int r = rb * 16 + lane / 4;
    if (r >= *live_rows) return;                      // A, less any dropped assignments
    const int t = src[r];
    const uint8_t* in = xin + (size_t)t * row_bytes + (lane % 4) * 16;
    uint8_t* out = x_perm + (size_t)r * 64 + (lane % 4) * 16;
    const int j0 = sg * kGatherSlices;
    const int j1 = j0 + kGatherSlices < slices ? j0 + kGatherSlices : slices;
    if (j1 - j0 == kGatherSlices) {
        // whole group: every load in flight before the first store
        uint4 v[kGatherSlices];
#pragma unroll
        for (int j = 0; j < kGatherSlices; ++j)
            v[j] = *(const uint4*)(in + (size_t)(j0 + j) * 64);
#pragma unroll
        for (int j = 0; j < kGatherSlices; ++j) {
            uint4* o = (uint4*)(out + (size_t)(j0 + j) * A * 64);
#if MOE_GATHER_NT
            const i32x4_t q = {(int)v[j].x, (int)v[j].y, (int)v[j].z, (int)v[j].w};
            __builtin_nontemporal_store(q, (i32x4_t*)o);
#else
            *o = v[j];
#endif
        }
    } else {
        for (int j = j0; j < j1; ++j)
            *(uint4*)(out + (size_t)j * A * 64) = *(const uint4*)(in + (size_t)j * 64);
    }
    if (out_scales && sg == 0 && lane % 4 == 0)
        for (int b = 0; b < nsc; ++b)
            out_scales[(size_t)r * nsc + b] = in_scales[(size_t)t * nsc + b];
}

// MXFP8 scale words into expert order: out[kb][r] = in[kb][src[r]] for the live rows (both
// blocked; one word = a row's four block codes of 128 columns)
__global__ __launch_bounds__(256) void perm_mx_scale_gather_kernel(
    const uint32_t* __restrict__ in, const int32_t* __restrict__ src,
    const int32_t* __restrict__ live_rows, int A, int T, int nkb, uint32_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)nkb * A) return;
    const int kb = (int)(i / A), r = (int)(i % A);
    if (r >= *live_rows) return;
    out[i] = in[(size_t)kb * T + src[r]];
}

}  // namespace

size_t permute_ws_bytes(int T, int k, int E) {
    size_t A = (size_t)T * k;
    size_t nchunk = (A + kPermChunk - 1) / kPermChunk;
    return nchunk * (size_t)E * sizeof(int32_t);
}

hipError_t launch_permute(int mode, int kblock, int cap, const void* x, const int32_t* topk_idx,
                          const float* topk_gate, int T, int H, int E, int k,
                          int32_t* counts, int32_t* offsets, int32_t* pos, int32_t* src,
                          float* gate_perm, void* x_perm, void* x_perm_scales, void* x_q,
                          void* x_q_scales, void* ws, hipStream_t s) {
    const int A = T * k;
    const int nchunk = (A + kPermChunk - 1) / kPermChunk;
    int32_t* chunk_counts = (int32_t*)ws;
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    perm_count_kernel<<<nchunk, 256, E * sizeof(int32_t), s>>>(topk_idx, A, E, chunk_counts);
    perm_scan_kernel<<<1, 1024, 0, s>>>(chunk_counts, nchunk, E, cap, counts, offsets);
    perm_rank_kernel<<<nchunk, 64, E * sizeof(int32_t), s>>>(topk_idx, topk_gate, A, E, k,
                                                             nbits, cap, chunk_counts, offsets,
                                                             pos, src, gate_perm);
    if (kblock < 0) {           // metadata only (the GEMM gathers the rows itself)
        if (mode == 2)
            return launch_quantize(x, 1, 1, T, H, 1, (uint8_t*)x_q, (float*)x_q_scales, s);
        if (mode == 3) {
            hipError_t e = launch_quantize_mx(x, 1, T, H, 1, (uint8_t*)x_q,
                                              (uint8_t*)x_q_scales, s);
            if (e != hipSuccess || !x_perm_scales) return e;
            const int64_t n = (int64_t)(H / 128) * A;
            perm_mx_scale_gather_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
                (const uint32_t*)x_q_scales, src, offsets + E, A, T, H / 128,
                (uint32_t*)x_perm_scales);
        }
        return hipGetLastError();
    }
    const int blocks = (T + 3) / 4;
    auto gather = [&](const void* in, int row_bytes, const float* in_sc, float* out_sc) {
        const int64_t waves = (int64_t)((A + 15) / 16) *
                              ((row_bytes / 64 + kGatherSlices - 1) / kGatherSlices);
        perm_gather_kblock_kernel<<<(unsigned)((waves + 3) / 4), 256, 0, s>>>(
            (const uint8_t*)in, src, A, offsets + E, row_bytes, (uint8_t*)x_perm, in_sc,
            H / 128, out_sc);
    };
    if (kblock && mode == 1) {
        gather(x, H * 2, nullptr, nullptr);
        return hipGetLastError();
    }
    if (kblock && mode == 2 && x_q) {
        // quantise each token once (token order), then gather codes and scales
        hipError_t e = launch_quantize(x, 1, 1, T, H, 1, (uint8_t*)x_q, (float*)x_q_scales, s);
        if (e != hipSuccess) return e;
        gather(x_q, H, (const float*)x_q_scales, (float*)x_perm_scales);
        return hipGetLastError();
    }
    if (mode == 2) {
        perm_quant_copy_kernel<false><<<blocks, 256, 0, s>>>((const uint4*)x, pos, T, H, k,
                                                             kblock, (uint2*)x_perm,
                                                             x_perm_scales, (uint2*)x_q,
                                                             x_q_scales);
    } else if (mode == 3) {     // row-major only (the ABI rejects a K-blocked MXFP8 x_perm)
        perm_quant_copy_kernel<true><<<blocks, 256, 0, s>>>((const uint4*)x, pos, T, H, k, 0,
                                                            (uint2*)x_perm, x_perm_scales,
                                                            (uint2*)x_q, x_q_scales);
    } else {
        const int elem = mode == 0 ? 4 : 2;
        perm_copy_kernel<<<blocks, 256, 0, s>>>((const uint4*)x, pos, T, H * elem / 16, k,
                                                kblock, (uint4*)x_perm);
    }
    return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, const int32_t* pos, int T, int k, int row_bytes,
                              void* out, hipStream_t s) {
    perm_copy_kernel<<<(T + 3) / 4, 256, 0, s>>>((const uint4*)x, pos, T, row_bytes / 16, k, 0,
                                               (uint4*)out);
    return hipGetLastError();
}

}  // namespace moe

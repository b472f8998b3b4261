// Unpermute / combine: y[t] = sum_j y_perm[pos[t, j]] (+ shared_y[t]), fp32 sum in slot
// order, one rounding to the output dtype; slots dropped by an expert capacity (pos < 0)
// contribute nothing. The gates were folded into the activations
// before the down projection (memory-efficient permutation, technical summary section
// 2.2), so this is a pure gather-sum: no weights, no atomics, deterministic.
//
// e4m3 block quantisation (the FP8 E4M3 format of "万亿参数MoE模型训练的技术挑战",
// section 2.1) of weights (128 x 128 blocks) and activations (1 x 128 blocks) lives here
// too: both are HBM-streaming kernels.
#include <type_traits>

#include "common.h"
#include "kernels.h"

#ifndef MOE_COMBINE_NT
#define MOE_COMBINE_NT 1
#endif
#ifndef MOE_COMBINE_U
#define MOE_COMBINE_U 2
#endif

namespace moe {
namespace {

MOE_DEVICE void add_bf16x8(float (&acc)[8], const uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc[2 * i] += bf16_to_f32((uint16_t)(w[i] & 0xFFFFu));
        acc[2 * i + 1] += bf16_to_f32((uint16_t)(w[i] >> 16));
    }
}

MOE_DEVICE uint4 load_stream(const uint4* p) {
#if MOE_COMBINE_NT
    const i32x4_t q = __builtin_nontemporal_load((const i32x4_t*)p);
    return uint4{(uint32_t)q.x, (uint32_t)q.y, (uint32_t)q.z, (uint32_t)q.w};
#else
    return *p;
#endif
}

// bf16: one wavefront per token, 8 values (16 bytes) per lane per step. KC > 0 is k known at
// compile time: the k row loads of a step are all issued before the first add, so a wave
// keeps k * 1 KB in flight. KC == 0 takes k at run time, one row at a time. Either way the
// adds run in slot order j = 0 .. k - 1, then the shared expert's row.
template <int KC>
__global__ __launch_bounds__(256) void combine_bf16_kernel(const uint4* __restrict__ y_perm,
                                                           const int32_t* __restrict__ pos,
                                                           const uint4* __restrict__ shared_y,
                                                           int T, int row_chunks, int k_rt,
                                                           uint4* __restrict__ y) {
    const int k = KC > 0 ? KC : k_rt;
    const int lane = threadIdx.x % kWave;
    const int t = blockIdx.x * 4 + threadIdx.x / kWave;
    if (t >= T) return;
    const int my_pos = lane < k ? pos[(size_t)t * k + lane] : 0;
    if (KC > 0) {
        // the k rows of the token, read from lanes 0 .. k-1 while every lane is active
        int rj[KC > 0 ? KC : 1];
#pragma unroll
        for (int j = 0; j < KC; ++j) rj[j] = __shfl(my_pos, j);
        // U chunks per lane per step: U * (KC + 1) loads in flight before the first add
        constexpr int U = MOE_COMBINE_U;
        for (int c0 = 0; c0 < row_chunks; c0 += U * kWave) {
            uint4 v[U][KC > 0 ? KC : 1], sv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * kWave + lane;
                const bool ok = c < row_chunks;
#pragma unroll
                for (int j = 0; j < KC; ++j)
                    v[u][j] = ok && rj[j] >= 0
                                  ? load_stream(y_perm + (size_t)rj[j] * row_chunks + c)
                                  : uint4{};
                sv[u] = shared_y && ok ? load_stream(shared_y + (size_t)t * row_chunks + c)
                                       : uint4{};
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * kWave + lane;
                if (c >= row_chunks) continue;
                float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
                for (int j = 0; j < KC; ++j)
                    if (rj[j] >= 0) add_bf16x8(acc, v[u][j]);
                if (shared_y) add_bf16x8(acc, sv[u]);
                uint4 o;
                o.x = pack_bf16x2(acc[0], acc[1]);
                o.y = pack_bf16x2(acc[2], acc[3]);
                o.z = pack_bf16x2(acc[4], acc[5]);
                o.w = pack_bf16x2(acc[6], acc[7]);
                y[(size_t)t * row_chunks + c] = o;
            }
        }
        return;
    }
    for (int c0 = 0; c0 < row_chunks; c0 += kWave) {
        const int c = c0 + lane;
        const bool ok = c < row_chunks;
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int j = 0; j < k; ++j) {
            const int r = __shfl(my_pos, j);
            if (ok && r >= 0) add_bf16x8(acc, y_perm[(size_t)r * row_chunks + c]);
        }
        if (shared_y && ok) add_bf16x8(acc, shared_y[(size_t)t * row_chunks + c]);
        if (!ok) continue;
        uint4 o;
        o.x = pack_bf16x2(acc[0], acc[1]);
        o.y = pack_bf16x2(acc[2], acc[3]);
        o.z = pack_bf16x2(acc[4], acc[5]);
        o.w = pack_bf16x2(acc[6], acc[7]);
        y[(size_t)t * row_chunks + c] = o;
    }
}

// fp32: 4 values (16 bytes) per lane per step.
__global__ __launch_bounds__(256) void combine_f32_kernel(const float4* __restrict__ y_perm,
                                                          const int32_t* __restrict__ pos,
                                                          const float4* __restrict__ shared_y,
                                                          int T, int row_chunks, int k,
                                                          float4* __restrict__ y) {
    const int lane = threadIdx.x % kWave;
    const int t = blockIdx.x * 4 + threadIdx.x / kWave;
    if (t >= T) return;
    int my_pos = lane < k ? pos[(size_t)t * k + lane] : 0;
    for (int c0 = 0; c0 < row_chunks; c0 += kWave) {
        const int c = c0 + lane;
        const bool ok = c < row_chunks;
        float4 acc = make_float4(0, 0, 0, 0);
        for (int j = 0; j < k; ++j) {
            int r = __shfl(my_pos, j);
            if (ok && r >= 0) {
                float4 v = y_perm[(size_t)r * row_chunks + c];
                acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
            }
        }
        if (!ok) continue;
        if (shared_y) {
            float4 v = shared_y[(size_t)t * row_chunks + c];
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        y[(size_t)t * row_chunks + c] = acc;
    }
}

// Eight consecutive values from element i (i a multiple of 8) as fp32: one 16-byte load for
// bf16, two for fp32.
MOE_DEVICE void load8_f32(const void* p, int dtype, size_t i, float (&f)[8]) {
    if (dtype == 0) {
        const float4 a = *(const float4*)((const float*)p + i);
        const float4 b = *(const float4*)((const float*)p + i + 4);
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
        f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    } else {
        const uint4 v = *(const uint4*)((const uint16_t*)p + i);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            f[2 * u] = bf16_to_f32((uint16_t)(w[u] & 0xFFFFu));
            f[2 * u + 1] = bf16_to_f32((uint16_t)(w[u] >> 16));
        }
    }
}

// Activation quantiser, 1 x 128 blocks: one wavefront per 128-column block... per row:
// each 16-lane group handles one block, 8 values per lane.
__global__ __launch_bounds__(256) void quant_rows_kernel(const void* __restrict__ in,
                                                         int in_dtype, int64_t rows, int cols,
                                                         uint8_t* __restrict__ q,
                                                         float* __restrict__ scales) {
    const int64_t nblk_row = cols / 128;
    const int64_t gblk = (int64_t)blockIdx.x * 16 + threadIdx.x / 16;   // global block id
    const int sub = threadIdx.x % 16;
    const bool ok = gblk < rows * nblk_row;
    const int64_t r = ok ? gblk / nblk_row : 0;
    const int64_t b = ok ? gblk % nblk_row : 0;
    const size_t base = (size_t)r * cols + (size_t)b * 128 + sub * 8;
    float f[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (ok) load8_f32(in, in_dtype, base, f);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    float sc = e4m3_scale(amax);
    if (!ok) return;
    uint2 packed;
    packed.x = e4m3x4(f[0] / sc, f[1] / sc, f[2] / sc, f[3] / sc);
    packed.y = e4m3x4(f[4] / sc, f[5] / sc, f[6] / sc, f[7] / sc);
    *(uint2*)(q + base) = packed;
    if (sub == 0) scales[gblk] = sc;
}

// MXFP8 quantiser, 1 x 32 blocks along the rows (activations and weights alike): four lanes
// per block, eight values per lane; the block's amax takes two butterflies. Scale bytes are
// row-major [R, cols/32] (blocked_rows == 0) or blocked [cols/128][R][4] (blocked_rows = R):
// the four codes of one row's 128 columns form one word, and the words of consecutive rows
// are adjacent.
__global__ __launch_bounds__(256) void quant_mx_kernel(const void* __restrict__ in, int in_dtype,
                                                       int64_t nblk, int cols, int blocked_rows,
                                                       uint8_t* __restrict__ q,
                                                       uint8_t* __restrict__ scales) {
    const int64_t blk = (int64_t)blockIdx.x * 64 + threadIdx.x / 4;   // 32-value block
    const int sub = threadIdx.x % 4;
    const bool ok = blk < nblk;
    const size_t base = (size_t)(ok ? blk : 0) * 32 + sub * 8;
    float f[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (ok) load8_f32(in, in_dtype, base, f);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    if (!ok) return;
    const int X = mx_exponent(amax);
    const float inv = exp2_neg(X);
    uint2 packed;
    packed.x = e4m3x4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv);
    packed.y = e4m3x4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv);
    *(uint2*)(q + base) = packed;
    if (sub == 0) {
        size_t si = (size_t)blk;
        if (blocked_rows > 0) {
            const int nb = cols / 32;
            const int64_t r = blk / nb;
            const int b = (int)(blk % nb);
            si = ((size_t)(b / 4) * blocked_rows + r) * 4 + b % 4;
        }
        scales[si] = (uint8_t)(X + 127);
    }
}

// [n, rows, cols4] 4-byte words -> [n][cols4][rows]: MXFP8 weight scales (one word = a row's
// four block codes of 128 K) into the blocked order of K-blocked weights.
__global__ __launch_bounds__(256) void pack_mx_scales_kernel(const uint32_t* __restrict__ in,
                                                             int64_t total, int rows, int cols4,
                                                             uint32_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int64_t per = (int64_t)rows * cols4;
    const int64_t m = i / per, rem = i % per;
    const int kb = (int)(rem / rows), r = (int)(rem % rows);
    out[i] = in[(m * rows + r) * cols4 + kb];
}

// Weight quantiser, 128 x 128 blocks: one 256-thread block per quantisation block; each
// thread handles half a row (64 values) of the block.
__global__ __launch_bounds__(256) void quant_weight_kernel(const void* __restrict__ in,
                                                           int in_dtype, int rows, int cols,
                                                           uint8_t* __restrict__ q,
                                                           float* __restrict__ scales) {
    __shared__ float red[4];
    const int nbr = rows / 128, nbc = cols / 128;
    const int64_t blk = blockIdx.x;                       // [mat, br, bc]
    const int64_t mat = blk / ((int64_t)nbr * nbc);
    const int br = (int)((blk / nbc) % nbr);
    const int bc = (int)(blk % nbc);
    const int r = br * 128 + threadIdx.x / 2;
    const int c0 = bc * 128 + (threadIdx.x % 2) * 64;
    const size_t base = ((size_t)mat * rows + r) * (size_t)cols + c0;
    float f[64];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        float g[8];
        load8_f32(in, in_dtype, base + 8 * u, g);
#pragma unroll
        for (int i = 0; i < 8; ++i) f[8 * u + i] = g[i];
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float sc = e4m3_scale(amax);
#pragma unroll
    for (int i = 0; i < 64; i += 16) {
        uint32_t w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            w[u] = e4m3x4(f[i + 4 * u] / sc, f[i + 4 * u + 1] / sc, f[i + 4 * u + 2] / sc,
                          f[i + 4 * u + 3] / sc);
        *(uint4*)(q + base + i) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    if (threadIdx.x == 0) scales[blk] = sc;
}

// K-blocked re-layout: one wavefront per (matrix, 64-byte K slice, 16 rows); lane l copies
// 16 bytes: row 16 * blockrow + l / 4, chunk l % 4. Reads are 64-byte row pieces, writes one
// contiguous kilobyte.
__global__ __launch_bounds__(256) void pack_kblock_kernel(const uint4* __restrict__ in,
                                                          int64_t n_mat, int rows,
                                                          int row_chunks, uint4* __restrict__ out) {
    const int lane = threadIdx.x % kWave;
    const int64_t w = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    const int row_groups = (rows + 15) / 16;
    const int slices = row_chunks / 4;
    const int64_t total = n_mat * slices * row_groups;
    if (w >= total) return;
    const int64_t mat = w / ((int64_t)slices * row_groups);
    const int rem = (int)(w % ((int64_t)slices * row_groups));
    const int j = rem / row_groups, rg = rem % row_groups;
    const int r = rg * 16 + lane / 4, c = lane % 4;
    if (r >= rows) return;
    const size_t mbase = (size_t)mat * rows * row_chunks;
    out[mbase + ((size_t)j * rows + r) * 4 + c] = in[mbase + (size_t)r * row_chunks + j * 4 + c];
}

// y += a, elementwise over n bf16 values (n % 8 == 0), summed in fp32 and rounded once.
__global__ __launch_bounds__(256) void add_bf16_kernel(uint4* __restrict__ y,
                                                       const uint4* __restrict__ a,
                                                       int64_t n8) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    add_bf16x8(acc, y[i]);
    add_bf16x8(acc, a[i]);
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    y[i] = o;
}

}  // namespace

hipError_t launch_pack_kblock(const void* in, int64_t n_mat, int rows, int cols, int elem_bytes,
                              void* out, hipStream_t s) {
    const int row_chunks = (int)((int64_t)cols * elem_bytes / 16);
    const int64_t waves = n_mat * (row_chunks / 4) * (int64_t)((rows + 15) / 16);
    pack_kblock_kernel<<<(unsigned)((waves + 3) / 4), 256, 0, s>>>((const uint4*)in, n_mat, rows,
                                                                   row_chunks, (uint4*)out);
    return hipGetLastError();
}

hipError_t launch_combine(int act_dtype, const void* y_perm, const int32_t* pos,
                          const void* shared_y, int T, int H, int k, void* y, hipStream_t s) {
    const int blocks = (T + 3) / 4;
    if (act_dtype == 0)
        combine_f32_kernel<<<blocks, 256, 0, s>>>((const float4*)y_perm, pos,
                                                  (const float4*)shared_y, T, H / 4, k,
                                                  (float4*)y);
    else {
        auto run = [&](auto kc) {
            combine_bf16_kernel<decltype(kc)::value><<<blocks, 256, 0, s>>>(
                (const uint4*)y_perm, pos, (const uint4*)shared_y, T, H / 8, k, (uint4*)y);
        };
        switch (k) {
        case 1: run(std::integral_constant<int, 1>{}); break;
        case 2: run(std::integral_constant<int, 2>{}); break;
        case 4: run(std::integral_constant<int, 4>{}); break;
        case 6: run(std::integral_constant<int, 6>{}); break;
        case 8: run(std::integral_constant<int, 8>{}); break;
        default: run(std::integral_constant<int, 0>{}); break;
        }
    }
    return hipGetLastError();
}

hipError_t launch_quantize(const void* in, int in_dtype, int64_t n_mat, int rows, int cols,
                           int block_rows, uint8_t* q, float* scales, hipStream_t s) {
    if (block_rows == 1) {
        int64_t nblocks = n_mat * rows * (int64_t)(cols / 128);
        quant_rows_kernel<<<(unsigned)((nblocks + 15) / 16), 256, 0, s>>>(
            in, in_dtype, n_mat * rows, cols, q, scales);
    } else {
        int64_t nblocks = n_mat * (int64_t)(rows / 128) * (cols / 128);
        quant_weight_kernel<<<(unsigned)nblocks, 256, 0, s>>>(in, in_dtype, rows, cols, q,
                                                              scales);
    }
    return hipGetLastError();
}

hipError_t launch_quantize_mx(const void* in, int in_dtype, int64_t rows, int cols,
                              int blocked, uint8_t* q, uint8_t* scales, hipStream_t s) {
    const int64_t nblk = rows * (cols / 32);
    if (nblk > 0)
        quant_mx_kernel<<<(unsigned)((nblk + 63) / 64), 256, 0, s>>>(
            in, in_dtype, nblk, cols, blocked ? (int)rows : 0, q, scales);
    return hipGetLastError();
}

hipError_t launch_pack_mx_scales(const uint8_t* in, int64_t n_mat, int rows, int cols,
                                 uint8_t* out, hipStream_t s) {
    const int64_t total = n_mat * rows * (int64_t)(cols / 4);
    if (total > 0)
        pack_mx_scales_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(
            (const uint32_t*)in, total, rows, cols / 4, (uint32_t*)out);
    return hipGetLastError();
}

hipError_t launch_add_bf16(void* y, const void* a, int64_t n, hipStream_t s) {
    const int64_t n8 = n / 8;
    add_bf16_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>((uint4*)y, (const uint4*)a, n8);
    return hipGetLastError();
}

}  // namespace moe

// Backward of the SwiGLU expert MLP with the gate folded into the activation, as grouped
// GEMMs on bf16 MFMA (fp32 accumulation), data and weight gradients as separate launches
// (the W/D split of the technical summary "使用 Megatron Core 大规模训练混合专家模型（MoE）",
// section 2.3). Per expert e with rows R_e and h = silu(Z_g) * Z_u:
//
//   dA      = dy_perm[R_e] W2_e            (dgrad 1; epilogue: SwiGLU backward)
//   dg[r]   = sum_f dA[r, f] h[r, f]
//   dZ_g    = g dA Z_u silu'(Z_g),   dZ_u = g dA silu(Z_g)
//   dx_perm = dZ W13_e                     (dgrad 2)
//   dW2_e   = dy_perm[R_e]^T act[R_e]      (wgrad 2)
//   dW13_e  = dZ[R_e]^T x_perm[R_e]        (wgrad 1)
//
// Every operand is read straight from its row-major storage. An operand whose K index is
// its row index (W2_e and W13_e in the data gradients, all four operands of the weight
// gradients) is staged in LDS as [k][m] and turned into MFMA fragments by the transposing
// LDS read ds_read_b64_tr_b16: within 16 lanes, lane i receives the four values of column
// n0 + i from rows k0 .. k0 + 3 when lane L points at row k0 + L / 4, column n0 + 4 (L % 4).
// The weight gradients run K (an expert's rows) to a ragged end: rows past it are loaded
// from a zeroed page of the workspace. dg is reduced per tile and then over tiles in a fixed
// order, so the whole backward is deterministic (no atomics).
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kBM = 128, kBN = 128, kBK = 32, kStages = 3;
constexpr int kWaves = 4, kThreads = kWaves * 64;          // 2 x 2 waves of 64 x 64
constexpr int kOpBytes = 8192;                             // one operand tile per stage
constexpr int kStageBytes = 2 * kOpBytes;
constexpr int kTN = 2, kTM = 2;                            // 32 x 32 sub-tiles per wave
constexpr int kZeroBytes = 1024;

enum { OPK = 0, OPT = 1 };        // operand rows hold K (contiguous) / hold M or N

struct Operand {
    const uint16_t* p;
    size_t ld;                    // elements between rows of the stored matrix
    size_t gstride;               // elements between groups (weights); 0 = rows are global
};

struct BwdArgs {
    Operand a, b;
    const int32_t* offsets;
    const int4* tiles;            // ragged-M mode: tile list and count
    const int* total;
    int M, N, K;                  // ragged-M: N, K; ragged-K: M, N (K = rows of the group)
    int ntm, ntn;
    int groups;
    uint16_t* out;
    size_t out_ld, out_gstride;
    // dgrad-1 epilogue
    const uint16_t* z;
    const float* gate;
    uint16_t* dz;
    float* dg_part;
    int F;
    const uint8_t* zero;
};

// swizzle of the 16-byte chunks of a [k][128] operand row: the four rows one transposing read
// touches land in four different 32-byte bank groups
MOE_DEVICE int swz_t(int k) { return 2 * (k & 3); }

MOE_DEVICE bf16x8_t tr_frag(const uint8_t* lo, const uint8_t* hi) {
    typedef short s4 __attribute__((ext_vector_type(4)));
    const s4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS s4*)(MOE_LDS void*)lo);
    const s4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS s4*)(MOE_LDS void*)hi);
    typedef short s8 __attribute__((ext_vector_type(8)));
    const s8 v = s8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(bf16x8_t, v);
}

// RAGGED_K = 0: tiles of ragged M from the schedule, K fixed. RAGGED_K = 1: tiles of every
// group's [M, N], K = the group's rows. EPI 0: bf16 store; EPI 1: SwiGLU backward.
template <int AO, int BO, int RAGGED_K, int EPI>
__global__ __launch_bounds__(kThreads) void bwd_gemm_kernel(BwdArgs ba) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
    const int wm = wave / 2, wn = wave % 2;
    // ---- tile
    int g, m0, Mg, rbase, mt, nt;
    {
        const int b = blockIdx.x, xcd = b % 8, i = b / 8;
        const int total = RAGGED_K ? ba.groups * ba.ntm * ba.ntn : *ba.total * ba.ntn;
        const int per = (total + 7) / 8;
        if (i >= per) return;
        const int L = xcd * per + i;
        if (L >= total) return;
        if (RAGGED_K) {
            g = L / (ba.ntm * ba.ntn);
            const int rem = L % (ba.ntm * ba.ntn);
            mt = rem / ba.ntn;
            nt = rem % ba.ntn;
            rbase = ba.offsets[g];
            Mg = ba.offsets[g + 1] - rbase;
            m0 = mt * kBM;
        } else {
            const int4 ti = ba.tiles[L / ba.ntn];
            nt = L % ba.ntn;
            g = ti.x & 0xFFFFF;
            m0 = ti.y;
            Mg = ti.z;
            rbase = ti.w;
            mt = 0;
        }
    }
    const int nk = RAGGED_K ? (Mg + kBK - 1) / kBK : ba.K / kBK;
    const int live = RAGGED_K ? kBM : (Mg - m0 < kBM ? Mg - m0 : kBM);

    // ---- DMA sources. Operand tile = 8 instructions of 1 KB; wave w issues q = w, w + 4.
    // OPK tile [128 rows][32 k]: instruction q fills rows 16 q + lane / 4.
    // OPT tile [32 k][128 cols]: instruction q fills k rows 4 q + lane / 16.
    const uint8_t* srcA[2];
    const uint8_t* srcB[2];
    int ka[2], kb[2];               // OPT: the k row each instruction fills (ragged K)
    auto op_src = [&](const Operand& op, int o, bool is_a, int q, const uint8_t*& src, int& krow) {
        if (o == OPK) {
            const int r = 16 * q + lane / 4;
            const int c = (lane % 4) ^ chunk_swz<4>(r);
            size_t row;
            if (is_a) {                       // ragged-M activations: global rows, clamped
                const int rr = m0 + r < Mg ? m0 + r : Mg - 1;
                row = (size_t)rbase + rr;
            } else {
                row = (size_t)nt * kBN + r;
            }
            src = (const uint8_t*)(op.p + (size_t)g * op.gstride + row * op.ld) + c * 16;
            krow = 0;
        } else {
            const int kr = 4 * q + lane / 16;
            const int c = (lane % 16) ^ swz_t(kr);
            const size_t col = (size_t)(is_a ? mt * kBM : nt * kBN) + c * 8;
            if (RAGGED_K)
                src = (const uint8_t*)(op.p + (size_t)rbase * op.ld + col);   // + k * ld
            else
                src = (const uint8_t*)(op.p + (size_t)g * op.gstride + col);  // + k * ld
            krow = kr;
        }
    };
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        op_src(ba.a, AO, true, wave + 4 * u, srcA[u], ka[u]);
        op_src(ba.b, BO, false, wave + 4 * u, srcB[u], kb[u]);
    }
    auto issue = [&](int kstep, int stage) {
        MOE_LDS uint8_t* base = (MOE_LDS uint8_t*)lds + stage * kStageBytes;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int q = wave + 4 * u;
            // A
            const uint8_t* sa;
            if (AO == OPK) {
                sa = srcA[u] + (size_t)kstep * kBK * 2;
            } else {
                const int kk = kstep * kBK + ka[u];
                sa = (RAGGED_K && kk >= Mg) ? ba.zero + (lane % 16) * 16
                                            : srcA[u] + (size_t)kk * ba.a.ld * 2;
            }
            __builtin_amdgcn_global_load_lds((const void*)sa, (MOE_LDS void*)(base + q * 1024),
                                             16, 0, 0);
            // B
            const uint8_t* sb;
            if (BO == OPK) {
                sb = srcB[u] + (size_t)kstep * kBK * 2;
            } else {
                const int kk = kstep * kBK + kb[u];
                sb = (RAGGED_K && kk >= Mg) ? ba.zero + (lane % 16) * 16
                                            : srcB[u] + (size_t)kk * ba.b.ld * 2;
            }
            __builtin_amdgcn_global_load_lds((const void*)sb,
                                             (MOE_LDS void*)(base + kOpBytes + q * 1024), 16, 0, 0);
        }
    };

    // ---- fragment addresses (bytes within an operand tile)
    // OPK: row (sub-tile base + lane % 32), chunk (2 s + lane / 32) ^ swz
    // OPT: k rows 16 s + 8 (h / 2) + u / 4 (+ 4), column base + 16 (h % 2) + 4 (u % 4)
    const int h16 = lane / 16, u16 = lane % 16;
    int offK[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) offK[s] = ((2 * s + lane / 32) ^ chunk_swz<4>(lane % 32)) * 16;
    auto frag = [&](const uint8_t* tile, int o, int sub_base, int s) -> bf16x8_t {
        if (o == OPK) {
            return *(const bf16x8_t*)(tile + (sub_base + lane % 32) * 64 + offK[s]);
        } else {
            const int k0 = 16 * s + 8 * (h16 / 2) + u16 / 4;
            const int col = sub_base + 16 * (h16 % 2) + 4 * (u16 % 4);
            const int chunk = (col / 8) ^ swz_t(k0);          // k0 and k0 + 4 share swz_t
            const int off = chunk * 16 + (col % 8) * 2;
            return tr_frag(tile + k0 * 256 + off, tile + (k0 + 4) * 256 + off);
        }
    };

    f32x16_t acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[i][j] = f32x16_t{};
    int nvi = (live - wm * 64 + 31) / 32;
    nvi = nvi < 0 ? 0 : (nvi > kTM ? kTM : nvi);
    nvi = __builtin_amdgcn_readfirstlane(nvi);

#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
        if (s < nk) issue(s, s);
    int stage = 0;
    for (int kt = 0; kt < nk; ++kt) {
        const int later = nk - 1 - kt;
        if (later >= 1) wait_vm_lgkm0<4>();
        else wait_vm_lgkm0<0>();
        block_sync();
        {
            const int kn = kt + kStages - 1;
            int sn = stage + kStages - 1;
            if (sn >= kStages) sn -= kStages;
            if (kn < nk) issue(kn, sn);
        }
        const uint8_t* ta = lds + stage * kStageBytes;
        const uint8_t* tb = ta + kOpBytes;
        if (nvi > 0) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                bf16x8_t av[kTM], bv[kTN];
#pragma unroll
                for (int j = 0; j < kTN; ++j) bv[j] = frag(tb, BO, wn * 64 + j * 32, s);
#pragma unroll
                for (int i = 0; i < kTM; ++i) av[i] = frag(ta, AO, wm * 64 + i * 32, s);
#pragma unroll
                for (int i = 0; i < kTM; ++i)
#pragma unroll
                    for (int j = 0; j < kTN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j],
                                                                            acc[i][j], 0, 0, 0);
            }
        }
        if (++stage == kStages) stage = 0;
    }

    // ---- epilogue. 32x32 layout: element r of lane l is row (r/4)*8 + (l/32)*4 + r%4,
    // column l % 32.
    if (EPI == 0) {
        uint16_t* out = ba.out + (RAGGED_K ? (size_t)g * ba.out_gstride : 0);
#pragma unroll
        for (int i = 0; i < kTM; ++i) {
            if (i >= nvi) continue;
#pragma unroll
            for (int j = 0; j < kTN; ++j) {
                const int col = nt * kBN + wn * 64 + j * 32 + lane % 32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = wm * 64 + i * 32 + (r / 4) * 8 + (lane / 32) * 4 + r % 4;
                    size_t orow;
                    if (RAGGED_K) {
                        orow = (size_t)mt * kBM + row;
                    } else {
                        if (m0 + row >= Mg) continue;
                        orow = (size_t)rbase + m0 + row;
                    }
                    out[orow * ba.out_ld + col] = f32_to_bf16(acc[i][j][r]);
                }
            }
        }
        return;
    }
    // SwiGLU backward on the dA tile (columns f of this N tile); dg partial per row
    const int F = ba.F;
    float dgp[kTM][16];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dgp[i][r] = 0.0f;
            const int row = wm * 64 + i * 32 + (r / 4) * 8 + (lane / 32) * 4 + r % 4;
            if (i >= nvi || m0 + row >= Mg) continue;
            const size_t grow = (size_t)rbase + m0 + row;
            const float gt = ba.gate ? ba.gate[grow] : 1.0f;
#pragma unroll
            for (int j = 0; j < kTN; ++j) {
                const int f = nt * kBN + wn * 64 + j * 32 + lane % 32;
                const float zg = bf16_to_f32(ba.z[grow * 2 * F + f]);
                const float zu = bf16_to_f32(ba.z[grow * 2 * F + F + f]);
                const float sg = 1.0f / (1.0f + expf(-zg));
                const float si = zg * sg;
                const float ds = sg * (1.0f + zg * (1.0f - sg));
                const float da = acc[i][j][r];
                const float dh = gt * da;
                ba.dz[grow * 2 * F + f] = f32_to_bf16(dh * zu * ds);
                ba.dz[grow * 2 * F + F + f] = f32_to_bf16(dh * si);
                dgp[i][r] += da * (si * zu);
            }
        }
    // rows' partial sums: over the 32 lanes of each half (columns), then over the two waves
    // of a row band (LDS), in a fixed order
    block_sync();
    float* red = (float*)lds;                          // [2][kBM]
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float v = dgp[i][r];
#pragma unroll
            for (int off = 1; off < 32; off <<= 1) v += __shfl_xor(v, off);
            const int row = wm * 64 + i * 32 + (r / 4) * 8 + (lane / 32) * 4 + r % 4;
            if (lane % 32 == 0) red[wn * kBM + row] = v;
        }
    __syncthreads();
    if (threadIdx.x < kBM) {
        const int row = threadIdx.x;
        if (m0 + row < Mg) {
            const size_t grow = (size_t)rbase + m0 + row;
            ba.dg_part[grow * ba.ntn + nt] = red[row] + red[kBM + row];
        }
    }
}

__global__ __launch_bounds__(256) void dg_reduce_kernel(const float* __restrict__ part, int A,
                                                        int ntn, float* __restrict__ dg) {
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r >= A) return;
    float s = 0.0f;
    for (int t = 0; t < ntn; ++t) s += part[(size_t)r * ntn + t];
    dg[r] = s;
}

__global__ __launch_bounds__(256) void zero_fill_kernel(uint32_t* p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

template <int AO, int BO, int RAGGED_K, int EPI>
hipError_t run_bwd(const BwdArgs& ba, int nblocks, hipStream_t s) {
    static bool attr_set = false;
    constexpr int lds_bytes = kStages * kStageBytes;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)bwd_gemm_kernel<AO, BO, RAGGED_K, EPI>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    if (nblocks > 0)
        bwd_gemm_kernel<AO, BO, RAGGED_K, EPI><<<nblocks, kThreads, lds_bytes, s>>>(ba);
    return hipGetLastError();
}

struct BwdWs {
    void* sched;
    uint8_t* zero;
    uint16_t* dz;
    float* dg_part;
    size_t total;
};

size_t al(size_t v) { return (v + 255) / 256 * 256; }

BwdWs carve_bwd(void* ws, int A, int E, int F) {
    BwdWs w;
    char* p = (char*)ws;
    size_t off = 0;
    w.sched = p ? p + off : nullptr;
    off += al(schedule_ws_bytes(A, E, kBM));
    w.zero = p ? (uint8_t*)(p + off) : nullptr;
    off += al(kZeroBytes);
    w.dz = p ? (uint16_t*)(p + off) : nullptr;
    off += al((size_t)A * 2 * F * 2);
    w.dg_part = p ? (float*)(p + off) : nullptr;
    off += al((size_t)A * (F / kBN) * 4);
    w.total = off;
    return w;
}

}  // namespace

size_t bwd_ws_bytes(int T, int k, int E, int H, int F) {
    (void)H;
    return carve_bwd(nullptr, T * k, E, F).total;
}

hipError_t launch_grouped_gemm_bwd(const void* dy_perm, const void* x_perm, const void* z,
                                   const void* act, const float* gate_perm,
                                   const int32_t* offsets, const void* w13, const void* w2,
                                   int A, int E, int H, int F, void* dx_perm, void* dw13,
                                   void* dw2, float* dgate_perm, void* ws, hipStream_t s) {
    BwdWs w = carve_bwd(ws, A, E, F);
    zero_fill_kernel<<<1, 256, 0, s>>>((uint32_t*)w.zero, kZeroBytes / 4);
    hipError_t e = launch_schedule(offsets, E, kBM, w.sched, s);
    if (e != hipSuccess) return e;
    const int4* tiles = (const int4*)((char*)w.sched + 256);
    const int* total = (const int*)w.sched;
    const size_t max_tiles = (size_t)(A + kBM - 1) / kBM + (size_t)E;
    const uint16_t* DY = (const uint16_t*)dy_perm;
    const uint16_t* X = (const uint16_t*)x_perm;
    const uint16_t* W13 = (const uint16_t*)w13;
    const uint16_t* W2 = (const uint16_t*)w2;
    auto round8 = [](size_t n) { return (int)((n + 7) / 8 * 8); };

    // dgrad 1: dA [A, F] = dy_perm W2_e (W2_e stored [H][F]: K rows) -> dZ, dg partials
    BwdArgs d1 = {};
    d1.a = {DY, (size_t)H, 0};
    d1.b = {W2, (size_t)F, (size_t)H * F};
    d1.offsets = offsets; d1.tiles = tiles; d1.total = total;
    d1.N = F; d1.K = H; d1.ntn = F / kBN; d1.groups = E;
    d1.z = (const uint16_t*)z; d1.gate = gate_perm; d1.dz = w.dz; d1.dg_part = w.dg_part;
    d1.F = F; d1.zero = w.zero;
    e = run_bwd<OPK, OPT, 0, 1>(d1, round8(max_tiles * d1.ntn), s);
    if (e != hipSuccess) return e;
    if (dgate_perm) {
        dg_reduce_kernel<<<(A + 255) / 256, 256, 0, s>>>(w.dg_part, A, F / kBN, dgate_perm);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // dgrad 2: dx_perm [A, H] = dZ W13_e (W13_e stored [2F][H]: K rows)
    BwdArgs d2 = {};
    d2.a = {w.dz, (size_t)2 * F, 0};
    d2.b = {W13, (size_t)H, (size_t)2 * F * H};
    d2.offsets = offsets; d2.tiles = tiles; d2.total = total;
    d2.N = H; d2.K = 2 * F; d2.ntn = H / kBN; d2.groups = E;
    d2.out = (uint16_t*)dx_perm; d2.out_ld = H; d2.zero = w.zero;
    e = run_bwd<OPK, OPT, 0, 0>(d2, round8(max_tiles * d2.ntn), s);
    if (e != hipSuccess) return e;
    // wgrad 2: dW2_e [H, F] = dy_perm[R_e]^T act[R_e]
    BwdArgs w2a = {};
    w2a.a = {DY, (size_t)H, 0};
    w2a.b = {(const uint16_t*)act, (size_t)F, 0};
    w2a.offsets = offsets; w2a.M = H; w2a.N = F; w2a.ntm = H / kBM; w2a.ntn = F / kBN;
    w2a.groups = E; w2a.out = (uint16_t*)dw2; w2a.out_ld = F; w2a.out_gstride = (size_t)H * F;
    w2a.zero = w.zero;
    e = run_bwd<OPT, OPT, 1, 0>(w2a, round8((size_t)E * w2a.ntm * w2a.ntn), s);
    if (e != hipSuccess) return e;
    // wgrad 1: dW13_e [2F, H] = dZ[R_e]^T x_perm[R_e]
    BwdArgs w1 = {};
    w1.a = {w.dz, (size_t)2 * F, 0};
    w1.b = {X, (size_t)H, 0};
    w1.offsets = offsets; w1.M = 2 * F; w1.N = H; w1.ntm = 2 * F / kBM; w1.ntn = H / kBN;
    w1.groups = E; w1.out = (uint16_t*)dw13; w1.out_ld = H; w1.out_gstride = (size_t)2 * F * H;
    w1.zero = w.zero;
    return run_bwd<OPT, OPT, 1, 0>(w1, round8((size_t)E * w1.ntm * w1.ntn), s);
}

}  // namespace moe

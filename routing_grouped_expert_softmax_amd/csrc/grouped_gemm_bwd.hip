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
#include <climits>
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// weight gradients dealt over the XCDs by a group plan (wgrad_plan_kernel), else in
// contiguous runs
#ifndef MOE_BWD_PLAN
#define MOE_BWD_PLAN 1
#endif
#ifndef MOE_BWD_LARGE
#define MOE_BWD_LARGE 1
#endif
#ifndef MOE_BWD_LARGE_BK
#define MOE_BWD_LARGE_BK 64
#endif
#ifndef MOE_BWD_LARGE_STAGES
#define MOE_BWD_LARGE_STAGES 2
#endif


constexpr int kZeroBytes = 1024;

// Tile configuration: BM x BN output tile, WM x WN waves, each wave (BM / WM) x (BN / WN) in
// 32 x 32 MFMA sub-tiles; K step BK (32 or 64), an LDS ring of STAGES steps.
template <int BM_, int BN_, int WM_, int WN_, int BK_ = 32, int STAGES_ = 3>
struct BwdCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int kBK = BK_, kStages = STAGES_;
    static constexpr int kCpr = kBK / 8;                  // 16-byte chunks of a K-major row
    static constexpr int kSub = kBK / 16;                 // MFMA K steps per stage
    static_assert(kBK == 32 || kBK == 64, "BK");
    static_assert(kStages >= 2, "stages");
    static constexpr int kWaves = WM * WN, kThreads = kWaves * 64;
    static constexpr int kTM = BM / WM / 32, kTN = BN / WN / 32;
    static constexpr int kABytes = BM * kBK * 2, kBBytes = BN * kBK * 2;
    static constexpr int kStageBytes = kABytes + kBBytes;
    static constexpr int kLdsLoop = kStages * kStageBytes;
    static constexpr int kLdsEp = BM * (BN + 8) * 2;          // bf16 epilogue staging
    static constexpr int kLds = kLdsLoop > kLdsEp ? kLdsLoop : kLdsEp;
    static_assert(kLds <= 160 * 1024, "LDS");
    static constexpr int kDmaA = kABytes / 1024 / kWaves, kDmaB = kBBytes / 1024 / kWaves;
    static_assert(kDmaA * 1024 * kWaves == kABytes && kDmaB * 1024 * kWaves == kBBytes, "DMA");
    static_assert(kTM >= 1 && kTN >= 1, "waves");
};
using BwdSmall = BwdCfg<128, 128, 2, 2>;      // 4 waves of 64 x 64
using BwdLarge = BwdCfg<256, 256, 2, 4, MOE_BWD_LARGE_BK, MOE_BWD_LARGE_STAGES>;  // 8 waves

enum { OPK = 0, OPT = 1 };        // operand rows hold K (contiguous) / hold M or N

struct Operand {
    const uint16_t* p;
    size_t ld;                    // elements between rows of the stored matrix
    size_t gstride;               // elements between groups (weights); 0 = rows are global
    int kb_rows;                  // 0: row-major; R: each group's [R, ld] matrix K-blocked
                                  // ([ld / 32][R][32 elements], the forward's weight layout)
    const int32_t* rows;          // ragged-M A only: row i of the operand is row rows[i] of p
                                  // (a gather), or nullptr
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
    // ragged-K: the groups dealt over the XCDs (xorder[x * groups / 8 + j] = the j-th group
    // XCD x walks), or nullptr for contiguous runs of tiles
    const int32_t* xorder;
};

// swizzle of the 16-byte chunks of a [k][cols] operand row (a row is a whole number of
// 256-byte bank lines, so a chunk's banks depend on its index mod 16 alone). A transposing
// read is served 32 lanes at a time: 64 bytes (4 chunks) of each of four consecutive k rows.
// XOR-ing the chunk index with 4 (k & 3) puts those four rows on four different 64-byte
// bank groups (with 2 (k & 3), rows k and k ^ 1 shared one and the reads were 2-way
// conflicted).
MOE_DEVICE int swz_t(int k) { return 4 * (k & 3); }

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
template <class CF, int AO, int BO, int RAGGED_K, int EPI>
MOE_DEVICE void bwd_tile(const BwdArgs& ba, int L, uint8_t* lds) {
    constexpr int kBM = CF::BM, kBN = CF::BN, kTM = CF::kTM, kTN = CF::kTN;
    constexpr int kWaves = CF::kWaves, kOpBytes = CF::kABytes;
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
    const int wm = wave / CF::WN, wn = wave % CF::WN;
    // ---- tile
    int g, m0, Mg, rbase, mt, nt;
    {
        if (RAGGED_K) {
            g = L / (ba.ntm * ba.ntn);
            const int rem = L % (ba.ntm * ba.ntn);
            mt = rem / ba.ntn;
            nt = rem % ba.ntn;
            rbase = ba.offsets[g];
            Mg = ba.offsets[g + 1] - rbase;
            m0 = mt * kBM;
        } else {
            // a group's M tiles go in bands of kBand, M fastest within a band, so the tiles
            // that read one weight tile run side by side on one XCD and the later ones find
            // it in L2 (N fastest: every M tile of an expert streamed its weights again)
            constexpr int kBand = 4;
            const int ntn = ba.ntn;
            const int4 t0 = ba.tiles[L / ntn];                       // some tile of L's group
            const int mt0 = L / ntn - t0.y / tile_span(t0.z, kBM);   // the group's first tile
            const int me = (t0.z + kBM - 1) / kBM;                   // the group's M tiles
            const int local = L - mt0 * ntn;
            const int band = local / (kBand * ntn) * kBand;
            const int mb = me - band < kBand ? me - band : kBand;
            const int r = local - band * ntn;
            const int4 ti = ba.tiles[mt0 + band + r % mb];
            nt = r / mb;
            g = ti.x & 0xFFFFF;
            m0 = ti.y;
            Mg = tile_end(ti.y, ti.z, kBM);   // the tile's end row within the group
            rbase = ti.w;
            mt = 0;
        }
    }
    constexpr int kBK = CF::kBK, kStages = CF::kStages, kCpr = CF::kCpr;
    const int nk = RAGGED_K ? (Mg + kBK - 1) / kBK : ba.K / kBK;
    const int live = RAGGED_K ? kBM : (Mg - m0 < kBM ? Mg - m0 : kBM);

    // ---- DMA sources. An operand tile is made of 1 KB instructions; wave w issues
    // q = w + kWaves u.
    // OPK tile [rows][BK k] (BK / 8 16-byte chunks per row): instruction q fills rows
    // (512 / BK) q + lane / (BK / 8).
    // OPT tile [BK k][C cols] (C = BM for A, BN for B; C / 8 16-byte chunks per k row):
    // instruction q fills k rows (512 / C) q + lane / (C / 8).
    const uint8_t* srcA[CF::kDmaA];
    const uint8_t* srcB[CF::kDmaB];
    int ka[CF::kDmaA], kb[CF::kDmaB];   // OPT: the k row each instruction fills (ragged K)
    auto op_src = [&](const Operand& op, int o, bool is_a, int q, const uint8_t*& src, int& krow) {
        if (o == OPK) {
            const int r = (64 / kCpr) * q + lane / kCpr;
            const int c = (lane % kCpr) ^ chunk_swz<kCpr>(r);
            size_t row;
            if (is_a) {                       // ragged-M activations: global rows, clamped
                const int rr = m0 + r < Mg ? m0 + r : Mg - 1;
                row = op.rows ? (size_t)op.rows[rbase + rr] : (size_t)rbase + rr;
            } else {
                row = (size_t)nt * kBN + r;
            }
            src = (const uint8_t*)(op.p + (size_t)g * op.gstride + row * op.ld) + c * 16;
            krow = 0;
        } else {
            const int cpr = (is_a ? kBM : kBN) / 8;
            const int kr = (64 / cpr) * q + lane / cpr;
            const int c = (lane % cpr) ^ swz_t(kr);
            const size_t col = (size_t)(is_a ? mt * kBM : nt * kBN) + c * 8;
            // byte offset of (row 0, col): K-blocked, the 8-element chunk at col sits in 64-byte
            // slice col / 32 of every row, and the rows of a slice are 64 bytes apart
            const size_t cb = op.kb_rows ? ((col / 32) * op.kb_rows * 32 + col % 32) * 2 : col * 2;
            if (RAGGED_K)
                src = (const uint8_t*)(op.p + (size_t)rbase * op.ld) + cb;     // + k * kstride
            else
                src = (const uint8_t*)(op.p + (size_t)g * op.gstride) + cb;    // + k * kstride
            krow = kr;
        }
    };
#pragma unroll
    for (int u = 0; u < CF::kDmaA; ++u) op_src(ba.a, AO, true, wave + kWaves * u, srcA[u], ka[u]);
#pragma unroll
    for (int u = 0; u < CF::kDmaB; ++u) op_src(ba.b, BO, false, wave + kWaves * u, srcB[u], kb[u]);
    auto issue = [&](int kstep, int stage) {
        MOE_LDS uint8_t* base = (MOE_LDS uint8_t*)lds + stage * CF::kStageBytes;
#pragma unroll
        for (int u = 0; u < CF::kDmaA; ++u) {
            const int q = wave + kWaves * u;
            const uint8_t* sa;
            if (AO == OPK) {
                sa = srcA[u] + (size_t)kstep * kBK * 2;
            } else {
                const int kk = kstep * kBK + ka[u];
                const size_t ks = ba.a.kb_rows ? 64 : ba.a.ld * 2;     // bytes between k rows
                sa = (RAGGED_K && kk >= Mg) ? ba.zero + (lane % (kBM / 8)) * 16
                                            : srcA[u] + (size_t)kk * ks;
            }
            __builtin_amdgcn_global_load_lds((const void*)sa, (MOE_LDS void*)(base + q * 1024),
                                             16, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < CF::kDmaB; ++u) {
            const int q = wave + kWaves * u;
            const uint8_t* sb;
            if (BO == OPK) {
                sb = srcB[u] + (size_t)kstep * kBK * 2;
            } else {
                const int kk = kstep * kBK + kb[u];
                const size_t ks = ba.b.kb_rows ? 64 : ba.b.ld * 2;     // bytes between k rows
                sb = (RAGGED_K && kk >= Mg) ? ba.zero + (lane % (kBN / 8)) * 16
                                            : srcB[u] + (size_t)kk * ks;
            }
            __builtin_amdgcn_global_load_lds((const void*)sb,
                                             (MOE_LDS void*)(base + kOpBytes + q * 1024), 16, 0, 0);
        }
    };

    // ---- fragment addresses (bytes within an operand tile)
    // OPK: row (sub-tile base + lane % 32), chunk (2 s + lane / 32) ^ swz
    // OPT: k rows 16 s + 8 (h / 2) + u / 4 (+ 4), column base + 16 (h % 2) + 4 (u % 4)
    const int h16 = lane / 16, u16 = lane % 16;
    int offK[CF::kSub];
#pragma unroll
    for (int s = 0; s < CF::kSub; ++s)
        offK[s] = ((2 * s + lane / 32) ^ chunk_swz<kCpr>(lane % 32)) * 16;
    auto frag = [&](const uint8_t* tile, int o, int cols, int sub_base, int s) -> bf16x8_t {
        if (o == OPK) {
            return *(const bf16x8_t*)(tile + (sub_base + lane % 32) * (kBK * 2) + offK[s]);
        } else {
            const int k0 = 16 * s + 8 * (h16 / 2) + u16 / 4;
            const int col = sub_base + 16 * (h16 % 2) + 4 * (u16 % 4);
            const int chunk = (col / 8) ^ swz_t(k0);          // k0 and k0 + 4 share swz_t
            const int off = chunk * 16 + (col % 8) * 2;
            return tr_frag(tile + k0 * cols * 2 + off, tile + (k0 + 4) * cols * 2 + off);
        }
    };

    f32x16_t acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[i][j] = f32x16_t{};
    int nvi = (live - wm * (kBM / CF::WM) + 31) / 32;
    nvi = nvi < 0 ? 0 : (nvi > kTM ? kTM : nvi);
    nvi = __builtin_amdgcn_readfirstlane(nvi);

#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
        if (s < nk) issue(s, s);
    int stage = 0;
    for (int kt = 0; kt < nk; ++kt) {
        // stage kt has landed once at most min(kStages - 2, later) younger stages remain
        const int later = nk - 1 - kt;
        constexpr int kStep = CF::kDmaA + CF::kDmaB;
        if (later >= kStages - 2) wait_vm_lgkm0<(kStages - 2) * kStep>();
        else if (later >= 1) wait_vm_lgkm0<cmin(1, kStages - 2) * kStep>();
        else wait_vm_lgkm0<0>();
        block_sync();
        {
            const int kn = kt + kStages - 1;
            int sn = stage + kStages - 1;
            if (sn >= kStages) sn -= kStages;
            if (kn < nk) issue(kn, sn);
        }
        const uint8_t* ta = lds + stage * CF::kStageBytes;
        const uint8_t* tb = ta + kOpBytes;
        if (nvi > 0) {
#pragma unroll
            for (int s = 0; s < CF::kSub; ++s) {
                bf16x8_t av[kTM], bv[kTN];
#pragma unroll
                for (int j = 0; j < kTN; ++j)
                    bv[j] = frag(tb, BO, kBN, wn * (kBN / CF::WN) + j * 32, s);
#pragma unroll
                for (int i = 0; i < kTM; ++i)
                    av[i] = frag(ta, AO, kBM, wm * (kBM / CF::WM) + i * 32, s);
#pragma unroll
                for (int i = 0; i < kTM; ++i)
#pragma unroll
                    for (int j = 0; j < kTN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[j], av[i],
                                                                            acc[i][j], 0, 0, 0);
            }
        }
        if (++stage == kStages) stage = 0;
    }

    // ---- epilogue. The B operand goes first into the MFMA, so element r of lane l of
    // sub-tile (i, j) is output row wm * BM / WM + 32 i + l % 32 and column
    // wn * BN / WN + 32 j + 8 (r / 4) + 4 (l / 32) + r % 4: every lane holds runs of four
    // consecutive columns of one row.
    if (EPI == 0) {
        // stage the bf16 tile in LDS ([BM][BN + 8]) with one 8-byte write per run, then write
        // 16-byte row chunks
        constexpr int kEpStride = kBN + 8;
        block_sync();                               // every wave is done with the stages
        uint16_t* ep = (uint16_t*)lds;
#pragma unroll
        for (int i = 0; i < kTM; ++i) {
            if (i >= nvi) continue;
            const int row = wm * (kBM / CF::WM) + i * 32 + lane % 32;
#pragma unroll
            for (int j = 0; j < kTN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int lcol = wn * (kBN / CF::WN) + j * 32 + 8 * q + 4 * (lane / 32);
                    *(uint2*)(ep + row * kEpStride + lcol) =
                        make_uint2(pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                                   pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
                }
        }
        __syncthreads();
        uint16_t* out = ba.out + (RAGGED_K ? (size_t)g * ba.out_gstride : 0);
        constexpr int kChunks = kBN / 8;
        const int rows = RAGGED_K ? kBM : live;
        for (int c = threadIdx.x; c < rows * kChunks; c += CF::kThreads) {
            const int row = c / kChunks, cc = c % kChunks;
            const uint4 v = *(const uint4*)(ep + row * kEpStride + cc * 8);
            const size_t orow = RAGGED_K ? (size_t)mt * kBM + row : (size_t)rbase + m0 + row;
            uint16_t* dst = out + orow * ba.out_ld + (size_t)nt * kBN + cc * 8;
            // weight gradients (read by no later kernel here) bypass the caches on the way out
            if (RAGGED_K)
                __builtin_nontemporal_store(i32x4_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w},
                                            (i32x4_t*)dst);
            else
                *(uint4*)dst = v;
        }
        return;
    }
    // SwiGLU backward on the dA tile (columns f of this N tile), four columns of one row per
    // run: Z_g, Z_u read and dZ_g, dZ_u written 8 bytes at a time; dg partial per row
    const int F = ba.F;
    float dgp[kTM];
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
        dgp[i] = 0.0f;
        const int row = wm * (kBM / CF::WM) + i * 32 + lane % 32;
        if (i >= nvi || m0 + row >= Mg) continue;
        const size_t grow = (size_t)rbase + m0 + row;
        const float gt = ba.gate ? ba.gate[grow] : 1.0f;
        const uint16_t* zr = ba.z + grow * 2 * F;
        uint16_t* dzr = ba.dz + grow * 2 * F;
#pragma unroll
        for (int j = 0; j < kTN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int f = nt * kBN + wn * (kBN / CF::WN) + j * 32 + 8 * q + 4 * (lane / 32);
                const uint2 zgv = *(const uint2*)(zr + f);
                const uint2 zuv = *(const uint2*)(zr + F + f);
                const uint32_t zgw[2] = {zgv.x, zgv.y}, zuw[2] = {zuv.x, zuv.y};
                float dzg[4], dzu[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float zg = bf16_to_f32((uint16_t)(zgw[e / 2] >> (16 * (e % 2))));
                    const float zu = bf16_to_f32((uint16_t)(zuw[e / 2] >> (16 * (e % 2))));
                    const float sg = 1.0f / (1.0f + expf(-zg));
                    const float si = zg * sg;
                    const float ds = sg * (1.0f + zg * (1.0f - sg));
                    const float da = acc[i][j][4 * q + e];
                    const float dh = gt * da;
                    dzg[e] = dh * zu * ds;
                    dzu[e] = dh * si;
                    dgp[i] += da * (si * zu);
                }
                *(uint2*)(dzr + f) = make_uint2(pack_bf16x2(dzg[0], dzg[1]), pack_bf16x2(dzg[2], dzg[3]));
                *(uint2*)(dzr + F + f) = make_uint2(pack_bf16x2(dzu[0], dzu[1]), pack_bf16x2(dzu[2], dzu[3]));
            }
    }
    // rows' partial sums: the lane's own 4 kTN columns, its partner lane l ^ 32 (the row's other
    // columns of the wave), then the WN waves of a row band (LDS), in a fixed order
    block_sync();
    float* red = (float*)lds;                          // [WN][kBM]
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
        const float v = dgp[i] + __shfl_xor(dgp[i], 32);
        const int row = wm * (kBM / CF::WM) + i * 32 + lane % 32;
        if (lane < 32) red[wn * kBM + row] = v;
    }
    __syncthreads();
    if (threadIdx.x < kBM) {
        const int row = threadIdx.x;
        if (m0 + row < Mg) {
            const size_t grow = (size_t)rbase + m0 + row;
            float v = red[row];
#pragma unroll
            for (int w = 1; w < CF::WN; ++w) v += red[w * kBM + row];
            ba.dg_part[grow * ba.ntn + nt] = v;
        }
    }
}

// One tile per workgroup. The hardware deals workgroups round-robin over the 8 XCDs, so
// workgroup b (on XCD b % 8) takes tile (b % 8) * per + b / 8: each XCD walks one contiguous
// run of tiles. With a group plan (ragged K), XCD x walks the tiles of its own list of
// groups instead, group after group (every group has ntm * ntn tiles).
template <class CF, int AO, int BO, int RAGGED_K, int EPI>
__global__ __launch_bounds__(CF::kThreads) void bwd_gemm_kernel(BwdArgs ba) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int xcd = blockIdx.x % 8, i = blockIdx.x / 8;
    if (RAGGED_K && ba.xorder) {
        const int tg = ba.ntm * ba.ntn, cap = ba.groups / 8;
        const int j = i / tg;
        if (j >= cap) return;
        int g = ba.xorder[xcd * cap + j];
        g = g < 0 ? 0 : (g >= ba.groups ? ba.groups - 1 : g);
        bwd_tile<CF, AO, BO, RAGGED_K, EPI>(ba, g * tg + i % tg, lds);
        return;
    }
    const int total = RAGGED_K ? ba.groups * ba.ntm * ba.ntn : *ba.total * ba.ntn;
    const int per = (total + 7) / 8;
    const int L = xcd * per + i;
    if (i >= per || L >= total) return;
    bwd_tile<CF, AO, BO, RAGGED_K, EPI>(ba, L, lds);
}

// The weight-gradient GEMMs' group plan. A group's tiles take time in proportion to its rows
// (their K) plus a fixed part (prologue and the output tile's stores, about kPlanTileRows
// rows' worth), and the tiles of one group stay on one XCD, which reads the group's rows
// once into its L2. Dealt in contiguous runs, a skewed load leaves one XCD with a third more
// work than the mean. Here each XCD gets groups / 8 groups, chosen largest first, each to
// the XCD with the least work so far among those with room (longest processing time first
// under a cardinality cap), so each XCD's list also runs from its largest group down.
// One workgroup: the groups are ranked by counting (ties by index), then one wave places
// them, lanes 0..7 holding the XCDs' loads.
constexpr int kPlanMaxGroups = 2048;
constexpr int kPlanTileRows = 192;

// minimum over each run of 8 lanes, in all 8: lanes ^ 1 and ^ 2 within a quad, then the
// mirror lane within the 8 (lane i and 7 - i hold the two quads' minima)
MOE_DEVICE unsigned min_of_8_lanes(unsigned v) {
    v = min(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
    v = min(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
    v = min(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false)); // half mirror
    return v;
}

__global__ __launch_bounds__(256) void wgrad_plan_kernel(const int32_t* __restrict__ offsets,
                                                         int E, int32_t* __restrict__ xorder) {
    __shared__ int cost[kPlanMaxGroups];
    __shared__ int ranked[kPlanMaxGroups];     // groups by cost, largest first
    __shared__ int rcost[kPlanMaxGroups];      // and their costs
    const int tid = threadIdx.x, lane = tid % 64;
    for (int e = tid; e < E; e += 256) {
        cost[e] = offsets[e + 1] - offsets[e] + kPlanTileRows;
        xorder[e] = e;          // every slot holds a valid group before the placement below
    }
    __syncthreads();
    for (int e = tid; e < E; e += 256) {
        const int ce = cost[e];
        int r = 0;
        for (int j = 0; j < E; ++j) {
            const int cj = cost[j];
            r += (cj > ce || (cj == ce && j < e)) ? 1 : 0;
        }
        ranked[r] = e;
        rcost[r] = ce;
    }
    __syncthreads();
    if (tid >= 64) return;
    // 32-bit keys (load >> sh) * 8 + lane: sh drops the low bits of loads past 2^27
    const long long total = (long long)(offsets[E] - offsets[0]) + (long long)E * kPlanTileRows;
    int sh = 0;
    while ((total >> sh) >= (1ll << 27)) ++sh;
    const int cap = E / 8;
    long long load = 0;          // lanes 0..7: XCD lane's work so far
    int n = 0;                   // and its groups so far
    int e_nx = ranked[0], c_nx = rcost[0];
    for (int r = 0; r < E; ++r) {
        const int e = e_nx, c = c_nx;
        if (r + 1 < E) {
            e_nx = ranked[r + 1];
            c_nx = rcost[r + 1];
        }
        // the least-loaded XCD with room (some XCD has room: r < E = 8 cap groups so far)
        const unsigned key = min_of_8_lanes(
            (lane < 8 && n < cap) ? ((unsigned)(load >> sh) << 3) | (unsigned)lane
                                  : 0xFFFFFFFFu);
        if (lane == (int)(key & 7) && n < cap) {
            xorder[lane * cap + n] = e;
            load += c;
            ++n;
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

// offsets {0, T} of a single group, and a zeroed page
__global__ __launch_bounds__(256) void fill_offsets2_kernel(int32_t* offs, int T, uint32_t* z,
                                                            int nz) {
    const int i = threadIdx.x;
    if (i < 2) offs[i] = i == 0 ? 0 : T;
    for (int j = i; j < nz; j += 256) z[j] = 0u;
}

__global__ __launch_bounds__(256) void zero_fill_kernel(uint32_t* p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

template <class CF, int AO, int BO, int RAGGED_K, int EPI>
hipError_t run_bwd(const BwdArgs& ba, int nblocks, hipStream_t s) {
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(
            (const void*)bwd_gemm_kernel<CF, AO, BO, RAGGED_K, EPI>,
            hipFuncAttributeMaxDynamicSharedMemorySize, CF::kLds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    if (nblocks > 0)
        bwd_gemm_kernel<CF, AO, BO, RAGGED_K, EPI><<<nblocks, CF::kThreads, CF::kLds, s>>>(ba);
    return hipGetLastError();
}

struct BwdWs {
    void* sched;
    int32_t* xorder;              // weight-gradient group plan (E entries)
    uint8_t* zero;
    uint16_t* dz;
    float* dg_part;
    size_t total;
};

size_t al(size_t v) { return (v + 255) / 256 * 256; }

// sized for the smaller tiles (more M tiles, more dg partials per row)
BwdWs carve_bwd(void* ws, int A, int E, int F) {
    BwdWs w;
    char* p = (char*)ws;
    size_t off = 0;
    w.sched = p ? p + off : nullptr;
    off += al(schedule_ws_bytes(A, E, BwdSmall::BM));
    w.xorder = p ? (int32_t*)(p + off) : nullptr;
    off += al((size_t)E * 4);
    w.zero = p ? (uint8_t*)(p + off) : nullptr;
    off += al(kZeroBytes);
    w.dz = p ? (uint16_t*)(p + off) : nullptr;
    off += al((size_t)A * 2 * F * 2);
    w.dg_part = p ? (float*)(p + off) : nullptr;
    off += al((size_t)A * (F / BwdSmall::BN) * 4);
    w.total = off;
    return w;
}

// The weight gradients run beside the data gradients (the W/D split: dW needs only the
// activations and dZ, so it need not wait for dx): dW2 on one side stream from the start,
// dW13 on another once dZ exists, both joined back to the caller's stream by events. The
// data-gradient kernels stream weights from HBM, the weight-gradient kernels mostly write
// dW, so they overlap (dW13 on the first side stream too would wait for dW2, which the
// data gradients slow down). Two side streams and five events per device, created on first
// use (default priority); the mutex keeps two host threads from interleaving their records
// of the shared events. A caller that queues several backward launches may defer the join
// (join = false) and join once at its end, holding the lock across them (bwd_side_lock), so
// that its next kernels need not wait for the weight gradients.
constexpr int kMaxDevices = 64;
struct SideRes {
    hipStream_t side = nullptr, side2 = nullptr;
    hipEvent_t ev[5] = {};
};
std::recursive_mutex g_side_mu;
SideRes g_side[kMaxDevices];

hipError_t side_res(SideRes** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    SideRes& r = g_side[dev];
    if (!r.side) {
        e = hipStreamCreateWithFlags(&r.side, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipStreamCreateWithFlags(&r.side2, hipStreamNonBlocking);
        for (int i = 0; i < 5 && e == hipSuccess; ++i)
            e = hipEventCreateWithFlags(&r.ev[i], hipEventDisableTiming);
        if (e != hipSuccess) return e;
    }
    *out = &r;
    return hipSuccess;
}

template <class CF>
hipError_t bwd_all(const BwdWs& w, const void* dy_perm, const void* x_perm, const void* z,
                   const void* act, const float* gate_perm, const int32_t* offsets,
                   const void* w13, const void* w2, int A, int E, int H, int F, void* dx_perm,
                   void* dw13, void* dw2, float* dgate_perm, hipStream_t s, bool join,
                   bool w_kblock, bool use_side, const BwdGather* gx) {
    constexpr int kBM = CF::BM, kBN = CF::BN;
    std::lock_guard<std::recursive_mutex> lock(g_side_mu);
    SideRes* sr = nullptr;
    hipError_t e = side_res(&sr);
    if (e != hipSuccess) return e;
    e = launch_schedule(offsets, E, kBM, w.sched, s);
    if (e != hipSuccess) return e;
    const int4* tiles = (const int4*)((char*)w.sched + 256);
    const int* total = (const int*)w.sched;
    const size_t max_tiles = (size_t)(A + kBM - 1) / kBM + (size_t)E;
    const uint16_t* DY = (const uint16_t*)dy_perm;
    const uint16_t* X = (const uint16_t*)x_perm;
    const uint16_t* W13 = (const uint16_t*)w13;
    const uint16_t* W2 = (const uint16_t*)w2;
    auto round8 = [](size_t n) { return (int)((n + 7) / 8 * 8); };
    // fork: the side stream starts after everything the caller queued (inputs, zero page)
    // (use_side = false: every launch on the caller's stream, in the same order)
    hipStream_t s_w2 = use_side ? sr->side : s, s_w13 = use_side ? sr->side2 : s;
    if (use_side) {
        e = hipEventRecord(sr->ev[0], s);
        if (e == hipSuccess) e = hipStreamWaitEvent(sr->side, sr->ev[0], 0);
        if (e != hipSuccess) return e;
    }
    // the expert-order copies the caller left to this call: x_perm on dW13's stream beside
    // dA (dW13 is its only reader), dy_perm on dW2's stream (dA reads dY's rows through src)
    if (gx && gx->x) {
        if (use_side) e = hipStreamWaitEvent(sr->side2, sr->ev[0], 0);
        if (e == hipSuccess) e = launch_gather_rows(gx->x, gx->pos, gx->T, gx->k, H * 2,
                                                    (void*)x_perm, s_w13);
        if (e != hipSuccess) return e;
    }
    if (gx && gx->dy) {
        e = launch_gather_rows(gx->dy, gx->pos, gx->T, gx->k, H * 2, (void*)dy_perm, s_w2);
        if (e != hipSuccess) return e;
    }
    // the weight gradients' XCD plan, for group counts it splits evenly: first on the stream
    // of dW2, which needs it, and off the caller's (dW13's stream waits for it below)
    const int32_t* xorder = nullptr;
    const bool plan = E % 8 == 0 && E >= 64 && E <= kPlanMaxGroups && MOE_BWD_PLAN;
    if (plan) {
        wgrad_plan_kernel<<<1, 256, 0, s_w2>>>(offsets, E, w.xorder);
        e = hipGetLastError();
        if (e == hipSuccess && use_side) e = hipEventRecord(sr->ev[4], s_w2);
        if (e != hipSuccess) return e;
        xorder = w.xorder;
    }

    // wgrad 2 (side): dW2_e [H, F] = dy_perm[R_e]^T act[R_e]
    BwdArgs w2a = {};
    w2a.a = {DY, (size_t)H, 0, 0};
    w2a.b = {(const uint16_t*)act, (size_t)F, 0, 0};
    w2a.offsets = offsets; w2a.M = H; w2a.N = F; w2a.ntm = H / CF::BM; w2a.ntn = F / CF::BN;
    w2a.groups = E; w2a.out = (uint16_t*)dw2; w2a.out_ld = F; w2a.out_gstride = (size_t)H * F;
    w2a.zero = w.zero; w2a.xorder = xorder;
    e = run_bwd<CF, OPT, OPT, 1, 0>(w2a, round8((size_t)E * w2a.ntm * w2a.ntn), s_w2);
    // dgrad 1: dA [A, F] = dy_perm W2_e (W2_e stored [H][F]: K rows) -> dZ, dg partials
    if (e == hipSuccess) {
        BwdArgs d1 = {};
        d1.a = {DY, (size_t)H, 0, 0, nullptr};
        if (gx && gx->dy) d1.a = {(const uint16_t*)gx->dy, (size_t)H, 0, 0, gx->src};
        d1.b = {W2, (size_t)F, (size_t)H * F, w_kblock ? H : 0};
        d1.offsets = offsets; d1.tiles = tiles; d1.total = total;
        d1.N = F; d1.K = H; d1.ntn = F / kBN; d1.groups = E;
        d1.z = (const uint16_t*)z; d1.gate = gate_perm; d1.dz = w.dz; d1.dg_part = w.dg_part;
        d1.F = F; d1.zero = w.zero;
        e = run_bwd<CF, OPK, OPT, 0, 1>(d1, round8(max_tiles * d1.ntn), s);
    }
    if (e == hipSuccess && dgate_perm) {
        dg_reduce_kernel<<<(A + 255) / 256, 256, 0, s>>>(w.dg_part, A, F / kBN, dgate_perm);
        e = hipGetLastError();
    }
    // dZ is ready: wgrad 1 (second side stream) and dgrad 2 (caller's stream)
    if (e == hipSuccess && use_side) e = hipEventRecord(sr->ev[1], s);
    if (e == hipSuccess && use_side) e = hipStreamWaitEvent(sr->side2, sr->ev[1], 0);
    if (e == hipSuccess && use_side && plan) e = hipStreamWaitEvent(sr->side2, sr->ev[4], 0);
    if (e == hipSuccess) {
        // wgrad 1: dW13_e [2F, H] = dZ[R_e]^T x_perm[R_e]
        BwdArgs w1 = {};
        w1.a = {w.dz, (size_t)2 * F, 0, 0};
        w1.b = {X, (size_t)H, 0, 0};
        w1.offsets = offsets; w1.M = 2 * F; w1.N = H; w1.ntm = 2 * F / CF::BM;
        w1.ntn = H / CF::BN; w1.groups = E; w1.out = (uint16_t*)dw13; w1.out_ld = H;
        w1.out_gstride = (size_t)2 * F * H; w1.zero = w.zero; w1.xorder = xorder;
        e = run_bwd<CF, OPT, OPT, 1, 0>(w1, round8((size_t)E * w1.ntm * w1.ntn), s_w13);
    }
    if (e == hipSuccess) {
        // dgrad 2: dx_perm [A, H] = dZ W13_e (W13_e stored [2F][H]: K rows)
        BwdArgs d2 = {};
        d2.a = {w.dz, (size_t)2 * F, 0, 0};
        d2.b = {W13, (size_t)H, (size_t)2 * F * H, w_kblock ? 2 * F : 0};
        d2.offsets = offsets; d2.tiles = tiles; d2.total = total;
        d2.N = H; d2.K = 2 * F; d2.ntn = H / kBN; d2.groups = E;
        d2.out = (uint16_t*)dx_perm; d2.out_ld = H; d2.zero = w.zero;
        e = run_bwd<CF, OPK, OPT, 0, 0>(d2, round8(max_tiles * d2.ntn), s);
    }
    // join (deferred when asked, unless a launch failed), so that nothing queued on the side
    // streams outlives the caller's view of this call
    if (!use_side || (!join && e == hipSuccess)) return e;
    hipError_t j = hipEventRecord(sr->ev[2], sr->side);
    if (j == hipSuccess) j = hipStreamWaitEvent(s, sr->ev[2], 0);
    if (j == hipSuccess) j = hipEventRecord(sr->ev[3], sr->side2);
    if (j == hipSuccess) j = hipStreamWaitEvent(s, sr->ev[3], 0);
    return e != hipSuccess ? e : j;
}

// Router weight and data gradients as one-group GEMMs of the same kernel:
//   dW_r [E, H] = dl^T x      (K = the T token rows, both operands read as [k][m])
//   dx_r [T, H] = dl W_r      (ragged-M mode with a single group of T rows, K = E)
template <class CF>
hipError_t router_bwd_all(const void* dl, const void* x, const void* w_router, int T, int E,
                          int H, const int32_t* offs2, void* sched, const uint8_t* zero,
                          void* dw_router, void* dx_router, hipStream_t s) {
    const uint16_t* DL = (const uint16_t*)dl;
    auto round8 = [](size_t n) { return (int)((n + 7) / 8 * 8); };
    BwdArgs wa = {};
    wa.a = {DL, (size_t)E, 0, 0};
    wa.b = {(const uint16_t*)x, (size_t)H, 0, 0};
    wa.offsets = offs2; wa.M = E; wa.N = H; wa.ntm = E / CF::BM; wa.ntn = H / CF::BN;
    wa.groups = 1; wa.out = (uint16_t*)dw_router; wa.out_ld = H; wa.out_gstride = 0;
    wa.zero = zero;
    hipError_t e = run_bwd<CF, OPT, OPT, 1, 0>(wa, round8((size_t)wa.ntm * wa.ntn), s);
    if (e != hipSuccess) return e;
    e = launch_schedule(offs2, 1, CF::BM, sched, s);
    if (e != hipSuccess) return e;
    BwdArgs da = {};
    da.a = {DL, (size_t)E, 0, 0};
    da.b = {(const uint16_t*)w_router, (size_t)H, 0, 0};
    da.offsets = offs2;
    da.tiles = (const int4*)((char*)sched + 256);
    da.total = (const int*)sched;
    da.N = H; da.K = E; da.ntn = H / CF::BN; da.groups = 1;
    da.out = (uint16_t*)dx_router; da.out_ld = H; da.zero = zero;
    const size_t max_tiles = (size_t)(T + CF::BM - 1) / CF::BM + 1;
    return run_bwd<CF, OPK, OPT, 0, 0>(da, round8(max_tiles * da.ntn), s);
}

}  // namespace

size_t bwd_ws_bytes(int T, int k, int E, int H, int F) {
    (void)H;
    return carve_bwd(nullptr, T * k, E, F).total;
}

void bwd_side_lock() { g_side_mu.lock(); }
void bwd_side_unlock() { g_side_mu.unlock(); }

hipError_t bwd_side_join(hipStream_t s) {
    std::lock_guard<std::recursive_mutex> lock(g_side_mu);
    SideRes* sr = nullptr;
    hipError_t e = side_res(&sr);
    if (e == hipSuccess) e = hipEventRecord(sr->ev[2], sr->side);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, sr->ev[2], 0);
    if (e == hipSuccess) e = hipEventRecord(sr->ev[3], sr->side2);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, sr->ev[3], 0);
    return e;
}

hipError_t launch_grouped_gemm_bwd(const void* dy_perm, const void* x_perm, const void* z,
                                   const void* act, const float* gate_perm,
                                   const int32_t* offsets, const void* w13, const void* w2,
                                   int A, int E, int H, int F, void* dx_perm, void* dw13,
                                   void* dw2, float* dgate_perm, void* ws, hipStream_t s,
                                   bool join, bool w_kblock, bool use_side,
                                   const BwdGather* gx) {
    BwdWs w = carve_bwd(ws, A, E, F);
    zero_fill_kernel<<<1, 256, 0, s>>>((uint32_t*)w.zero, kZeroBytes / 4);
    // 256 x 256 tiles when every GEMM dimension divides by 256 (F, 2F and H), else 128 x 128
    if (F % BwdLarge::BN == 0 && H % BwdLarge::BN == 0 && MOE_BWD_LARGE)
        return bwd_all<BwdLarge>(w, dy_perm, x_perm, z, act, gate_perm, offsets, w13, w2, A, E,
                                 H, F, dx_perm, dw13, dw2, dgate_perm, s, join, w_kblock, use_side, gx);
    return bwd_all<BwdSmall>(w, dy_perm, x_perm, z, act, gate_perm, offsets, w13, w2, A, E, H,
                             F, dx_perm, dw13, dw2, dgate_perm, s, join, w_kblock, use_side, gx);
}

size_t router_bwd_ws_bytes(int T) {
    return 256 + kZeroBytes + schedule_ws_bytes(T, 1, BwdSmall::BM);
}

// ws: {0, T} offsets (256 bytes), a zero page, the tile schedule
hipError_t launch_router_bwd(const void* dl, const void* x, const void* w_router, int T, int E,
                             int H, void* dw_router, void* dx_router, void* ws, hipStream_t s) {
    int32_t* offs2 = (int32_t*)ws;
    uint8_t* zero = (uint8_t*)ws + 256;
    void* sched = (char*)ws + 256 + kZeroBytes;
    fill_offsets2_kernel<<<1, 256, 0, s>>>(offs2, T, (uint32_t*)zero, kZeroBytes / 4);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (E % BwdLarge::BM == 0 && H % BwdLarge::BN == 0 && MOE_BWD_LARGE)
        return router_bwd_all<BwdLarge>(dl, x, w_router, T, E, H, offs2, sched, zero,
                                        dw_router, dx_router, s);
    return router_bwd_all<BwdSmall>(dl, x, w_router, T, E, H, offs2, sched, zero, dw_router,
                                    dx_router, s);
}

hipError_t launch_offsets2(int32_t* offs, int T, hipStream_t s) {
    fill_offsets2_kernel<<<1, 256, 0, s>>>(offs, T, nullptr, 0);
    return hipGetLastError();
}

}  // namespace moe

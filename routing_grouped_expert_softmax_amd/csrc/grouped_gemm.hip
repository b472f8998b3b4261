// SwiGLU experts as one grouped GEMM over ragged, expert-grouped rows.
//
// The technical summary "使用 Megatron Core 大规模训练混合专家模型（MoE）" (section 2.4) runs
// the many small expert GEMMs as one grouped GEMM; this is the gfx950 version:
//
//  * a schedule kernel turns the device-resident expert offsets into a list of M tiles
//    (segment, expert, first row, rows), so no host synchronisation is needed;
//  * one launch covers every (M tile, N tile) of every expert (and of the shared expert);
//    workgroups past the live tile count exit at once;
//  * workgroups are remapped so that each XCD (the hardware deals workgroups round-robin
//    over 8 XCDs) works through one contiguous run of tiles; within an expert the M tiles
//    that share a weight tile are neighbours and the N tiles of a band share its
//    activation rows in that XCD's L2 (pick_tile);
//  * bf16 tiles go global -> LDS by direct DMA (rings of 32-K slots, XOR-swizzled 16-byte
//    chunks) and into v_mfma_f32_32x32x16_bf16 with fp32 accumulation, the two waves of
//    every SIMD in opposite phases (one reads operands and issues DMAs while the other runs
//    its MFMAs, bf16_kloop_pp); e4m3 tiles into
//    the block-scaled v_mfma_scale_f32_32x32x64_f8f6f4, with the fp32 block scales applied
//    per 128-deep K block;
//  * GEMM1 loads the gate rows [n0, n0+BN/2) and the matching up rows [F+n0, ...) of W13
//    into one B tile, so a lane holds Z_gate and Z_up of the same (row, column) and the
//    epilogue writes act = g * silu(Z_gate) * Z_up directly: the gate is folded into the
//    activation before the down projection (memory-efficient permutation, section 2.2),
//    and Z itself is never stored unless a backward asks for it.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------------------
// tile schedule
// ---------------------------------------------------------------------------------------
struct SegDev {
    const void* a;
    const void* a_scales;      // e4m3: fp32 per 1 x 128; MXFP8: E8M0 bytes per 1 x 32
    const float* gate;
    const void* w;
    const void* w_scales;      // e4m3: fp32 per 128 x 128; MXFP8: E8M0 bytes per 1 x 32
    void* out;
    void* out_scales;          // GEMM1 act scales, as a_scales
    void* z_out;
    // operand addressing in bytes: row r, 64-byte K slice j of `a` is at
    // a + r * a_row + j * a_kstep (row-major: a_row = K * eb, a_kstep = 64; K-blocked:
    // a_row = 64, a_kstep = rows_total * 64); the same for each group's weight, whose
    // group g starts at w + g * w_mat
    size_t a_row, a_kstep, w_row, w_kstep, w_mat;
    int rows_total;
    int out_kblock;
    const int32_t* a_rows;   // nullptr, or the source row of each launch row (a gather)
    // MXFP8 scale addressing in bytes: the word (four block codes of 128 K) of row r, K block
    // kb is at a_scales + r * sa_row + kb * sa_kb (row-major: K/32, 4; blocked: 4, rows * 4);
    // the same for each group's w_scales (group stride N * K/32) and for GEMM1's out_scales
    uint32_t sa_row, sa_kb, sw_row, sw_kb, so_row, so_kb;
    int a_sc_direct;         // scales of launch row r at row r even when a_rows gathers codes
};

struct SchedArgs {
    const int32_t* offsets[2];
    int groups[2];
    int rows[2];
    int nseg;
};

// tiles[i] = {seg << 20 | group, first row within the group, rows of the group,
//             global row of the group's first row}; *total = number of M tiles. A group's
// rows are dealt evenly over its tiles (tile_span), so a tile spans [m0, tile_end(m0, ..)).
// One block of 1024 threads; each thread owns two consecutive group slots.
__global__ __launch_bounds__(1024) void schedule_kernel(SchedArgs sa, int bm,
                                                        int4* __restrict__ tiles,
                                                        int* __restrict__ total) {
    __shared__ int wsum[16];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    int nslot = 0;
    for (int s = 0; s < sa.nseg; ++s) nslot += sa.groups[s];
    int seg_of[2], grp_of[2], m_of[2], base_of[2], nt_of[2];
    int mine = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        int slot = 2 * tid + q;
        seg_of[q] = -1;
        nt_of[q] = 0;
        if (slot < nslot) {
            int s = 0, g = slot;
            if (g >= sa.groups[0]) { s = 1; g -= sa.groups[0]; }
            int base, m;
            if (sa.offsets[s]) {
                base = sa.offsets[s][g];
                m = sa.offsets[s][g + 1] - base;
            } else {
                base = 0;
                m = sa.rows[s];
            }
            seg_of[q] = s; grp_of[q] = g; m_of[q] = m; base_of[q] = base;
            nt_of[q] = (m + bm - 1) / bm;
        }
        mine += nt_of[q];
    }
    int v = mine;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int o = __shfl_up(v, off);
        if (lane >= off) v += o;
    }
    if (lane == kWave - 1) wsum[wave] = v;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    int start = before + v - mine;
    if (tid == blockDim.x - 1) *total = before + v;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        for (int i = 0; i < nt_of[q]; ++i)
            tiles[start + i] = make_int4((seg_of[q] << 20) | grp_of[q],
                                         i * tile_span(m_of[q], bm), m_of[q], base_of[q]);
        start += nt_of[q];
    }
}

// Mixed tile shapes for the bf16 kernel. A group of n rows takes n / 256 full 256-row M tiles
// (256 x 256 output tiles) and, for a remainder r = n % 256: one more 256-row tile if r > 128,
// else one 128-row tile on the 128 x (256 w1) shape (w1 = 1 or 2). The unit table lists every
// output tile in launch order: per group, bands of up to `mgroup` 256-row M tiles; within a
// band, for each column block c of 256 w1 columns, the band's tiles at the N tiles
// w1 c .. w1 c + w1 - 1, then the group's 128-row tile at block c (with the group's last
// band), so the tiles that read the same weight rows get neighbouring ids.
// ntn0 = N / 256 (a multiple of w1). Every block of the grid computes the per-group prefix and
// writes its share of the units.
__global__ __launch_bounds__(1024) void schedule_mixed_kernel(SchedArgs sa, int ntn0, int w1,
                                                              int mgroup,
                                                              int4* __restrict__ units,
                                                              int* __restrict__ unit_nt,
                                                              int* __restrict__ total) {
    constexpr int kSlots = 2048;                       // two group slots per thread
    __shared__ int wsum[16];
    __shared__ int s_start[kSlots + 1], s_n[kSlots], s_base[kSlots], s_x[kSlots];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int ntn1 = ntn0 / w1;                        // 128-row tiles' N tiles
    int nslot = 0;
    for (int s = 0; s < sa.nseg; ++s) nslot += sa.groups[s];
    int cnt_of[2];
    int mine = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int slot = 2 * tid + q;
        cnt_of[q] = 0;
        if (slot < nslot) {
            int s = 0, g = slot;
            if (g >= sa.groups[0]) { s = 1; g -= sa.groups[0]; }
            int base, n;
            if (sa.offsets[s]) {
                base = sa.offsets[s][g];
                n = sa.offsets[s][g + 1] - base;
            } else {
                base = 0;
                n = sa.rows[s];
            }
            const int rem = n % 256;
            const int n256 = n / 256 + (rem > 128 ? 1 : 0);
            const int has128 = rem > 0 && rem <= 128 ? 1 : 0;
            cnt_of[q] = n256 * ntn0 + has128 * ntn1;
            s_n[slot] = n;
            s_base[slot] = base;
            s_x[slot] = (s << 20) | g;
        }
        mine += cnt_of[q];
    }
    int v = mine;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(v, off);
        if (lane >= off) v += o;
    }
    if (lane == kWave - 1) wsum[wave] = v;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const int p0 = before + v - mine;
    if (2 * tid < nslot) s_start[2 * tid] = p0;
    if (2 * tid + 1 < nslot) s_start[2 * tid + 1] = p0 + cnt_of[0];
    int all = 0;
    for (int w = 0; w < 16; ++w) all += wsum[w];
    if (tid == 0) {
        s_start[nslot] = all;
        if (blockIdx.x == 0) *total = all;
    }
    __syncthreads();
    // every unit in parallel over the grid's blocks (each block repeats the scan above): its
    // slot (the last slot whose start <= u), then its position in the slot's launch order
    const int uf = ntn0 * mgroup;                      // units of a full band
    for (int u = blockIdx.x * blockDim.x + tid; u < all; u += gridDim.x * blockDim.x) {
        int lo = 0, hi = nslot;                        // first slot with start > u, in (lo, hi]
        while (lo < hi) {
            const int mid = (lo + hi) / 2;
            if (s_start[mid] <= u) lo = mid + 1;
            else hi = mid;
        }
        const int slot = lo - 1;
        const int n = s_n[slot], rem = n % 256;
        const int n256 = n / 256 + (rem > 128 ? 1 : 0);
        const int has128 = rem > 0 && rem <= 128 ? 1 : 0;
        const int nbands = n256 > 0 ? (n256 + mgroup - 1) / mgroup : 1;
        int li = u - s_start[slot], b, nb, extra;
        if (li < (nbands - 1) * uf) {
            b = li / uf;
            li -= b * uf;
            nb = mgroup;
            extra = 0;
        } else {
            b = nbands - 1;
            li -= b * uf;
            nb = n256 - b * mgroup;
            extra = has128;
        }
        const int stride = w1 * nb + extra;
        const int c = li / stride, q = li % stride;
        if (q < w1 * nb) {
            const int m = b * mgroup + q % nb;
            const int m0 = m * 256, m1 = m0 + 256 < n ? m0 + 256 : n;
            units[u] = make_int4(s_x[slot], m0, m1, s_base[slot]);
            unit_nt[u] = w1 * c + q / nb;
        } else {
            units[u] = make_int4(s_x[slot] | (1 << 21), n / 256 * 256, n, s_base[slot]);
            unit_nt[u] = c;
        }
    }
}

struct GemmArgs {
    SegDev seg[2];
    const int4* tiles;
    const int* total;
    int N, K;          // GEMM N (before SwiGLU pairing) and K
    int ntn;           // N tiles
    int per_xcd_max;   // launched blocks / 8
    int bm;            // M tile rows
    int mgroup;        // M tiles of one group visited together per N tile
    // mixed bf16 schedule (schedule_mixed_kernel): one entry per output tile, in launch order
    const int4* units; // {seg << 20 | shape << 21 | group, first row, end row, global row base}
    const int* unit_nt;// the tile's N tile (of its shape's N tiling)
};

// Map this workgroup to a live tile; false when there is none.
//
// Tile order. The tiles of one group (expert) form a block [its M tiles] x [ntn N tiles]
// that occupies the same run of linear ids whatever the order inside it. Inside, M tiles go
// in bands of up to mgroup, and within a band the M index runs fastest: the M tiles that
// read the same weight tile get neighbouring ids, so they start together and the later
// readers find that weight in L2 (or the memory-side cache) instead of HBM. Each N tile
// of a band still reuses the band's activation rows from one XCD's L2.
//
// XCD-aware launch: the hardware deals workgroups round-robin over 8 XCDs, so workgroup b
// runs on XCD b % 8; it takes linear id (b % 8) * per + b / 8, which gives every XCD one
// contiguous run of ids.
MOE_DEVICE bool pick_tile(const GemmArgs& ga, int& mt, int& nt) {
    const int b = blockIdx.x;
    const int xcd = b % 8, i = b / 8;
    const int total = *ga.total * ga.ntn;
    const int per = (total + 7) / 8;
    if (i >= per) return false;
    const int L = xcd * per + i;
    if (L >= total) return false;
    const int ntn = ga.ntn, bm = ga.bm;
    const int4 t = ga.tiles[L / ntn];                 // some M tile of L's group
    const int mt0 = L / ntn - t.y / tile_span(t.z, bm);   // the group's first M tile
    const int me = (t.z + bm - 1) / bm;               // the group's M tiles
    const int local = L - mt0 * ntn;
    const int band = local / (ga.mgroup * ntn) * ga.mgroup;
    const int mb = me - band < ga.mgroup ? me - band : ga.mgroup;
    const int r = local - band * ntn;
    mt = mt0 + band + r % mb;
    nt = r / mb;
    return true;
}

// ---------------------------------------------------------------------------------------
// bf16 MFMA kernel
//
// LDS holds a ring of SA slots of BM A rows and a ring of SB slots of BN B rows, each row
// BK bf16 (64 or 128 bytes). Tiles are filled by direct global -> LDS loads
// (global_load_lds_dwordx4: no staging registers); one wave instruction fills 1 KB =
// 1024 / (2 BK) rows. Within a row the 16-byte chunks are XOR-swizzled (physical chunk =
// logical chunk ^ swz(row)) so that the 32 rows one MFMA operand read touches spread over
// the LDS banks. The prefetch distance is SA - 1 K steps for A and SB - 1 for B.
//
// Ragged tails: a wave skips the loads and MFMAs of its 32-row sub-tiles that lie wholly
// past the expert's last row, so a tile with few live rows costs few MFMA cycles.
// ---------------------------------------------------------------------------------------

#ifndef MOE_BF_INTERLEAVE
#define MOE_BF_INTERLEAVE 1
#endif
// Ping-pong K loop (bf16_kloop_pp) for 8-wave 256 x 256 tiles with K step 32 and >= 3 slots.
#ifndef MOE_BF_PINGPONG
#define MOE_BF_PINGPONG 1
#endif
// Interleaved K loop (bf16_kloop_il) for configurations the ping-pong loop does not take
#ifndef MOE_BF_KLOOP_IL
#define MOE_BF_KLOOP_IL 1
#endif


template <int KIND, int BM, int BN, int BK, int WM, int WN, int SA, int SB>
struct BfCfg {
    static constexpr int kThreads = WM * WN * kWave;
    static constexpr int kWaves = WM * WN;
    static constexpr int kRowBytes = BK * 2;
    static constexpr int kCpr = kRowBytes / 16;             // 16-byte chunks per row
    static constexpr int kRowsPerDma = kWave / kCpr;        // rows one wave DMA fills
    static constexpr int kDmaA = BM / kRowsPerDma / kWaves; // A DMAs per wave per step
    static constexpr int kDmaB = BN / kRowsPerDma / kWaves; // B DMAs per wave per step
    static constexpr int kASlot = BM * kRowBytes;           // one A ring slot
    static constexpr int kBSlot = BN * kRowBytes;           // one B ring slot
    static constexpr int kBRing = SA * kASlot;              // B ring offset in LDS
    static constexpr int kTM = BM / WM / 32;                // 32x32 tiles per wave (M)
    static constexpr int kTN = BN / WN / 32;                // 32x32 tiles per wave (N)
    static constexpr int kSub = BK / 16;                    // MFMA K steps per stage
    static constexpr int kSlices = kRowBytes / 64;          // 64-byte K slices per stage
    static constexpr int kSA = SA, kSB = SB;
    static constexpr int kBM = BM, kBN = BN, kBK = BK, kWM = WM, kWN = WN;
    // Row order of the waves' 32-row sub-tiles: interleaved (sub-tile i of wave row wm at
    // rows (i * WM + wm) * 32), so a ragged tile's live rows spread over all the waves, or
    // blocked (wm * BM / WM + i * 32).
    static constexpr bool kInterleave = MOE_BF_INTERLEAVE != 0;
    static constexpr MOE_DEVICE int sub_row(int wm, int i) {
        return kInterleave ? (i * WM + wm) * 32 : wm * (BM / WM) + i * 32;
    }
    static constexpr int kEpCols = KIND == 0 ? BN / 2 : BN;       // output columns of a tile
    static constexpr int kEpStride = kEpCols + 8;                 // bf16, padded row
    static constexpr size_t kLdsLoop = (size_t)SA * kASlot + (size_t)SB * kBSlot;
    static constexpr size_t kLdsEp = (size_t)BM * kEpStride * 2;
    // GEMM1: the tile's row gates, staged at tile start past the ring and the epilogue
    // staging (one 4-byte word per tile row), or read from global memory by the epilogue
    // when they would not fit
    static constexpr size_t kGateOff = ((kLdsLoop > kLdsEp ? kLdsLoop : kLdsEp) + 15) / 16 * 16;
    static constexpr bool kGateLds = KIND == 0 && kGateOff + (size_t)BM * 4 <= 160 * 1024;
    static constexpr size_t kLds = kGateLds ? kGateOff + (size_t)BM * 4 : kGateOff;
    static_assert(BK == 32 || BK == 64, "BK");
    static_assert(kDmaA * kRowsPerDma * kWaves == BM && kDmaB * kRowsPerDma * kWaves == BN,
                  "DMA split");
    static_assert(KIND == 1 || kTN % 2 == 0, "GEMM1 needs gate/up tile pairs");
    static_assert(kLds <= 160 * 1024, "LDS");
    static_assert(SA >= 2 && SB >= SA && (SB == SA || SA == 2), "ring depths");
    static_assert((SA - 2) * (kDmaA + kDmaB) + kDmaB < 64, "vmcnt");
};

// MFMAs of one K step for a wave's NV live 32-row sub-tiles (A rows in one ring slot, B
// rows in another). Operand fragments are double-buffered in registers: the LDS reads of
// sub-step s + 1 are placed between the MFMAs of sub-step s (sched_group_barrier: MFMA /
// DS-read interleave).
template <class C, int NV, bool TR>
MOE_DEVICE void bf16_stage_mma(const uint8_t* base_a, const uint8_t* base_b,
                               const int (&a_off)[C::kTM], const int (&b_off)[C::kTN],
                               const int (&chunk_off)[C::kSub],
                               f32x16_t (&acc)[C::kTM][C::kTN]) {
    if (NV == 0) return;
    constexpr int NVv = NV > 0 ? NV : 1;
    bf16x8_t av[2][NVv], bv[2][C::kTN];
#pragma unroll
    for (int j = 0; j < C::kTN; ++j) bv[0][j] = *(const bf16x8_t*)(base_b + b_off[j] + chunk_off[0]);
#pragma unroll
    for (int i = 0; i < NV; ++i) av[0][i] = *(const bf16x8_t*)(base_a + a_off[i] + chunk_off[0]);
#pragma unroll
    for (int s = 0; s < C::kSub; ++s) {
        const int cur = s & 1, nxt = cur ^ 1;
        if (s + 1 < C::kSub) {
#pragma unroll
            for (int j = 0; j < C::kTN; ++j)
                bv[nxt][j] = *(const bf16x8_t*)(base_b + b_off[j] + chunk_off[s + 1]);
#pragma unroll
            for (int i = 0; i < NV; ++i)
                av[nxt][i] = *(const bf16x8_t*)(base_a + a_off[i] + chunk_off[s + 1]);
        }
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
            for (int j = 0; j < C::kTN; ++j)
                acc[i][j] = TR ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[cur][j], av[cur][i],
                                                                         acc[i][j], 0, 0, 0)
                               : __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[cur][i], bv[cur][j],
                                                                         acc[i][j], 0, 0, 0);
    }
#ifndef MOE_NO_SCHED_INTERLEAVE
    constexpr int kReads = C::kTN + NVv;
    constexpr int kMfma = NVv * C::kTN;
    __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
#pragma unroll
    for (int s = 0; s < C::kSub; ++s) {
#pragma unroll
        for (int x = 0; x < kMfma; ++x) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (s + 1 < C::kSub && x < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    }
#endif
}

// K loop with direct global -> LDS loads into two rings: A (activations) SA slots deep,
// B (weights) SB >= SA slots deep. Step t issues A(t + SA - 1) and then B(t + SB - 1), so the
// weight stream -- which carries most of the HBM misses -- is prefetched further ahead.
// vmcnt: loads complete in issue order, so step kt may proceed once at most the loads issued
// after the later of A(kt), B(kt) remain.
template <class C, int NV, bool TR, class IssueA, class IssueB>
MOE_DEVICE void bf16_kloop(int nk, const uint8_t* lds, IssueA& issue_a, IssueB& issue_b,
                           const int (&a_off)[C::kTM], const int (&b_off)[C::kTN],
                           const int (&chunk_off)[C::kSub],
                           f32x16_t (&acc)[C::kTM][C::kTN]) {
    constexpr int SA = C::kSA, SB = C::kSB;
    constexpr int kStep = C::kDmaA + C::kDmaB;
    if (SB == SA) {
#pragma unroll
        for (int s = 0; s < SA - 1; ++s)
            if (s < nk) { issue_a(s, s); issue_b(s, s); }
    } else {            // SA == 2: B(0) .. B(SB - 3), A(0), B(SB - 2)
#pragma unroll
        for (int s = 0; s < SB - 2; ++s)
            if (s < nk) issue_b(s, s);
        issue_a(0, 0);
        if (SB - 2 < nk) issue_b(SB - 2, SB - 2);
    }
    int sa = 0, sb = 0;
    for (int kt = 0; kt < nk; ++kt) {
        if (SB == SA) {
            // stage kt has landed once at most min(SA - 2, nk - 1 - kt) later steps remain
            const int later = nk - 1 - kt;
            if (later >= SA - 2) wait_vm_lgkm0<(SA - 2) * kStep>();
            else if (later >= 2) wait_vm_lgkm0<cmin(2, SA - 2) * kStep>();
            else if (later >= 1) wait_vm_lgkm0<cmin(1, SA - 2) * kStep>();
            else wait_vm_lgkm0<0>();
        } else {
            // after A(kt) only B(kt + SB - 2) was issued, if it exists
            if (kt + SB - 2 < nk) wait_vm_lgkm0<C::kDmaB>();
            else wait_vm_lgkm0<0>();
        }
        block_sync();
        {
            int na = sa + SA - 1;
            if (na >= SA) na -= SA;
            int nb = sb + SB - 1;
            if (nb >= SB) nb -= SB;
            if (kt + SA - 1 < nk) issue_a(kt + SA - 1, na);
            if (kt + SB - 1 < nk) issue_b(kt + SB - 1, nb);
        }
        bf16_stage_mma<C, NV, TR>(lds + sa * C::kASlot, lds + C::kBRing + sb * C::kBSlot, a_off,
                                  b_off, chunk_off, acc);
        if (++sa == SA) sa = 0;
        if (++sb == SB) sb = 0;
    }
}

// Ping-pong K loop. The 8 waves form two groups of four, one wave of each group on every
// SIMD (waves w and w + 4 share a SIMD). A K step (one ring slot: 32 K of A and of B) is two
// phases per group: M (LDS reads of the step's two MFMA sub-steps into registers, plus this
// group's DMAs of step s + S - 1: group 0 fills the A slot, group 1 the B slot) and C (the
// step's MFMAs, from registers). Group 1 starts one barrier late, so between any two
// barriers one group runs MFMAs while the other reads and issues loads, and every SIMD's
// matrix unit has one wave feeding it in every phase. Every wave passes the same number of
// barriers (group 1's extra one first, group 0's last). Slot s % S is last read in interval
// 2s + 1 and refilled (step s + S) from interval 2s + 2; a group waits for its own DMAs of
// step s + 1 before the barrier that ends interval 2s + 1.
template <class C, int NV>
MOE_DEVICE void bf16_kloop_pp(int nst, const uint8_t* lds, const uint8_t* const (&src)[4],
                              size_t step_bytes, int grp, int gw,
                              const int (&a_off)[C::kTM], const int (&b_off)[C::kTN],
                              const int (&chunk_off)[C::kSub],
                              f32x16_t (&acc)[C::kTM][C::kTN]) {
    constexpr int S = C::kSA;
    constexpr int kQ = 4;                        // DMAs per wave per step (16 KB / 1 KB / 4)
    // DMA look-ahead in steps: slot (s - 1) % S is refilled (step s + S - 1) in the M phase
    // of step s, after its last reader (group 1's M phase of step s - 1)
    constexpr int LA = S - 1;
    static_assert(LA >= 1, "look-ahead");
    static_assert(C::kSA == C::kSB && S >= 3 && C::kSub == 2 && C::kWaves == 8 &&
                  C::kASlot == 16384 && C::kBSlot == 16384 && (S - 1) * kQ < 64, "ping-pong");
    constexpr int NVv = NV > 0 ? NV : 1;
    bf16x8_t av[2][NVv], bv[2][C::kTN];
    const int ring = grp == 0 ? 0 : C::kBRing;
    auto issue = [&](int st) {
        MOE_LDS uint8_t* base = (MOE_LDS uint8_t*)lds + ring + (st % S) * 16384;
#pragma unroll
        for (int q = 0; q < kQ; ++q)
            __builtin_amdgcn_global_load_lds((const void*)(src[q] + (size_t)st * step_bytes),
                                             (MOE_LDS void*)(base + (gw + q * 4) * 1024), 16,
                                             0, 0);
    };
    auto read = [&](int st) {
        if (NV == 0) return;
        const uint8_t* ca = lds + (st % S) * C::kASlot;
        const uint8_t* cb = lds + C::kBRing + (st % S) * C::kBSlot;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int j = 0; j < C::kTN; ++j)
                bv[u][j] = *(const bf16x8_t*)(cb + b_off[j] + chunk_off[u]);
#pragma unroll
            for (int i = 0; i < NV; ++i)
                av[u][i] = *(const bf16x8_t*)(ca + a_off[i] + chunk_off[u]);
        }
    };
    auto mma = [&]() {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < NV; ++i)
#pragma unroll
                for (int j = 0; j < C::kTN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[u][j], av[u][i],
                                                                        acc[i][j], 0, 0, 0);
    };
    // this group's DMAs of step s + 1 have landed (later steps may still be in flight)
    auto wait_next = [&](int st) {
        if (st + LA < nst) wait_vm_lgkm0<(LA - 1) * kQ>();
        else wait_vm_lgkm0<0>();
    };
#pragma unroll
    for (int st = 0; st < LA; ++st)
        if (st < nst) issue(st);
    if (nst - 1 >= LA - 1) wait_vm_lgkm0<(LA - 1) * kQ>();
    else wait_vm_lgkm0<0>();
    block_sync();                                // step 0 visible
    if (grp == 1) block_sync();
    for (int st = 0; st < nst; ++st) {
        read(st);                                // M
        if (st + LA < nst) issue(st + LA);
        if (grp == 0) wait_vm_lgkm0<63>();       // LDS reads only
        else wait_next(st);
        block_sync();
        mma();                                   // C
        if (grp == 0) wait_next(st);
        block_sync();
    }
    if (grp == 0) block_sync();
    wait_vm_lgkm0<0>();
}

// Interleaved K loop, for tiles whose A and B slots differ in size (the 128 x 512 shape):
// K step 32 (two MFMA sub-steps), S >= 3 ring slots, one barrier per K step placed between
// the step's two sub-steps:
//   phase A: LDS reads of sub-step 1 of step kt, interleaved with the MFMAs of sub-step 0;
//   wait for this wave's DMAs of step kt + 1 and for its LDS reads, then the barrier (step
//   kt + 1 is visible, and every wave is done reading slot kt % S);
//   phase B: the DMAs of step kt + S into slot kt % S and the reads of sub-step 0 of step
//   kt + 1, interleaved with the MFMAs of sub-step 1.
// A DMA has S - 1 steps to land. Past the last step the DMAs re-load the last step into the
// free slot, and the reads of the step after the last read a slot that holds a landed copy
// (no branch in the loop, so the scheduler can interleave; those values are never used).
template <class C, int NV, class IssueA, class IssueB>
MOE_DEVICE void bf16_kloop_il(int nk, const uint8_t* lds, IssueA& issue_a, IssueB& issue_b,
                              const int (&a_off)[C::kTM], const int (&b_off)[C::kTN],
                              const int (&chunk_off)[C::kSub],
                              f32x16_t (&acc)[C::kTM][C::kTN]) {
    constexpr int S = C::kSA;
    constexpr int Q = C::kDmaA + C::kDmaB;               // DMAs per wave per step
    static_assert(C::kSA == C::kSB && S >= 3 && C::kSub == 2 && (S - 1) * Q < 64,
                  "interleaved loop");
    constexpr int NVv = NV > 0 ? NV : 1;
    constexpr int kMfma = NVv * C::kTN, kReads = NVv + C::kTN;
    bf16x8_t av[2][NVv], bv[2][C::kTN];
    auto read = [&](int st, int u) {
        if (NV == 0) return;
        const uint8_t* ca = lds + (st % S) * C::kASlot;
        const uint8_t* cb = lds + C::kBRing + (st % S) * C::kBSlot;
#pragma unroll
        for (int j = 0; j < C::kTN; ++j) bv[u][j] = *(const bf16x8_t*)(cb + b_off[j] + chunk_off[u]);
#pragma unroll
        for (int i = 0; i < NV; ++i) av[u][i] = *(const bf16x8_t*)(ca + a_off[i] + chunk_off[u]);
    };
    auto mma = [&](int u) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
            for (int j = 0; j < C::kTN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[u][j], av[u][i], acc[i][j],
                                                                    0, 0, 0);
    };
    auto issue = [&](int st) {
        const int t = st < nk ? st : nk - 1;
        issue_a(t, st % S);
        issue_b(t, st % S);
    };
#pragma unroll
    for (int st = 0; st < S; ++st) issue(st);
    wait_vm_lgkm0<(S - 1) * Q>();                        // step 0 landed
    block_sync();
    read(0, 0);
    for (int kt = 0; kt < nk; ++kt) {
        read(kt, 1);                                     // phase A
        mma(0);
        if (NV > 0) {
#pragma unroll
            for (int x = 0; x < kMfma; ++x) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (x < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }
        wait_vm_lgkm0<(S - 2) * Q>();                    // step kt + 1 landed, reads done
        block_sync();
        issue(kt + S);                                   // phase B
        read(kt + 1, 0);
        mma(1);
        if (NV > 0) {
#pragma unroll
            for (int x = 0; x < kMfma; ++x) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (x < Q) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                if (x < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }
    }
    wait_vm_lgkm0<0>();
}

// One output tile of the bf16 kernel: rows [m0, Mg) of group g of segment seg (the group's
// rows start at global row rbase), N tile nt.
template <int KIND, int BM, int BN, int BK, int WM, int WN, int SA, int SB>
MOE_DEVICE void bf16_tile(const GemmArgs& ga, int seg, int g, int m0, int Mg, int rbase, int nt,
                          uint8_t* lds) {
    using C = BfCfg<KIND, BM, BN, BK, WM, WN, SA, SB>;
    const SegDev S = seg == 0 ? ga.seg[0] : ga.seg[1];
    const int N = ga.N, K = ga.K;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int wm = wave / WN, wn = wave % WN;
    // live rows of the tile, and this wave's live 32-row sub-tiles (its sub-tile i is tile
    // rows C::sub_row(wm, i) + [0, 32); the live ones are a prefix i < nvi)
    const int live = Mg - m0 < BM ? Mg - m0 : BM;
    int nvi = C::kInterleave ? ((live + 31) / 32 - wm + WM - 1) / WM
                             : (live - wm * (BM / WM) + 31) / 32;
    nvi = nvi < 0 ? 0 : (nvi > C::kTM ? C::kTM : nvi);
    nvi = __builtin_amdgcn_readfirstlane(nvi);

    // ---- DMA sources: instruction q of this wave fills tile rows
    //      kRowsPerDma * (wave + q * kWaves) + [0, kRowsPerDma) of A or of B
    const uint8_t* srcA[C::kDmaA];
    const uint8_t* srcB[C::kDmaB];
#pragma unroll
    for (int q = 0; q < C::kDmaA; ++q) {
        const int r = C::kRowsPerDma * (wave + q * C::kWaves) + lane / C::kCpr;
        const int c = (lane % C::kCpr) ^ chunk_swz<C::kCpr>(r);
        const int rr = m0 + r < Mg ? m0 + r : Mg - 1;              // clamp the ragged tail
        const int arow = S.a_rows ? S.a_rows[rbase + rr] : rbase + rr;
        const uint8_t* rowp = (const uint8_t*)S.a + (size_t)arow * S.a_row;
        srcA[q] = rowp + (size_t)(c / 4) * S.a_kstep + (c % 4) * 16;
    }
#pragma unroll
    for (int q = 0; q < C::kDmaB; ++q) {
        const int rb = C::kRowsPerDma * (wave + q * C::kWaves) + lane / C::kCpr;
        const int c = (lane % C::kCpr) ^ chunk_swz<C::kCpr>(rb);
        int wrow;
        if (KIND == 0)
            wrow = rb < BN / 2 ? nt * (BN / 2) + rb : N / 2 + nt * (BN / 2) + (rb - BN / 2);
        else
            wrow = nt * BN + rb;
        const uint8_t* rowp = (const uint8_t*)S.w + (size_t)g * S.w_mat + (size_t)wrow * S.w_row;
        srcB[q] = rowp + (size_t)(c / 4) * S.w_kstep + (c % 4) * 16;
    }
    // bytes per K step (64-byte K slices per step times the slice stride)
    const size_t a_step = (size_t)C::kSlices * S.a_kstep, w_step = (size_t)C::kSlices * S.w_kstep;
    auto issue_a = [&](int kstep, int slot) {
        MOE_LDS uint8_t* base = (MOE_LDS uint8_t*)lds + slot * C::kASlot;
#pragma unroll
        for (int q = 0; q < C::kDmaA; ++q)
            __builtin_amdgcn_global_load_lds((const void*)(srcA[q] + (size_t)kstep * a_step),
                                             (MOE_LDS void*)(base + (wave + q * C::kWaves) * 1024),
                                             16, 0, 0);
    };
    auto issue_b = [&](int kstep, int slot) {
        MOE_LDS uint8_t* base = (MOE_LDS uint8_t*)lds + C::kBRing + slot * C::kBSlot;
#pragma unroll
        for (int q = 0; q < C::kDmaB; ++q)
            __builtin_amdgcn_global_load_lds((const void*)(srcB[q] + (size_t)kstep * w_step),
                                             (MOE_LDS void*)(base + (wave + q * C::kWaves) * 1024),
                                             16, 0, 0);
    };

    // ---- MFMA operand addresses (bytes within a stage)
    int a_off[C::kTM], b_off[C::kTN];
#pragma unroll
    for (int i = 0; i < C::kTM; ++i)
        a_off[i] = (C::sub_row(wm, i) + lane % 32) * C::kRowBytes;
#pragma unroll
    for (int j = 0; j < C::kTN; ++j) {
        int row;
        if (KIND == 0) {
            constexpr int half = C::kTN / 2;
            const int col = wn * (BN / 2 / WN) + (j % half) * 32 + lane % 32;
            row = j < half ? col : BN / 2 + col;
        } else {
            row = wn * (BN / WN) + j * 32 + lane % 32;
        }
        b_off[j] = row * C::kRowBytes;                      // within a B ring slot
    }
    // physical chunk of logical chunk (2 s + lane / 32) of a row whose low bits are lane % 32
    int chunk_off[C::kSub];
#pragma unroll
    for (int s = 0; s < C::kSub; ++s)
        chunk_off[s] = ((2 * s + lane / 32) ^ chunk_swz<C::kCpr>(lane % 32)) * 16;

    f32x16_t acc[C::kTM][C::kTN];
#pragma unroll
    for (int i = 0; i < C::kTM; ++i)
#pragma unroll
        for (int j = 0; j < C::kTN; ++j) acc[i][j] = f32x16_t{};

    // GEMM1: the gates of the tile's live rows into LDS (read by the epilogue, after the
    // K loop's barriers), loaded while the first operand tiles are in flight
    float* gate_lds = (float*)(lds + C::kGateOff);
    if (C::kGateLds && tid < live) gate_lds[tid] = S.gate ? S.gate[rbase + m0 + tid] : 1.0f;

    // one branch-free K loop per count of live sub-tiles (every variant has the same
    // barriers, so waves of one block may take different variants)
    const int nk = K / BK;
    // ping-pong: one group of four waves fills the A slots, the other the B slots
    constexpr bool kPP = MOE_BF_PINGPONG && BM == 256 && BN == 256 && BK == 32 && SA == SB &&
                         SA >= 3 && WM * WN == 8;
    constexpr bool kIL = !kPP && BK == 32 && SA == SB && SA >= 3 && MOE_BF_KLOOP_IL;
    // wave-uniform (scalar) so the group's extra barrier is a scalar branch: s_barrier does
    // not look at the exec mask
    const int grp = __builtin_amdgcn_readfirstlane(wave / 4);
    const int gw = __builtin_amdgcn_readfirstlane(wave % 4);
    const uint8_t* src[4];
    if (kPP) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = C::kRowsPerDma * (gw + q * 4) + lane / C::kCpr;
            const int c = (lane % C::kCpr) ^ chunk_swz<C::kCpr>(r);
            if (grp == 0) {
                const int rr = m0 + r < Mg ? m0 + r : Mg - 1;
                const int arow = S.a_rows ? S.a_rows[rbase + rr] : rbase + rr;
                src[q] = (const uint8_t*)S.a + (size_t)arow * S.a_row +
                         (size_t)(c / 4) * S.a_kstep + (c % 4) * 16;
            } else {
                int wrow;
                if (KIND == 0)
                    wrow = r < BN / 2 ? nt * (BN / 2) + r : N / 2 + nt * (BN / 2) + (r - BN / 2);
                else
                    wrow = nt * BN + r;
                src[q] = (const uint8_t*)S.w + (size_t)g * S.w_mat + (size_t)wrow * S.w_row +
                         (size_t)(c / 4) * S.w_kstep + (c % 4) * 16;
            }
        }
    }
    const size_t pp_step = grp == 0 ? a_step : w_step;
    switch (nvi) {
#define MOE_KLOOP_CASE(V)                                                                   \
    case V:                                                                                 \
        if (V <= C::kTM) {                                                                  \
            constexpr int NV = V <= C::kTM ? V : C::kTM;                                    \
            if constexpr (kPP)                                                              \
                bf16_kloop_pp<C, NV>(nk, lds, src, pp_step, grp, gw, a_off, b_off,          \
                                     chunk_off, acc);                                       \
            else if constexpr (kIL)                                                         \
                bf16_kloop_il<C, NV>(nk, lds, issue_a, issue_b, a_off, b_off, chunk_off,    \
                                     acc);                                                  \
            else                                                                            \
                bf16_kloop<C, NV, true>(nk, lds, issue_a, issue_b, a_off, b_off, chunk_off,  \
                                        acc);                                               \
        }                                                                                   \
        break;
    MOE_KLOOP_CASE(0)
    MOE_KLOOP_CASE(1)
    MOE_KLOOP_CASE(2)
    MOE_KLOOP_CASE(3)
    MOE_KLOOP_CASE(4)
    MOE_KLOOP_CASE(5)
    MOE_KLOOP_CASE(6)
    MOE_KLOOP_CASE(7)
    MOE_KLOOP_CASE(8)
#undef MOE_KLOOP_CASE
    default: break;
    }

    // epilogue, straight from the registers. The weights are the first MFMA operand, so
    // element r of lane l of sub-tile (i, j) is tile row sub_row(wm, i) + l % 32 and column
    // 8 (r / 4) + 4 (l / 32) + r % 4 of the sub-tile's 32: every lane holds runs of four
    // consecutive columns of one row and writes each run with one 8-byte store (a row's 64
    // bytes of a sub-tile come from lanes l and l + 32 in four stores).
    uint16_t* out = (uint16_t*)S.out;
    if (KIND == 0) {
        constexpr int half = C::kTN / 2;
        const int F = N / 2;
        uint16_t* zo = (uint16_t*)S.z_out;
        const int h = lane / 32;
#pragma unroll
        for (int i = 0; i < C::kTM; ++i) {
            if (i >= nvi) continue;
            const int row = C::sub_row(wm, i) + lane % 32;
            const bool live_row = m0 + row < Mg;       // lanes l and l + 32 share a row
            const int lr = live_row ? row : live - 1;
            const size_t grow = (size_t)rbase + m0 + lr;
            const float gt = C::kGateLds ? gate_lds[lr] : S.gate ? S.gate[grow] : 1.0f;
#pragma unroll
            for (int jj = 0; jj < half; ++jj)
#pragma unroll
                for (int qp = 0; qp < 4; qp += 2) {
                    // runs qp and qp + 1 of act, paired across lanes l, l + 32 (pair_runs_x4)
                    const f32x16_t& g = acc[i][jj];
                    const f32x16_t& u = acc[i][half + jj];
                    float a[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) a[e] = gt * (silu_fast(g[4 * qp + e]) * u[4 * qp + e]);
                    const uint4 v = pair_runs_x4(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                                 pack_bf16x2(a[4], a[5]), pack_bf16x2(a[6], a[7]));
                    const int col = nt * (BN / 2) + wn * (BN / 2 / WN) + jj * 32 + 8 * (qp + h);
                    const size_t oi = S.out_kblock
                                          ? ((size_t)(col / 32) * S.rows_total + grow) * 32 + col % 32
                                          : grow * F + col;
                    if (live_row) *(uint4*)(out + oi) = v;
                    if (zo) {
                        const uint4 zg = pair_runs_x4(pack_bf16x2(g[4 * qp], g[4 * qp + 1]),
                                                      pack_bf16x2(g[4 * qp + 2], g[4 * qp + 3]),
                                                      pack_bf16x2(g[4 * qp + 4], g[4 * qp + 5]),
                                                      pack_bf16x2(g[4 * qp + 6], g[4 * qp + 7]));
                        const uint4 zu = pair_runs_x4(pack_bf16x2(u[4 * qp], u[4 * qp + 1]),
                                                      pack_bf16x2(u[4 * qp + 2], u[4 * qp + 3]),
                                                      pack_bf16x2(u[4 * qp + 4], u[4 * qp + 5]),
                                                      pack_bf16x2(u[4 * qp + 6], u[4 * qp + 7]));
                        if (live_row) {
                            *(uint4*)(zo + grow * N + col) = zg;
                            *(uint4*)(zo + grow * N + F + col) = zu;
                        }
                    }
                }
        }
    } else {
        // GEMM2's bf16 tile (128 KB) goes through LDS: each lane's runs of four columns as
        // 8-byte writes into [BM][kEpCols + 8], then 16-byte row chunks to global memory
        // (measured 1-3% faster here than 8- or 16-byte stores straight from the registers)
        constexpr int kEpCols = C::kEpCols, kEpStride = C::kEpStride;
        block_sync();                                   // every wave is done with the stages
        uint16_t* ep = (uint16_t*)lds;
#pragma unroll
        for (int i = 0; i < C::kTM; ++i) {
            if (i >= nvi) continue;
            const int row = C::sub_row(wm, i) + lane % 32;
#pragma unroll
            for (int j = 0; j < C::kTN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int lcol = wn * (BN / WN) + j * 32 + 8 * q + 4 * (lane / 32);
                    *(uint2*)(ep + row * kEpStride + lcol) =
                        make_uint2(pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                                   pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
                }
        }
        __syncthreads();
        constexpr int kChunks = kEpCols / 8;            // 16-byte chunks per tile row
        const int c0 = nt * kEpCols;                    // first output column of the tile
        for (int c = tid; c < live * kChunks; c += C::kThreads) {
            const int row = c / kChunks, cc = c % kChunks;
            const uint4 v = *(const uint4*)(ep + row * kEpStride + cc * 8);
            *(uint4*)(out + ((size_t)rbase + m0 + row) * N + c0 + cc * 8) = v;
        }
    }
}

// One 256 x 256 (or other single-shape) tile per workgroup, from the M-tile schedule.
template <int KIND, int BM, int BN, int BK, int WM, int WN, int SA, int SB>
__global__ __launch_bounds__(WM * WN * 64) void gemm_bf16_kernel(GemmArgs ga) {
    extern __shared__ __align__(16) uint8_t lds[];
    int mt, nt;
    if (!pick_tile(ga, mt, nt)) return;
    const int4 ti = ga.tiles[mt];
    bf16_tile<KIND, BM, BN, BK, WM, WN, SA, SB>(ga, ti.x >> 20, ti.x & 0xFFFFF, ti.y,
                                                tile_end(ti.y, ti.z, ga.bm), ti.w, nt, lds);
}

// Mixed shapes (schedule_mixed_kernel): workgroup b takes unit (b % 8) * per + b / 8, so
// each XCD walks one contiguous run of the unit table; shape 0 runs the 256 x 256
// configuration, shape 1 the 128 x 512 one.
template <int KIND, class C0, class C1>
__global__ __launch_bounds__(512) void gemm_bf16_mixed_kernel(GemmArgs ga) {
    static_assert(C0::kThreads == 512 && C1::kThreads == 512, "8 waves");
    extern __shared__ __align__(16) uint8_t lds[];
    const int b = blockIdx.x;
    const int xcd = b % 8, i = b / 8;
    const int total = *ga.total;
    const int per = (total + 7) / 8;
    if (i >= per) return;
    const int L = xcd * per + i;
    if (L >= total) return;
    const int4 u = ga.units[L];
    const int nt = ga.unit_nt[L];
    const int seg = (u.x >> 20) & 1, g = u.x & 0xFFFFF;
    if ((u.x >> 21) == 0)
        bf16_tile<KIND, C0::kBM, C0::kBN, C0::kBK, C0::kWM, C0::kWN, C0::kSA, C0::kSB>(
            ga, seg, g, u.y, u.z, u.w, nt, lds);
    else
        bf16_tile<KIND, C1::kBM, C1::kBN, C1::kBK, C1::kWM, C1::kWN, C1::kSA, C1::kSB>(
            ga, seg, g, u.y, u.z, u.w, nt, lds);
}

// ---------------------------------------------------------------------------------------
// e4m3 MFMA kernel: block-scaled fp8 operands (1 x 128 activation scales, 128 x 128 weight
// scales), fp32 accumulation.
//
// One LDS stage holds one 128-wide K block: [BM A rows | BN B rows] x 128 bytes plus the
// fp32 scales of the BM A rows for that block (each wave DMAs 16 of them). The MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4 with unit E8M0 scales) sums the K block into a partial
// tile, which is then promoted into the accumulator with the block's two scales:
//   acc[m][n] += partial[m][n] * s_a[m][kb] * s_w[n / 128][kb].
// GEMM1's tile spans 128 act columns, i.e. exactly one 1 x 128 quantisation block of act,
// so the epilogue folds the gate in, reduces each row's amax across lanes and waves (LDS),
// and writes the e4m3 codes and their scale directly.
// ---------------------------------------------------------------------------------------
template <int KIND, int BM, int BN, int WM, int WN, int STAGES>
struct F8Cfg {
    static constexpr int kThreads = WM * WN * kWave;
    static constexpr int kWaves = WM * WN;
    static constexpr int kRowBytes = 128;                   // 128 e4m3 of K
    static constexpr int kRows = BM + BN;
    static constexpr int kTileBytes = kRows * kRowBytes;
    static constexpr int kRpw = BM / kWaves;                // A-row scales DMA'd per wave
    static constexpr int kScaleBytes = kWaves * 256;        // 64 floats per wave (kRpw used)
    static constexpr int kStageBytes = kTileBytes + kScaleBytes;
    static constexpr int kDma = kRows / 8 / kWaves;         // tile DMAs per wave per stage
    static constexpr int kVm = kDma + 1;                    // + the scale DMA
    static constexpr int kTM = BM / WM / 32;
    static constexpr int kTN = BN / WN / 32;
    static constexpr int kStages = STAGES;
    static constexpr size_t kLds = (size_t)STAGES * kStageBytes;
    static_assert(BM % kWaves == 0 && kRpw <= 64, "one scale group of kRpw rows per wave");
    static_assert(kRows % (8 * kWaves) == 0, "DMA split");
    static_assert(KIND == 1 || (kTN == 2 && BN == 256), "GEMM1: one 128-column act block");
    static_assert(kLds <= 160 * 1024, "LDS");
    static_assert(STAGES >= 2 && (STAGES - 2) * kVm < 64, "vmcnt");
    static_assert(BM * WN * 4 <= kStageBytes, "epilogue amax buffer");
};

MOE_DEVICE i32x8_t lds_frag32(const uint8_t* p0, const uint8_t* p1) {
    const i32x4_t lo = *(const i32x4_t*)p0, hi = *(const i32x4_t*)p1;
    return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// K loop of the e4m3 kernel. The MFMA takes the weight fragment as its first operand and the
// activation fragment as its second, so a lane's 16 accumulator values of a 32 x 32 sub-tile
// are one output row m (lane % 32) and 16 output columns n that lie in one 128-column weight
// block: the promotion factor s_a[m][kb] * s_w[nb][kb] is one scalar per lane and sub-tile,
// and promoting a partial tile costs 16 FMAs and one multiply per lane.
template <class C, int NV, class Issue>
MOE_DEVICE void e4m3_kloop(int nk, const uint8_t* lds, Issue& issue, const int (&a_off)[C::kTM],
                           const int (&b_off)[C::kTN], const int (&co)[2][2], int wm, int lane,
                           const float* __restrict__ wsc,
                           const int (&wsc_off)[C::kTN], f32x16_t (&acc)[C::kTM][C::kTN]) {
    constexpr int STAGES = C::kStages;
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < nk) issue(s, s);
    // the weight-block scales of K block kt + 1 are loaded during block kt (a scalar load whose
    // wait would otherwise sit in front of the block's first MFMAs)
    float sw_next[C::kTN];
#pragma unroll
    for (int j = 0; j < C::kTN; ++j) sw_next[j] = NV > 0 ? wsc[wsc_off[j]] : 0.0f;
    int stage = 0;
    for (int kt = 0; kt < nk; ++kt) {
        const int later = nk - 1 - kt;
        if (later >= STAGES - 2) wait_vm_lgkm0<(STAGES - 2) * C::kVm>();
        else if (later >= 2) wait_vm_lgkm0<cmin(2, STAGES - 2) * C::kVm>();
        else if (later >= 1) wait_vm_lgkm0<cmin(1, STAGES - 2) * C::kVm>();
        else wait_vm_lgkm0<0>();
        block_sync();
        {
            const int kn = kt + STAGES - 1;
            int sn = stage + STAGES - 1;
            if (sn >= STAGES) sn -= STAGES;
            if (kn < nk) issue(kn, sn);
        }
        if (NV > 0) {
            constexpr int NVv = NV > 0 ? NV : 1;
            const uint8_t* base = lds + stage * C::kStageBytes;
            const float* sa_l = (const float*)(base + C::kTileBytes);
            float sw[C::kTN];
#pragma unroll
            for (int j = 0; j < C::kTN; ++j) {
                sw[j] = sw_next[j];
                if (kt + 1 < nk) sw_next[j] = wsc[wsc_off[j] + kt + 1];
            }
            i32x8_t bv[2][C::kTN];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int j = 0; j < C::kTN; ++j)
                    bv[s2][j] = lds_frag32(base + b_off[j] + co[s2][0], base + b_off[j] + co[s2][1]);
#pragma unroll
            for (int i = 0; i < NVv; ++i) {
                // this lane's output row of sub-tile i and its activation scale (wave w DMA'd
                // the scales of tile rows kRpw w + [0, kRpw) to float kRpw-group * 64)
                const int row = wm * (C::kTM * 32) + i * 32 + lane % 32;
                const float sa = sa_l[(row / C::kRpw) * 64 + row % C::kRpw];
                const i32x8_t a0 = lds_frag32(base + a_off[i] + co[0][0], base + a_off[i] + co[0][1]);
                const i32x8_t a1 = lds_frag32(base + a_off[i] + co[1][0], base + a_off[i] + co[1][1]);
#pragma unroll
                for (int j = 0; j < C::kTN; ++j) {
                    f32x16_t pt = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        bv[0][j], a0, f32x16_t{}, 0, 0, 0, 0x7F7F7F7F, 0, 0x7F7F7F7F);
                    pt = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        bv[1][j], a1, pt, 0, 0, 0, 0x7F7F7F7F, 0, 0x7F7F7F7F);
                    const float c = sa * sw[j];
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] = fmaf(pt[r], c, acc[i][j][r]);
                }
            }
        }
        if (++stage == STAGES) stage = 0;
    }
}

template <int KIND, int BM, int BN, int WM, int WN, int STAGES>
__global__ __launch_bounds__(WM * WN * 64) void gemm_e4m3_kernel(GemmArgs ga) {
    using C = F8Cfg<KIND, BM, BN, WM, WN, STAGES>;
    extern __shared__ __align__(16) uint8_t lds[];
    int mt, nt;
    if (!pick_tile(ga, mt, nt)) return;
    const int4 ti = ga.tiles[mt];
    const int seg = ti.x >> 20, g = ti.x & 0xFFFFF;
    const int m0 = ti.y, Mg = tile_end(ti.y, ti.z, ga.bm), rbase = ti.w;   // Mg: tile end
    const SegDev S = seg == 0 ? ga.seg[0] : ga.seg[1];
    const int N = ga.N, K = ga.K, KB = K / 128;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int wm = wave / WN, wn = wave % WN;
    const int live = Mg - m0 < BM ? Mg - m0 : BM;
    int nvi = (live - wm * (BM / WM) + 31) / 32;
    nvi = nvi < 0 ? 0 : (nvi > C::kTM ? C::kTM : nvi);
    nvi = __builtin_amdgcn_readfirstlane(nvi);

    // ---- tile DMA sources (as the bf16 kernel, 128-byte stage rows): 32-bit offsets from the
    // segment's activation base and the group's weight base
    const uint8_t* abase = (const uint8_t*)S.a;
    const uint8_t* wbase = (const uint8_t*)S.w + (size_t)g * S.w_mat;
    // instruction q fills tile rows 64 q + rl (rl = 8 wave + lane / 8): A rows (gathered) for
    // q < kDmaA, else B rows 64 (q - kDmaA) + rl of the weight tile. Rows 64 apart share the
    // chunk swizzle, so a B instruction's source is a wave-uniform row base plus one lane
    // offset (lane_b) for all of them (fewer VGPRs than one offset per instruction).
    constexpr int kDmaA = BM / 64, kDmaB = C::kDma - kDmaA;
    static_assert(BM % 64 == 0 && (KIND == 1 || (BN / 2) % 64 == 0), "64-row DMA groups");
    const int rl = 8 * wave + lane / 8;
    const int cl = (lane % 8) ^ chunk_swz<8>(rl);
    const size_t a_step = S.a_kstep, w_step = S.w_kstep;
    uint32_t src[kDmaA];
#pragma unroll
    for (int q = 0; q < kDmaA; ++q) {
        const int r = 64 * q + rl;
        const int rr = m0 + r < Mg ? m0 + r : Mg - 1;
        const size_t rowp = (size_t)(S.a_rows ? S.a_rows[rbase + rr] : rbase + rr) * S.a_row;
        src[q] = (uint32_t)(rowp + (size_t)(cl / 4) * a_step + (cl % 4) * 16);
    }
    const uint32_t lane_b =
        (uint32_t)((size_t)rl * S.w_row + (size_t)(cl / 4) * w_step + (cl % 4) * 16);
    auto wrow0 = [&](int qb) -> size_t {            // first weight row of B instruction qb
        const int rb = 64 * qb;
        if (KIND == 0)
            return rb < BN / 2 ? (size_t)nt * (BN / 2) + rb
                               : (size_t)N / 2 + (size_t)nt * (BN / 2) + (rb - BN / 2);
        return (size_t)nt * BN + rb;
    };
    // A-row scales: wave w loads rows kRpw w + lane % kRpw of this tile
    const float* ssrc;
    {
        const int r = C::kRpw * wave + lane % C::kRpw;
        const int rr = m0 + r < Mg ? m0 + r : Mg - 1;
        ssrc = (const float*)S.a_scales + (size_t)(S.a_rows ? S.a_rows[rbase + rr] : rbase + rr) * KB;
    }
    auto issue = [&](int kstep, int stage) {
        MOE_LDS uint8_t* base = (MOE_LDS uint8_t*)lds + stage * C::kStageBytes;
#pragma unroll
        for (int q = 0; q < kDmaA; ++q)
            __builtin_amdgcn_global_load_lds(
                (const void*)(abase + src[q] + (size_t)kstep * 2 * a_step),
                (MOE_LDS void*)(base + (wave + q * C::kWaves) * 1024), 16, 0, 0);
#pragma unroll
        for (int qb = 0; qb < kDmaB; ++qb)
            __builtin_amdgcn_global_load_lds(
                (const void*)(wbase + wrow0(qb) * S.w_row + lane_b + (size_t)kstep * 2 * w_step),
                (MOE_LDS void*)(base + (wave + (kDmaA + qb) * C::kWaves) * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(ssrc + kstep),
                                         (MOE_LDS void*)(base + C::kTileBytes + wave * 256), 4, 0, 0);
    };

    int a_off[C::kTM], b_off[C::kTN];
#pragma unroll
    for (int i = 0; i < C::kTM; ++i) a_off[i] = (wm * (BM / WM) + i * 32 + lane % 32) * 128;
#pragma unroll
    for (int j = 0; j < C::kTN; ++j) {
        int row;
        if (KIND == 0) {
            constexpr int half = C::kTN / 2;
            const int col = wn * (BN / 2 / WN) + (j % half) * 32 + lane % 32;
            row = BM + (j < half ? col : BN / 2 + col);
        } else {
            row = BM + wn * (BN / WN) + j * 32 + lane % 32;
        }
        b_off[j] = row * 128;
    }
    // the lane's 32 bytes of K sub-step s: logical chunks 4 s + 2 h, 4 s + 2 h + 1
    int co[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int u = 0; u < 2; ++u)
            co[s][u] = ((4 * s + 2 * (lane / 32) + u) ^ chunk_swz<8>(lane % 32)) * 16;
    // weight-scale offsets (per sub-tile j): [g][n_block][kb]
    const int nbn = N / 128;
    int wsc_off[C::kTN];
#pragma unroll
    for (int j = 0; j < C::kTN; ++j) {
        int nb;
        if (KIND == 0) nb = j < C::kTN / 2 ? nt : N / 256 + nt;   // gate block nt, up block F/128 + nt
        else nb = (nt * BN + wn * (BN / WN) + j * 32) / 128;
        wsc_off[j] = __builtin_amdgcn_readfirstlane((g * nbn + nb) * KB);   // wave-uniform
    }

    f32x16_t acc[C::kTM][C::kTN];
#pragma unroll
    for (int i = 0; i < C::kTM; ++i)
#pragma unroll
        for (int j = 0; j < C::kTN; ++j) acc[i][j] = f32x16_t{};
    switch (nvi) {
#define MOE_F8_CASE(V)                                                                      \
    case V:                                                                                 \
        if (V <= C::kTM) {                                                                  \
            constexpr int NV = V <= C::kTM ? V : C::kTM;                                    \
            e4m3_kloop<C, NV>(KB, lds, issue, a_off, b_off, co, wm, lane,                   \
                              (const float*)S.w_scales, wsc_off, acc);                      \
        }                                                                                   \
        break;
    MOE_F8_CASE(0)
    MOE_F8_CASE(1)
    MOE_F8_CASE(2)
    MOE_F8_CASE(3)
    MOE_F8_CASE(4)
#undef MOE_F8_CASE
    default: break;
    }

    // Epilogue. Accumulator layout (weights as the first MFMA operand): element r of lane l of
    // sub-tile (i, j) is tile row wm * (BM / WM) + 32 i + l % 32 and tile column
    // wn * (BN / WN) + 32 j + 8 (r / 4) + 4 (l / 32) + r % 4, so every lane holds runs of four
    // consecutive columns of one row and writes them with one store.
    if (KIND == 1) {
        uint16_t* out = (uint16_t*)S.out;
#pragma unroll
        for (int i = 0; i < C::kTM; ++i) {
            if (i >= nvi) continue;
            const int row = wm * (BM / WM) + i * 32 + lane % 32;
            const bool live_row = m0 + row < Mg;       // lanes l and l + 32 share a row
            const size_t grow = (size_t)rbase + m0 + (live_row ? row : 0);
#pragma unroll
            for (int j = 0; j < C::kTN; ++j)
#pragma unroll
                for (int qp = 0; qp < 4; qp += 2) {
                    const f32x16_t& a = acc[i][j];
                    const uint4 v = pair_runs_x4(pack_bf16x2(a[4 * qp], a[4 * qp + 1]),
                                                 pack_bf16x2(a[4 * qp + 2], a[4 * qp + 3]),
                                                 pack_bf16x2(a[4 * qp + 4], a[4 * qp + 5]),
                                                 pack_bf16x2(a[4 * qp + 6], a[4 * qp + 7]));
                    const int col = nt * BN + wn * (BN / WN) + j * 32 + 8 * (qp + lane / 32);
                    if (live_row) *(uint4*)(out + grow * N + col) = v;
                }
        }
        return;
    }
    // ---- GEMM1: act = gate * silu(Z_g) * Z_u (sub-tile 0: gate columns, 1: the matching up
    // columns), quantised per row over this tile's 128 act columns (one 1 x 128 block): amax
    // over the lane's 16 values, its partner lane l ^ 32, then the WN waves (LDS)
    const int F = N / 2;
    float av[C::kTM][16];
    float* amax_l = (float*)lds;                       // [WN][BM]
    block_sync();                                      // every wave is done with the stages
#pragma unroll
    for (int i = 0; i < C::kTM; ++i) {
        const int row = wm * (BM / WM) + i * 32 + lane % 32;
        const int lr = m0 + row < Mg ? row : live - 1;
        const float gt = S.gate ? S.gate[(size_t)rbase + m0 + lr] : 1.0f;
        float m = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            av[i][r] = gt * (silu_fast(acc[i][0][r]) * acc[i][1][r]);
            m = fmaxf(m, fabsf(av[i][r]));
        }
        m = fmaxf(m, __shfl_xor(m, 32));
        if (lane < 32) amax_l[wn * BM + row] = m;
    }
    __syncthreads();
    uint8_t* outq = (uint8_t*)S.out;
#pragma unroll
    for (int i = 0; i < C::kTM; ++i) {
        if (i >= nvi) continue;
        const int row = wm * (BM / WM) + i * 32 + lane % 32;
        const bool live_row = m0 + row < Mg;           // lanes l and l + 32 share a row
        float m = 0.0f;
#pragma unroll
        for (int w = 0; w < WN; ++w) m = fmaxf(m, amax_l[w * BM + row]);
        const float sc = e4m3_scale(m);
        const size_t grow = (size_t)rbase + m0 + (live_row ? row : 0);
        uint32_t codes[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            codes[q] = e4m3x4(av[i][4 * q] / sc, av[i][4 * q + 1] / sc, av[i][4 * q + 2] / sc,
                              av[i][4 * q + 3] / sc);
#pragma unroll
        for (int qp = 0; qp < 4; qp += 2) {
            const uint2 v = pair_runs_x2(codes[qp], codes[qp + 1]);
            const int col = nt * (BN / 2) + wn * (BN / 2 / WN) + 8 * (qp + lane / 32);
            const size_t oi = S.out_kblock ? ((size_t)(col / 64) * S.rows_total + grow) * 64 + col % 64
                                           : grow * F + col;
            if (live_row) *(uint2*)(outq + oi) = v;
        }
        if (live_row && wn == 0 && lane < 32) ((float*)S.out_scales)[grow * (F / 128) + nt] = sc;
    }
}

// ---------------------------------------------------------------------------------------
// MXFP8 MFMA kernel: e4m3 operands with one E8M0 scale (a power of two) per 1 x 32 block
// along K, for the activations and for the weights alike.
//
// v_mfma_scale_f32_32x32x64_f8f6f4 applies block scales itself: of the 64 K of one step,
// K [0, 32) takes its scale from lanes 0-31 (row / column l % 32) and K [32, 64) from lanes
// 32-63, and a lane of half h holds K [16 h, 16 h + 16) in its first 16 bytes and
// K [32 + 16 h, 48 + 16 h) in its other 16 (measured on gfx950 with distinct per-lane scales;
// the scale operand's byte is picked by op_sel). So with each 32-byte MX block laid on one
// hardware block, a half-wave's lanes pass their rows' scale byte of that block and the
// products go straight into the fp32 accumulator: no partial tile, no promotion step.
//
// One LDS stage holds BK (128 or 64) K: [BM A rows | BN B rows] x BK bytes, its 16-byte chunks
// XOR-swizzled so that the lanes of a ds_read_b128 phase hit distinct banks (128-byte rows:
// chunk_swz<8>; 64-byte rows, four per bank line: chunk ^ (row / 2) % 4), then one
// 4-byte word per tile row: the E8M0 codes of the row's four blocks of the 128 K that hold
// the stage (byte b = block b), DMA'd by one 4-byte load per lane and wave. 64-K stages take
// half the LDS each, so twice as many fit and more loads are in flight per workgroup.
// GEMM1's epilogue folds the gate in and quantises act per 1 x 32 block: one block is the 32
// columns of a 32 x 32 sub-tile in one row, held by the 32 lanes of a half-wave, so its
// amax takes five butterflies and no cross-wave step.
// ---------------------------------------------------------------------------------------
template <int KIND, int BM, int BN, int WM, int WN, int STAGES, int BK>
struct MxCfg {
    static constexpr int kThreads = WM * WN * kWave;
    static constexpr int kWaves = WM * WN;
    static constexpr int kRowBytes = BK;                    // BK e4m3 of K per stage
    static constexpr int kChunks = BK / 16;                 // 16-byte chunks per stage row
    static constexpr int kRpi = 1024 / BK;                  // stage rows per 1 KB DMA
    static constexpr int kSub = BK / 64;                    // MFMA K steps per stage
    static constexpr int kRows = BM + BN;
    static constexpr int kTileBytes = kRows * kRowBytes;
    static constexpr int kScaleBytes = kWaves * 256;        // 64 words per wave
    static constexpr int kStageBytes = kTileBytes + kScaleBytes;
    static constexpr int kDma = kRows / kRpi / kWaves;      // tile DMAs per wave per stage
    static constexpr int kVm = kDma + 1;                    // + the scale-word DMA
    static constexpr int kTM = BM / WM / 32;
    static constexpr int kTN = BN / WN / 32;
    static constexpr int kStages = STAGES;
    static constexpr size_t kLds = (size_t)STAGES * kStageBytes;
    // epilogue staging: GEMM1 act codes [BM][BN/2 + 16] bytes and scale codes [BM][BN/64];
    // GEMM2 bf16 [BM][BN + 8]
    static constexpr int kEpStride = KIND == 0 ? BN / 2 + 16 : BN + 8;
    static constexpr size_t kEpBytes =
        KIND == 0 ? (size_t)BM * kEpStride + (size_t)BM * (BN / 64) : (size_t)BM * kEpStride * 2;
    static_assert(BK == 64 || BK == 128, "stage depth");
    static_assert(kRows <= kWaves * 64, "one scale DMA per wave covers the tile's rows");
    static_assert(kRows % (kRpi * kWaves) == 0 && BM % (kRpi * kWaves) == 0, "DMA split");
    static_assert(KIND == 1 || kTN % 2 == 0, "GEMM1: gate and up sub-tiles in pairs");
    static_assert(kLds <= 160 * 1024 && kEpBytes <= kLds, "LDS");
    static_assert(STAGES >= 2 && (STAGES - 2) * kVm < 64, "vmcnt");
};

// physical 16-byte chunk of logical chunk c in stage row r
template <int BK>
MOE_DEVICE int mx_swz(int c, int r) { return BK == 128 ? c ^ chunk_swz<8>(r) : c ^ ((r >> 1) & 3); }

template <class C, int NV, class Issue>
MOE_DEVICE void mx_kloop(int nk, const uint8_t* lds, Issue& issue, const int (&a_off)[C::kTM],
                         const int (&b_off)[C::kTN], const int (&co)[2][2], int half,
                         f32x16_t (&acc)[C::kTM][C::kTN]) {
    constexpr int STAGES = C::kStages;
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < nk) issue(s, s);
    int stage = 0;
    for (int kt = 0; kt < nk; ++kt) {
        const int later = nk - 1 - kt;
        if (later >= STAGES - 2) wait_vm_lgkm0<(STAGES - 2) * C::kVm>();
        else if (later >= 2) wait_vm_lgkm0<cmin(2, STAGES - 2) * C::kVm>();
        else if (later >= 1) wait_vm_lgkm0<cmin(1, STAGES - 2) * C::kVm>();
        else wait_vm_lgkm0<0>();
        block_sync();
        {
            const int kn = kt + STAGES - 1;
            int sn = stage + STAGES - 1;
            if (sn >= STAGES) sn -= STAGES;
            if (kn < nk) issue(kn, sn);
        }
        if (NV > 0) {
            constexpr int NVv = NV > 0 ? NV : 1;
            const uint8_t* base = lds + stage * C::kStageBytes;
            const uint32_t* words = (const uint32_t*)(base + C::kTileBytes);
            // this lane's scale bytes: block 2 s + half of its row within the stage's 128 K
            // (a 64-K stage is the (kt % 2)-th half of it), as byte 2 s after the shift
            const int sh = 8 * half + (C::kSub == 1 ? 16 * (kt & 1) : 0);
            uint32_t sb[C::kTN], sa[NVv];
#pragma unroll
            for (int j = 0; j < C::kTN; ++j) sb[j] = words[b_off[j] / C::kRowBytes] >> sh;
#pragma unroll
            for (int i = 0; i < NVv; ++i) sa[i] = words[a_off[i] / C::kRowBytes] >> sh;
#pragma unroll
            for (int s = 0; s < C::kSub; ++s) {
                i32x8_t bv[C::kTN];
#pragma unroll
                for (int j = 0; j < C::kTN; ++j)
                    bv[j] = lds_frag32(base + b_off[j] + co[s][0], base + b_off[j] + co[s][1]);
#pragma unroll
                for (int i = 0; i < NVv; ++i) {
                    const i32x8_t av =
                        lds_frag32(base + a_off[i] + co[s][0], base + a_off[i] + co[s][1]);
#pragma unroll
                    for (int j = 0; j < C::kTN; ++j) {
                        // weights as the first operand (transposed accumulators), each
                        // operand with its own block scales
                        if (s == 0)
                            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                bv[j], av, acc[i][j], 0, 0, 0, sb[j], 0, sa[i]);
                        else
                            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                bv[j], av, acc[i][j], 0, 0, 2, sb[j], 2, sa[i]);
                    }
                }
            }
        }
        if (++stage == STAGES) stage = 0;
    }
}

template <int KIND, int BM, int BN, int WM, int WN, int STAGES, int BK>
__global__ __launch_bounds__(WM * WN * 64) void gemm_mx_kernel(GemmArgs ga) {
    using C = MxCfg<KIND, BM, BN, WM, WN, STAGES, BK>;
    extern __shared__ __align__(16) uint8_t lds[];
    int mt, nt;
    if (!pick_tile(ga, mt, nt)) return;
    const int4 ti = ga.tiles[mt];
    const int seg = ti.x >> 20, g = ti.x & 0xFFFFF;
    const int m0 = ti.y, Mg = tile_end(ti.y, ti.z, ga.bm), rbase = ti.w;   // Mg: tile end
    const SegDev S = seg == 0 ? ga.seg[0] : ga.seg[1];
    const int N = ga.N, K = ga.K, KB = K / 32;          // KB: scale bytes per row
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int wm = wave / WN, wn = wave % WN, half = lane / 32;
    const int live = Mg - m0 < BM ? Mg - m0 : BM;
    int nvi = (live - wm * (BM / WM) + 31) / 32;
    nvi = nvi < 0 ? 0 : (nvi > C::kTM ? C::kTM : nvi);
    nvi = __builtin_amdgcn_readfirstlane(nvi);

    // weight row of tile row rb (GEMM1: gate rows, then the matching up rows)
    auto wrow_of = [&](int rb) {
        if (KIND == 0)
            return rb < BN / 2 ? nt * (BN / 2) + rb : N / 2 + nt * (BN / 2) + (rb - BN / 2);
        return nt * BN + rb;
    };
    auto arow_of = [&](int r) {
        const int rr = m0 + r < Mg ? m0 + r : Mg - 1;
        return S.a_rows ? S.a_rows[rbase + rr] : rbase + rr;
    };
    // ---- tile DMA sources: 32-bit offsets from the activation base and the group's weights
    const uint8_t* abase = (const uint8_t*)S.a;
    const uint8_t* wbase = (const uint8_t*)S.w + (size_t)g * S.w_mat;
    uint32_t src[C::kDma];
#pragma unroll
    for (int q = 0; q < C::kDma; ++q) {
        const int r = C::kRpi * (wave + q * C::kWaves) + lane / C::kChunks;
        const int c = mx_swz<BK>(lane % C::kChunks, r);       // logical chunk this lane loads
        const size_t rowp = r < BM ? (size_t)arow_of(r) * S.a_row : (size_t)wrow_of(r - BM) * S.w_row;
        const size_t step = r < BM ? S.a_kstep : S.w_kstep;
        src[q] = (uint32_t)(rowp + (size_t)(c / 4) * step + (c % 4) * 16);
    }
    const size_t a_step = S.a_kstep, w_step = S.w_kstep;
    // scale words: wave w DMAs those of tile rows 64 w + lane (lanes past the tile's rows
    // fetch the last row's word into the unused tail of the area)
    const uint8_t* ssrc;
    uint32_t s_kb;
    {
        int r = 64 * wave + lane;
        if (r >= C::kRows) r = C::kRows - 1;
        if (r < BM) {
            const int rr = m0 + r < Mg ? m0 + r : Mg - 1;
            const int srow = S.a_sc_direct ? rbase + rr : arow_of(r);
            ssrc = (const uint8_t*)S.a_scales + (size_t)srow * S.sa_row;
            s_kb = S.sa_kb;
        } else {
            ssrc = (const uint8_t*)S.w_scales + (size_t)g * N * KB +
                   (size_t)wrow_of(r - BM) * S.sw_row;
            s_kb = S.sw_kb;
        }
    }
    auto issue = [&](int kstep, int stage) {
        MOE_LDS uint8_t* base = (MOE_LDS uint8_t*)lds + stage * C::kStageBytes;
#pragma unroll
        for (int q = 0; q < C::kDma; ++q) {
            constexpr int kSl = BK / 64;                       // 64-byte K slices per stage
            const bool is_a = q * C::kRpi * C::kWaves < BM;
            __builtin_amdgcn_global_load_lds(
                (const void*)((is_a ? abase : wbase) + src[q] +
                              (size_t)kstep * kSl * (is_a ? a_step : w_step)),
                (MOE_LDS void*)(base + (wave + q * C::kWaves) * 1024), 16, 0, 0);
        }
        __builtin_amdgcn_global_load_lds((const void*)(ssrc + (size_t)(kstep * BK / 128) * s_kb),
                                         (MOE_LDS void*)(base + C::kTileBytes + wave * 256), 4, 0, 0);
    };

    int a_off[C::kTM], b_off[C::kTN];
#pragma unroll
    for (int i = 0; i < C::kTM; ++i) a_off[i] = (wm * (BM / WM) + i * 32 + lane % 32) * C::kRowBytes;
#pragma unroll
    for (int j = 0; j < C::kTN; ++j) {
        int row;
        if (KIND == 0) {
            constexpr int hf = C::kTN / 2;
            const int col = wn * (BN / 2 / WN) + (j % hf) * 32 + lane % 32;
            row = BM + (j < hf ? col : BN / 2 + col);
        } else {
            row = BM + wn * (BN / WN) + j * 32 + lane % 32;
        }
        b_off[j] = row * C::kRowBytes;
    }
    // the lane's bytes of K sub-step s (64 K): K [16 h, 16 h + 16) and [32 + 16 h, 48 + 16 h)
    // of it, i.e. logical chunks 4 s + h and 4 s + 2 + h of the stage row (every row the lane
    // reads has the low bits of lane % 32)
    int co[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int u = 0; u < 2; ++u) co[s][u] = mx_swz<BK>(4 * s + 2 * u + half, lane % 32) * 16;

    f32x16_t acc[C::kTM][C::kTN];
#pragma unroll
    for (int i = 0; i < C::kTM; ++i)
#pragma unroll
        for (int j = 0; j < C::kTN; ++j) acc[i][j] = f32x16_t{};
    const int nk = K / BK;
    switch (nvi) {
#define MOE_MX_CASE(V)                                                                      \
    case V:                                                                                 \
        if (V <= C::kTM) {                                                                  \
            constexpr int NV = V <= C::kTM ? V : C::kTM;                                    \
            mx_kloop<C, NV>(nk, lds, issue, a_off, b_off, co, half, acc);                   \
        }                                                                                   \
        break;
    MOE_MX_CASE(0)
    MOE_MX_CASE(1)
    MOE_MX_CASE(2)
    MOE_MX_CASE(3)
    MOE_MX_CASE(4)
#undef MOE_MX_CASE
    default: break;
    }

    // ---- epilogue. Weights are the first MFMA operand: element r of lane l of sub-tile
    // (i, j) is tile row wm * (BM / WM) + 32 i + l % 32 and column
    // wn * (BN / WN) + 32 j + 8 (r / 4) + 4 (l / 32) + r % 4 (runs of four columns per lane).
    if (KIND == 1) {
        // bf16 tile staged in LDS (8-byte writes), then 16-byte row chunks
        block_sync();                                  // every wave is done with the stages
        uint16_t* ep = (uint16_t*)lds;
#pragma unroll
        for (int i = 0; i < C::kTM; ++i) {
            if (i >= nvi) continue;
            const int row = wm * (BM / WM) + i * 32 + lane % 32;
#pragma unroll
            for (int j = 0; j < C::kTN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int lcol = wn * (BN / WN) + j * 32 + 8 * q + 4 * half;
                    *(uint2*)(ep + row * C::kEpStride + lcol) =
                        make_uint2(pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                                   pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
                }
        }
        __syncthreads();
        constexpr int kChunks = BN / 8;
        uint16_t* out = (uint16_t*)S.out;
        for (int c = tid; c < live * kChunks; c += C::kThreads) {
            const int row = c / kChunks, cc = c % kChunks;
            const uint4 v = *(const uint4*)(ep + row * C::kEpStride + cc * 8);
            *(uint4*)(out + ((size_t)rbase + m0 + row) * N + nt * BN + cc * 8) = v;
        }
        return;
    }
    // GEMM1: act = gate * silu(Z_g) * Z_u, quantised per 1 x 32 block. A block is the 32
    // columns of gate sub-tile jj in one row: lane l holds 16 of them and lane l + 32 the
    // other 16, so its amax takes the lane's own maximum and one exchange. Codes go out as
    // 8-column runs (pair_runs_x2), the row's four block scales of this tile's 128 act columns
    // (one per wave column) as bytes of its scale word.
    constexpr int hf = C::kTN / 2;
    static_assert(hf == 1 && BN / 2 / WN == 32, "one 32-column block per wave and row");
    const int F = N / 2;
    uint8_t* outq = (uint8_t*)S.out;
    uint8_t* outs = (uint8_t*)S.out_scales;
#pragma unroll
    for (int i = 0; i < C::kTM; ++i) {
        if (i >= nvi) continue;
        const int row = wm * (BM / WM) + i * 32 + lane % 32;
        const bool live_row = m0 + row < Mg;           // lanes l and l + 32 share a row
        const int lr = live_row ? row : live - 1;
        const size_t grow = (size_t)rbase + m0 + lr;
        const float gt = S.gate ? S.gate[grow] : 1.0f;
        float v[16];
        float m = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            v[r] = gt * (silu_fast(acc[i][0][r]) * acc[i][hf][r]);
            m = fmaxf(m, fabsf(v[r]));
        }
        m = fmaxf(m, __shfl_xor(m, 32));
        const int X = mx_exponent(m);
        const float inv = exp2_neg(X);
        uint32_t codes[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            codes[q] = e4m3x4(v[4 * q] * inv, v[4 * q + 1] * inv, v[4 * q + 2] * inv,
                              v[4 * q + 3] * inv);
#pragma unroll
        for (int qp = 0; qp < 4; qp += 2) {
            const uint2 w = pair_runs_x2(codes[qp], codes[qp + 1]);
            const int col = nt * (BN / 2) + wn * 32 + 8 * (qp + half);
            if (live_row) *(uint2*)(outq + grow * F + col) = w;
        }
        if (live_row && lane < 32)
            outs[grow * S.so_row + (size_t)nt * S.so_kb + wn] = (uint8_t)(X + 127);
    }
}

// ---------------------------------------------------------------------------------------
// fp32 kernel (FMA): 64 rows x 64 columns per 256-thread block, K in steps of 16.
// GEMM1: the 64 columns are 32 gate + the 32 matching up columns; thread (ty, tx) computes
// rows 4ty..4ty+3 and act columns 2tx, 2tx+1 (gate and up each).
// GEMM2: thread computes rows 4ty..4ty+3 and columns 4tx..4tx+3.
// ---------------------------------------------------------------------------------------
constexpr int kF32BM = 64;
template <int KIND>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs ga) {
    constexpr int BM = 64, BN = 64, BK = 16;
    __shared__ float As[BK][BM + 4];
    __shared__ float Bs[BK][BN + 4];
    int mt, nt;
    if (!pick_tile(ga, mt, nt)) return;
    const int4 ti = ga.tiles[mt];
    const int seg = ti.x >> 20, g = ti.x & 0xFFFFF;
    const int m0 = ti.y, Mg = tile_end(ti.y, ti.z, ga.bm), rbase = ti.w;   // Mg: tile end
    const SegDev S = seg == 0 ? ga.seg[0] : ga.seg[1];
    const int N = ga.N, K = ga.K;
    const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
    const float* A = (const float*)S.a;
    const float* W = (const float*)S.w + (size_t)g * N * K;
    // loader: each thread loads 4 A values and 4 B values per K step
    const int lr = tid / 4, lk = (tid % 4) * 4;          // row 0..63, k 0,4,8,12
    int ar = m0 + lr < Mg ? m0 + lr : Mg - 1;
    const float* a_src = A + (size_t)(rbase + ar) * K + lk;
    int wrow;
    if (KIND == 0)
        wrow = lr < 32 ? nt * 32 + lr : N / 2 + nt * 32 + (lr - 32);
    else
        wrow = nt * BN + lr;
    const float* b_src = W + (size_t)wrow * K + lk;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += BK) {
        float4 av = *(const float4*)(a_src + k0);
        float4 bv = *(const float4*)(b_src + k0);
        As[lk + 0][lr] = av.x; As[lk + 1][lr] = av.y; As[lk + 2][lr] = av.z; As[lk + 3][lr] = av.w;
        Bs[lk + 0][lr] = bv.x; Bs[lk + 1][lr] = bv.y; Bs[lk + 2][lr] = bv.z; Bs[lk + 3][lr] = bv.w;
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
            if (KIND == 0) {
                b[0] = Bs[kk][2 * tx];
                b[1] = Bs[kk][2 * tx + 1];
                b[2] = Bs[kk][32 + 2 * tx];
                b[3] = Bs[kk][32 + 2 * tx + 1];
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
    float* out = (float*)S.out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = ty * 4 + i;
        if (m0 + row >= Mg) continue;
        const size_t grow = (size_t)rbase + m0 + row;
        if (KIND == 0) {
            const int F = N / 2;
            const float gt = S.gate ? S.gate[grow] : 1.0f;
            float* zo = (float*)S.z_out;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int col = nt * 32 + 2 * tx + j;
                const float zg = acc[i][j], zu = acc[i][2 + j];
                out[grow * F + col] = gt * (silu_f32(zg) * zu);
                if (zo) {
                    zo[grow * N + col] = zg;
                    zo[grow * N + F + col] = zu;
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) out[grow * N + nt * BN + tx * 4 + j] = acc[i][j];
        }
    }
}

// ---------------------------------------------------------------------------------------
// configurations
// ---------------------------------------------------------------------------------------
// M tiles of one expert visited together per N tile (see pick_tile).
#ifndef MOE_TILE_MGROUP
#define MOE_TILE_MGROUP 4
#endif

// bf16 tile configurations (BM, BN, BK, WM, WN, A ring depth, B ring depth). GEMM1's BN counts gate + up rows
// (BN / 2 act columns).
#ifndef MOE_BF_UP_CFG
#define MOE_BF_UP_CFG 256, 256, 32, 2, 4, 4, 4
#endif
#ifndef MOE_BF_DOWN_CFG
#define MOE_BF_DOWN_CFG 256, 256, 32, 2, 4, 4, 4
#endif

template <int KIND, int BM, int BN, int BK, int WM, int WN, int SA, int SB>
hipError_t run_bf16(const GemmArgs& ga, int nblocks, hipStream_t s) {
    using C = BfCfg<KIND, BM, BN, BK, WM, WN, SA, SB>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(
            (const void*)gemm_bf16_kernel<KIND, BM, BN, BK, WM, WN, SA, SB>,
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::kLds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    gemm_bf16_kernel<KIND, BM, BN, BK, WM, WN, SA, SB><<<nblocks, C::kThreads, C::kLds, s>>>(ga);
    return hipGetLastError();
}

// Mixed shapes (schedule_mixed_kernel): the 256 x 256 configuration above plus this 128-row one
// (128 x 256 or 128 x 512) for a group's last <= 128 rows, when N is a multiple of its width
#ifndef MOE_BF_MIXED
#define MOE_BF_MIXED 1
#endif
#ifndef MOE_BF_UP_CFG128
#define MOE_BF_UP_CFG128 128, 512, 32, 2, 4, 3, 3
#endif
#ifndef MOE_BF_DOWN_CFG128
#define MOE_BF_DOWN_CFG128 128, 512, 32, 2, 4, 3, 3
#endif

template <int KIND, class C0, class C1>
hipError_t run_bf16_mixed(const GemmArgs& ga, int nblocks, hipStream_t s) {
    constexpr size_t kLds = C0::kLds > C1::kLds ? C0::kLds : C1::kLds;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)gemm_bf16_mixed_kernel<KIND, C0, C1>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    gemm_bf16_mixed_kernel<KIND, C0, C1><<<nblocks, 512, kLds, s>>>(ga);
    return hipGetLastError();
}

template <int BM, int BN, int BK, int WM, int WN, int SA, int SB>
constexpr int cfg_bm() { return BM; }
template <int BM, int BN, int BK, int WM, int WN, int SA, int SB>
constexpr int cfg_bn() { return BN; }

// e4m3 tile configuration (BM, BN, WM, WN, STAGES), both GEMMs
#ifndef MOE_F8_UP_CFG
#define MOE_F8_UP_CFG 256, 256, 2, 4, 2
#endif
#ifndef MOE_F8_DOWN_CFG
#define MOE_F8_DOWN_CFG 256, 256, 2, 4, 2
#endif

template <int KIND, int BM, int BN, int WM, int WN, int STAGES>
hipError_t run_e4m3(const GemmArgs& ga, int nblocks, hipStream_t s) {
    using C = F8Cfg<KIND, BM, BN, WM, WN, STAGES>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(
            (const void*)gemm_e4m3_kernel<KIND, BM, BN, WM, WN, STAGES>,
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::kLds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    gemm_e4m3_kernel<KIND, BM, BN, WM, WN, STAGES><<<nblocks, C::kThreads, C::kLds, s>>>(ga);
    return hipGetLastError();
}

// MXFP8 tile configuration (BM, BN, WM, WN, STAGES, BK), both GEMMs
#ifndef MOE_MX_UP_CFG
#define MOE_MX_UP_CFG 256, 256, 2, 4, 2, 128
#endif
#ifndef MOE_MX_DOWN_CFG
#define MOE_MX_DOWN_CFG 256, 256, 2, 4, 2, 128
#endif

template <int KIND, int BM, int BN, int WM, int WN, int STAGES, int BK>
hipError_t run_mx(const GemmArgs& ga, int nblocks, hipStream_t s) {
    using C = MxCfg<KIND, BM, BN, WM, WN, STAGES, BK>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(
            (const void*)gemm_mx_kernel<KIND, BM, BN, WM, WN, STAGES, BK>,
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::kLds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    gemm_mx_kernel<KIND, BM, BN, WM, WN, STAGES, BK><<<nblocks, C::kThreads, C::kLds, s>>>(ga);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int STAGES, int BK>
constexpr int mx_bm() { return BM; }
template <int BM, int BN, int WM, int WN, int STAGES, int BK>
constexpr int mx_bn() { return BN; }

template <int BM, int BN, int WM, int WN, int STAGES>
constexpr int f8_bm() { return BM; }
template <int BM, int BN, int WM, int WN, int STAGES>
constexpr int f8_bn() { return BN; }

int bm_for(int kind, int dtype) {
    if (dtype == 0) return kF32BM;
    if (dtype == 2) return kind == 0 ? f8_bm<MOE_F8_UP_CFG>() : f8_bm<MOE_F8_DOWN_CFG>();
    if (dtype == 3) return kind == 0 ? mx_bm<MOE_MX_UP_CFG>() : mx_bm<MOE_MX_DOWN_CFG>();
    return kind == 0 ? cfg_bm<MOE_BF_UP_CFG>() : cfg_bm<MOE_BF_DOWN_CFG>();
}
int bn_for(int kind, int dtype) {
    if (dtype == 0) return 64;
    if (dtype == 2) return kind == 0 ? f8_bn<MOE_F8_UP_CFG>() : f8_bn<MOE_F8_DOWN_CFG>();
    if (dtype == 3) return kind == 0 ? mx_bn<MOE_MX_UP_CFG>() : mx_bn<MOE_MX_DOWN_CFG>();
    return kind == 0 ? cfg_bn<MOE_BF_UP_CFG>() : cfg_bn<MOE_BF_DOWN_CFG>();
}

size_t max_mtiles(int max_rows_total, int groups_total, int bm) {
    return (size_t)(max_rows_total + bm - 1) / bm + (size_t)groups_total;
}

// ---------------------------------------------------------------------------------------
// Router scores as a split-K GEMM: logits[t, e] = sum_h x[t, h] w[e, h] (bf16 operands, fp32
// accumulation). One workgroup per (256 tokens, 256 experts, K range); the K ranges are dealt
// round-robin over the XCDs (block b runs on XCD b % 8), so with 8 ranges each XCD streams one
// eighth of the router weight, which stays in its L2, while the tokens' rows are read once.
// Each range writes an fp32 partial tile; the partials are then summed in range order
// (deterministic). Same DMA rings and MFMA loop as the expert GEMMs.
// ---------------------------------------------------------------------------------------
using RouterCfg = BfCfg<1, 256, 256, 64, 2, 4, 2, 2>;

struct RouterArgs {
    const uint8_t* x;   // [T, H] bf16
    const uint8_t* w;   // [E, H] bf16
    float* part;        // [ksplit][T][E]
    int T, H, E, ksplit, ntn;
};

__global__ __launch_bounds__(RouterCfg::kThreads) void router_gemm_kernel(RouterArgs ra) {
    using C = RouterCfg;
    extern __shared__ __align__(16) uint8_t lds[];
    const int b = blockIdx.x;
    const int ks = b % ra.ksplit, rest = b / ra.ksplit;
    const int nt = rest % ra.ntn, mt = rest / ra.ntn;
    const int m0 = mt * 256, n0 = nt * 256;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int wm = wave / 4, wn = wave % 4;
    const int klen = ra.H / ra.ksplit;                       // elements of this K range
    const size_t row_bytes = (size_t)ra.H * 2;
    const size_t kofs = (size_t)ks * klen * 2;

    const uint8_t* srcA[C::kDmaA];
    const uint8_t* srcB[C::kDmaB];
#pragma unroll
    for (int q = 0; q < C::kDmaA; ++q) {
        const int r = C::kRowsPerDma * (wave + q * C::kWaves) + lane / C::kCpr;
        const int c = (lane % C::kCpr) ^ chunk_swz<C::kCpr>(r);
        const int t = m0 + r < ra.T ? m0 + r : ra.T - 1;
        srcA[q] = ra.x + (size_t)t * row_bytes + kofs + c * 16;
    }
#pragma unroll
    for (int q = 0; q < C::kDmaB; ++q) {
        const int r = C::kRowsPerDma * (wave + q * C::kWaves) + lane / C::kCpr;
        const int c = (lane % C::kCpr) ^ chunk_swz<C::kCpr>(r);
        const int e = n0 + r < ra.E ? n0 + r : ra.E - 1;
        srcB[q] = ra.w + (size_t)e * row_bytes + kofs + c * 16;
    }
    auto issue_a = [&](int kstep, int slot) {
        MOE_LDS uint8_t* base = (MOE_LDS uint8_t*)lds + slot * C::kASlot;
#pragma unroll
        for (int q = 0; q < C::kDmaA; ++q)
            __builtin_amdgcn_global_load_lds((const void*)(srcA[q] + (size_t)kstep * 128),
                                             (MOE_LDS void*)(base + (wave + q * C::kWaves) * 1024),
                                             16, 0, 0);
    };
    auto issue_b = [&](int kstep, int slot) {
        MOE_LDS uint8_t* base = (MOE_LDS uint8_t*)lds + C::kBRing + slot * C::kBSlot;
#pragma unroll
        for (int q = 0; q < C::kDmaB; ++q)
            __builtin_amdgcn_global_load_lds((const void*)(srcB[q] + (size_t)kstep * 128),
                                             (MOE_LDS void*)(base + (wave + q * C::kWaves) * 1024),
                                             16, 0, 0);
    };
    int a_off[C::kTM], b_off[C::kTN];
#pragma unroll
    for (int i = 0; i < C::kTM; ++i) a_off[i] = (C::sub_row(wm, i) + lane % 32) * C::kRowBytes;
#pragma unroll
    for (int j = 0; j < C::kTN; ++j) b_off[j] = (wn * 64 + j * 32 + lane % 32) * C::kRowBytes;
    int chunk_off[C::kSub];
#pragma unroll
    for (int s = 0; s < C::kSub; ++s)
        chunk_off[s] = ((2 * s + lane / 32) ^ chunk_swz<C::kCpr>(lane % 32)) * 16;
    f32x16_t acc[C::kTM][C::kTN];
#pragma unroll
    for (int i = 0; i < C::kTM; ++i)
#pragma unroll
        for (int j = 0; j < C::kTN; ++j) acc[i][j] = f32x16_t{};
    bf16_kloop<C, C::kTM, true>(klen / 64, lds, issue_a, issue_b, a_off, b_off, chunk_off, acc);

    // weights as the first MFMA operand: element r of lane l of sub-tile (i, j) is token
    // m0 + sub_row(wm, i) + l % 32 and expert n0 + wn * 64 + 32 j + 8 (r / 4) + 4 (l / 32) + r % 4,
    // so a lane writes four consecutive experts of one token with one 16-byte store (E is a
    // multiple of 4 on this path, router_gemm_ksplit, so a run is all in range or all out)
    float* out = ra.part + (size_t)ks * ra.T * ra.E;
#pragma unroll
    for (int i = 0; i < C::kTM; ++i) {
        const int t = m0 + C::sub_row(wm, i) + lane % 32;
        if (t >= ra.T) continue;
#pragma unroll
        for (int j = 0; j < C::kTN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int e = n0 + wn * 64 + j * 32 + 8 * q + 4 * (lane / 32);
                if (e < ra.E)
                    *(f32x4_t*)(out + (size_t)t * ra.E + e) =
                        f32x4_t{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                acc[i][j][4 * q + 3]};
            }
    }
}

// logits = sum over the K ranges of the partial tiles, in range order.
__global__ __launch_bounds__(256) void router_reduce_kernel(const float* __restrict__ part,
                                                            int64_t n, int ksplit,
                                                            float* __restrict__ logits) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i + 4 <= n) {
        float4 a = *(const float4*)(part + i);
        for (int k = 1; k < ksplit; ++k) {
            const float4 v = *(const float4*)(part + (size_t)k * n + i);
            a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
        }
        *(float4*)(logits + i) = a;
    } else {
        for (int64_t j = i; j < n; ++j) {
            float a = part[j];
            for (int k = 1; k < ksplit; ++k) a += part[(size_t)k * n + j];
            logits[j] = a;
        }
    }
}

}  // namespace

int router_gemm_ksplit(int T, int H, int E, size_t scratch_bytes) {
    if (E < 64 || E % 4 || H % 64) return 0;
    const int steps = H / 64;
    for (int ks = 8; ks >= 2; ks /= 2)
        if (steps % ks == 0 && (size_t)ks * T * E * sizeof(float) <= scratch_bytes) return ks;
    return 1;
}

hipError_t launch_router_gemm(const void* x, const void* w_router, int T, int H, int E,
                              int ksplit, float* part, float* logits, hipStream_t s) {
    using C = RouterCfg;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)router_gemm_kernel,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)C::kLdsLoop);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    RouterArgs ra;
    ra.x = (const uint8_t*)x;
    ra.w = (const uint8_t*)w_router;
    ra.part = ksplit > 1 ? part : logits;
    ra.T = T;
    ra.H = H;
    ra.E = E;
    ra.ksplit = ksplit;
    ra.ntn = (E + 255) / 256;
    const unsigned blocks = (unsigned)((T + 255) / 256) * ra.ntn * ksplit;
    router_gemm_kernel<<<blocks, C::kThreads, C::kLdsLoop, s>>>(ra);
    if (ksplit > 1) {
        const int64_t n = (int64_t)T * E;
        router_reduce_kernel<<<(unsigned)((n / 4 + 255) / 256 + 1), 256, 0, s>>>(part, n,
                                                                               ksplit, logits);
    }
    return hipGetLastError();
}

hipError_t launch_schedule(const int32_t* offsets, int groups, int bm, void* ws, hipStream_t s) {
    SchedArgs sa = {};
    sa.offsets[0] = offsets;
    sa.groups[0] = groups;
    sa.nseg = 1;
    schedule_kernel<<<1, 1024, 0, s>>>(sa, bm, (int4*)((char*)ws + 256), (int*)ws);
    return hipGetLastError();
}

size_t schedule_ws_bytes(int max_rows, int groups, int bm) {
    return 256 + max_mtiles(max_rows, groups, bm) * sizeof(int4);
}

// The mixed bf16 schedule applies when both configurations fit N: 256 x 256 tiles as the
// single-shape configuration, and N a multiple of 512.
template <int BM, int BN, int BK, int WM, int WN, int SA, int SB>
constexpr int cfg_w1() { return BN / 256; }
int bf16_w1(int kind) { return kind == 0 ? cfg_w1<MOE_BF_UP_CFG128>() : cfg_w1<MOE_BF_DOWN_CFG128>(); }

bool bf16_mixed(int kind, int dtype, int N) {
    return MOE_BF_MIXED && dtype == 1 && bm_for(kind, dtype) == 256 &&
           bn_for(kind, dtype) == 256 && N % (256 * bf16_w1(kind)) == 0;
}

// mixed schedule: at most max_mtiles 256-row M tiles of N / 256 units each (a 128-row tile
// has half as many units); the unit table follows the 256-byte header, then the N tiles
size_t mixed_units(int max_rows_total, int groups_total, int N) {
    return max_mtiles(max_rows_total, groups_total, 256) * (size_t)(N / 256);
}

GemmPlan grouped_gemm_plan(int kind, int dtype, int max_rows_total, int groups_total, int N,
                           int K) {
    (void)K;
    GemmPlan p;
    p.bm = bm_for(kind, dtype);
    p.ws_bytes = 256 + max_mtiles(max_rows_total, groups_total, p.bm) * sizeof(int4);
    if (bf16_mixed(kind, dtype, N))
        p.ws_bytes = 256 + mixed_units(max_rows_total, groups_total, N) * (sizeof(int4) + sizeof(int));
    return p;
}

hipError_t launch_grouped_gemm(int kind, int dtype, const Segment* segs, int nseg,
                               int max_rows_total, int N, int K, void* ws, hipStream_t s) {
    const int bm = bm_for(kind, dtype), bn = bn_for(kind, dtype);
    int groups_total = 0;
    SchedArgs sa = {};
    GemmArgs ga = {};
    for (int i = 0; i < nseg; ++i) {
        sa.offsets[i] = segs[i].offsets;
        sa.groups[i] = segs[i].groups;
        sa.rows[i] = segs[i].rows;
        groups_total += segs[i].groups;
        const size_t eb = dtype == 0 ? 4 : dtype == 1 ? 2 : 1;
        const Segment& g = segs[i];
        SegDev d;
        d.a = g.a; d.a_scales = g.a_scales; d.gate = g.gate; d.w = g.w;
        d.w_scales = g.w_scales; d.out = g.out; d.out_scales = g.out_scales; d.z_out = g.z_out;
        d.a_row = g.a_kblock ? 64 : (size_t)K * eb;
        d.a_kstep = g.a_kblock ? (size_t)g.rows_total * 64 : 64;
        d.w_row = g.w_kblock ? 64 : (size_t)K * eb;
        d.w_kstep = g.w_kblock ? (size_t)N * 64 : 64;
        d.w_mat = (size_t)N * K * eb;
        d.rows_total = g.rows_total;
        d.out_kblock = g.out_kblock;
        d.a_rows = g.a_rows;
        if (dtype == 3) {          // MXFP8 scale strides (bytes)
            const uint32_t kbr = (uint32_t)(K / 32), obr = (uint32_t)(N / 2 / 32);
            d.sa_row = g.a_sc_blocked ? 4u : kbr;
            d.sa_kb = g.a_sc_blocked ? (uint32_t)g.a_sc_rows * 4u : 4u;
            d.sw_row = g.w_sc_blocked ? 4u : kbr;
            d.sw_kb = g.w_sc_blocked ? (uint32_t)N * 4u : 4u;
            d.so_row = g.out_sc_blocked ? 4u : obr;
            d.so_kb = g.out_sc_blocked ? (uint32_t)g.rows_total * 4u : 4u;
            d.a_sc_direct = g.a_sc_direct;
        } else {
            d.sa_row = d.sa_kb = d.sw_row = d.sw_kb = d.so_row = d.so_kb = 0;
            d.a_sc_direct = 0;
        }
        ga.seg[i] = d;
    }
    sa.nseg = nseg;
    int* total = (int*)ws;
    int4* tiles = (int4*)((char*)ws + 256);
    if (bf16_mixed(kind, dtype, N)) {
        const size_t nunits = mixed_units(max_rows_total, groups_total, N);
        int* unit_nt = (int*)((char*)ws + 256 + nunits * sizeof(int4));
        schedule_mixed_kernel<<<16, 1024, 0, s>>>(sa, N / 256, bf16_w1(kind), MOE_TILE_MGROUP,
                                                  tiles, unit_nt, total);
        ga.units = tiles;
        ga.unit_nt = unit_nt;
        ga.total = total;
        ga.N = N;
        ga.K = K;
        ga.ntn = N / bn;
        ga.bm = bm;
        ga.mgroup = MOE_TILE_MGROUP;
        const int nblocks = (int)((nunits + 7) / 8 * 8);
        ga.per_xcd_max = nblocks / 8;
        if (kind == 0)
            return run_bf16_mixed<0, BfCfg<0, MOE_BF_UP_CFG>, BfCfg<0, MOE_BF_UP_CFG128>>(
                ga, nblocks, s);
        return run_bf16_mixed<1, BfCfg<1, MOE_BF_DOWN_CFG>, BfCfg<1, MOE_BF_DOWN_CFG128>>(
            ga, nblocks, s);
    }
    schedule_kernel<<<1, 1024, 0, s>>>(sa, bm, tiles, total);
    ga.tiles = tiles;
    ga.total = total;
    ga.N = N;
    ga.K = K;
    ga.ntn = N / bn;
    ga.bm = bm;
    ga.mgroup = MOE_TILE_MGROUP;
    size_t mtiles = max_mtiles(max_rows_total, groups_total, bm);
    size_t nblocks = mtiles * ga.ntn;
    nblocks = (nblocks + 7) / 8 * 8;
    ga.per_xcd_max = (int)(nblocks / 8);
    if (dtype == 0) {
        if (kind == 0) gemm_f32_kernel<0><<<(unsigned)nblocks, 256, 0, s>>>(ga);
        else gemm_f32_kernel<1><<<(unsigned)nblocks, 256, 0, s>>>(ga);
        return hipGetLastError();
    }
    if (dtype == 1) {
        if (kind == 0) return run_bf16<0, MOE_BF_UP_CFG>(ga, (int)nblocks, s);
        return run_bf16<1, MOE_BF_DOWN_CFG>(ga, (int)nblocks, s);
    }
    if (dtype == 2) {
        if (kind == 0) return run_e4m3<0, MOE_F8_UP_CFG>(ga, (int)nblocks, s);
        return run_e4m3<1, MOE_F8_DOWN_CFG>(ga, (int)nblocks, s);
    }
    if (dtype == 3) {
        if (kind == 0) return run_mx<0, MOE_MX_UP_CFG>(ga, (int)nblocks, s);
        return run_mx<1, MOE_MX_DOWN_CFG>(ga, (int)nblocks, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace moe

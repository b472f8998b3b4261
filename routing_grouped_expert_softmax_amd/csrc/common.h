// Device helpers shared by the MoE kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_DEVICE __device__ __forceinline__
#ifndef MOE_FAST_SILU
#define MOE_FAST_SILU 1
#endif

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------------------
// Row split of a ragged group into M tiles. A group of `rows` rows takes
// me = ceil(rows / bm) tiles as always, but the rows are dealt out evenly: every tile but the
// last spans tile_span(rows, bm) rows (a multiple of 32, at most bm). The tiles of a group
// then carry about the same work, so the tiles that read the same weight tile run in step
// and the later readers find it in L2; with a bm-row first tile and a short tail the short
// tile runs far ahead and both stream the weights from HBM. ceil(rows / span) == me always:
// span <= bm gives at least me tiles and span >= rows / me at most me.
__host__ __device__ __forceinline__ int tile_span(int rows, int bm) {
    const int me = (rows + bm - 1) / bm;
    if (me <= 1) return bm;
    const int per = (rows + me - 1) / me;
    return (per + 31) / 32 * 32;
}
// end row (exclusive, within the group) of the tile that starts at row m0
__host__ __device__ __forceinline__ int tile_end(int m0, int rows, int bm) {
    const int e = m0 + tile_span(rows, bm);
    return e < rows ? e : rows;
}

MOE_DEVICE float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (inputs are finite).
MOE_DEVICE uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

MOE_DEVICE uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// ---------------------------------------------------------------------------------------
// OCP E4M3 (e4m3fn): bias 7, largest finite 448, subnormal step 2^-9, no infinities.
// Round to nearest, ties to even, saturating at +-448; the sign of -0.0 is kept.
// e4m3x4 packs the codes of four values into a word (byte i = value i) with gfx950's
// conversion instruction (v_cvt_pk_fp8_f32, two values per instruction, round to nearest
// even) on inputs clamped to [-448, 448] first: unclamped, a value past 448 would not
// saturate. Checked on the device against the bit-level rule above for every finite fp32
// with |x| <= 464: identical codes. Inputs are finite (a NaN would give the code of -448).
// ---------------------------------------------------------------------------------------
MOE_DEVICE float e4m3_clamp(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

MOE_DEVICE uint32_t e4m3x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), w, true);
    return (uint32_t)w;
}

// e4m3 block scale: fp32(amax / 448), 1 for an all-zero block.
MOE_DEVICE float e4m3_scale(float amax) { return amax == 0.0f ? 1.0f : amax / 448.0f; }

// MXFP8 (OCP Microscaling, E4M3 elements, 32-value blocks): the shared exponent of a block
// whose largest magnitude is amax is floor(log2 amax) - 8 (8 being the exponent of E4M3's
// largest normal, 448 = 1.75 * 2^8), clamped to [-127, 127]; zero and fp32-subnormal maxima
// give -127. The block's E8M0 code is X + 127 and its elements the e4m3 codes of v * 2^-X, so the
// largest lands in [256, 512) and only [448, 512) saturates. For finite amax, X <= 119.
MOE_DEVICE int mx_exponent(float amax) {
    const int X = (int)((__float_as_uint(amax) >> 23) & 0xFFu) - 127 - 8;
    return X < -127 ? -127 : X;
}

// 2^-X as fp32 for X in [-127, 119] (an exact power of two: the scaling is exact unless the
// product is an fp32 subnormal, far below E4M3's smallest subnormal)
MOE_DEVICE float exp2_neg(int X) { return __uint_as_float((uint32_t)(127 - X) << 23); }

// ---------------------------------------------------------------------------------------
// Wavefront reductions (deterministic butterflies)
// ---------------------------------------------------------------------------------------
MOE_DEVICE uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint64_t o = __shfl_xor(v, off);
        v = o > v ? o : v;
    }
    return v;
}

MOE_DEVICE float wave_sum_f32(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// Order-preserving map of a finite float to uint32 (-0.0 is mapped like +0.0).
MOE_DEVICE uint32_t float_order_key(float f) {
    f = (f == 0.0f) ? 0.0f : f;
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

MOE_DEVICE float float_from_order_key(uint32_t o) {
    uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
    return __uint_as_float(u);
}

// 64-bit rank key: a larger key wins, and on equal keys the lower index wins.
MOE_DEVICE uint64_t rank_key(float key, int index) {
    return ((uint64_t)float_order_key(key) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)index);
}
MOE_DEVICE int rank_key_index(uint64_t rk) { return (int)(0xFFFFFFFFu - (uint32_t)rk); }
MOE_DEVICE float rank_key_value(uint64_t rk) { return float_from_order_key((uint32_t)(rk >> 32)); }

MOE_DEVICE float silu_f32(float u) { return u / (1.0f + expf(-u)); }

// SiLU for the forward GEMM1 epilogues, written from its definition
// silu(u) = u / (1 + e^-u) with e^-u = 2^(-u log2 e): the hardware exp2 and reciprocal are
// each within about 1 ulp of fp32, far below the bf16 (or e4m3) rounding of the stored
// activation, and take a few instructions instead of a full-precision expf and an IEEE
// division. Large -u gives exp2 = +inf and a result of -0 (the exact value is below bf16's
// smallest normal); large +u gives u.
MOE_DEVICE float silu_fast(float u) {
#if MOE_FAST_SILU
    const float e = __builtin_amdgcn_exp2f(-u * 1.44269504088896340736f);
    return u * __builtin_amdgcn_rcpf(1.0f + e);
#else
    return silu_f32(u);
#endif
}

// ---------------------------------------------------------------------------------------
// Output runs of the transposed 32 x 32 MFMA accumulators: lane l and lane l + 32 hold the
// 4-column runs 8 q + 4 (l / 32) + [0, 4) of the same row. For two consecutive q (x: run q,
// y: run q + 1, packed), v_permlane32_swap trades lane l's y for lane l + 32's x, so lane l
// ends with columns 8 q .. 8 q + 7 and lane l + 32 with 8 q + 8 .. 8 q + 15: twice the bytes
// per store. Every lane of the wave must execute it.
// ---------------------------------------------------------------------------------------
MOE_DEVICE uint4 pair_runs_x4(uint32_t x0, uint32_t x1, uint32_t y0, uint32_t y1) {
    const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
    return make_uint4(s0[0], s1[0], s0[1], s1[1]);
}
MOE_DEVICE uint2 pair_runs_x2(uint32_t x, uint32_t y) {
    const auto s = __builtin_amdgcn_permlane32_swap(x, y, false, false);
    return make_uint2(s[0], s[1]);
}

// ---------------------------------------------------------------------------------------
// LDS pipeline helpers of the MFMA kernels
// ---------------------------------------------------------------------------------------
#define MOE_LDS __attribute__((address_space(3)))

// s_waitcnt with vmcnt <= N, lgkmcnt == 0 (gfx9 encoding; expcnt not waited for).
template <int N>
MOE_DEVICE void wait_vm_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Workgroup barrier without a memory fence: the pipelines order their LDS traffic with
// explicit waits; the empty asm statements keep the compiler from moving memory accesses
// across the barrier.
MOE_DEVICE void block_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

constexpr int cmin(int a, int b) { return a < b ? a : b; }

// Chunk swizzle of a K-contiguous tile row (depends on the row's low 4 bits only, so a
// 32-row operand read sees the same pattern at every 32-row offset). 8 chunks (128-byte
// rows): a ds_read_b128 serves 16 lanes (16 rows) per 256-byte bank line, and two 128-byte
// rows share a line, so rows 0..15 of one logical chunk must land on 16 different 16-byte
// bank groups: (row parity, physical chunk) all distinct. (r & 7) alone gives rows r and r + 8
// the same group, a 2-way conflict that SQ_LDS_BANK_CONFLICT measured at half of the LDS's
// busy cycles; flipping bit 0 on rows 8..15 separates them, and rows 0..7 stay distinct.
// 4 chunks (64-byte rows): rows of one parity among any 4 consecutive even (odd) rows, and
// rows 4 apart, land in different chunks.
template <int CPR>
MOE_DEVICE int chunk_swz(int r) {
    if (CPR == 8) return (r & 7) ^ ((r >> 3) & 1);
    return ((r >> 1) & 3) ^ ((r >> 3) & 1);
}

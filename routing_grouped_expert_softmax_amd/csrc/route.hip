// Router: logits = x W_r^T, and the per-token top-k selection with gates.
//
// Selection is the top-k step of the per-token loop in the study notes
// "Megatron-Core MoE -- 大规模稀疏专家并行实践" (实践案例, 案例 1). It runs one wavefront per token:
// lane l holds the keys of experts l, l+64, l+128, ... and k rounds of a 64-bit wavefront
// max over (order-preserving key, inverted expert index) pick the next expert, so equal keys
// go to the lower index without any arithmetic on the keys. The router logits stay fp32 (the
// study notes warn that low-precision router scores collapse experts, 踩过的坑).
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kRouteWaves = 4;      // tokens per 256-thread block
constexpr int kStatsMaxE = 1024;    // E limit of the ABI

MOE_DEVICE float wave_max_f32(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

// Load-balancing statistics (STATS): the block's sum over its kRouteWaves tokens of the
// router probabilities p[t, :] (each wave's token in LDS, then summed in wave order per
// expert) -> prob_part[block, E]. Tokens past T add zeros.
template <int VPL>
MOE_DEVICE void stats_block_sum(const float (&p)[VPL], bool valid, int E, int lane, int wave,
                                float* __restrict__ prob_part) {
    __shared__ float pl[kRouteWaves][kStatsMaxE];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const int e = v * kWave + lane;
        if (e < E) pl[wave][e] = valid ? p[v] : 0.0f;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kRouteWaves * kWave) {
        float acc = pl[0][e];
#pragma unroll
        for (int w = 1; w < kRouteWaves; ++w) acc += pl[w][e];
        prob_part[(size_t)blockIdx.x * E + e] = acc;
    }
}

// ---------------------------------------------------------------------------------------
// top-k over the keys a wavefront holds; returns, in lane j < k, the j-th expert.
//
// Every expert's 64-bit rank key (order-preserving key, then inverted index) is distinct, so
// the k selected experts are exactly those whose rank key is at least the k-th largest one.
// That threshold is found bit by bit from the top, counting with ballots (no data crosses
// lanes): a candidate bit stays set when at least k keys reach the prefix with it set. Then
// the slot of each selected expert is the number of keys above its own (all of which are
// selected), counted the same way, and the lane of that slot takes the expert. Keys of 0
// mark absent experts; k never exceeds the number of present ones.
// ---------------------------------------------------------------------------------------
template <int VPL>
MOE_DEVICE int count_ge(const uint64_t (&rk)[VPL], uint64_t v) {
    int n = 0;
#pragma unroll
    for (int q = 0; q < VPL; ++q) n += __popcll(__ballot(rk[q] >= v));
    return n;
}

template <int VPL>
MOE_DEVICE int wave_topk(uint64_t (&rk)[VPL], int k, int lane) {
    // the k-th largest key: the largest tau with count(rk >= tau) >= k. The top 32 bits (the
    // order key) first; the index bits only matter when the k-th key ties with others.
    uint64_t tau = 0;
    for (int b = 63; b >= 32; --b) {
        const uint64_t cand = tau | (1ull << b);
        if (count_ge<VPL>(rk, cand) >= k) tau = cand;
    }
    if (count_ge<VPL>(rk, tau) != k) {
        for (int b = 31; b >= 0; --b) {
            const uint64_t cand = tau | (1ull << b);
            if (count_ge<VPL>(rk, cand) >= k) tau = cand;
        }
    }
    int mine = -1;
#pragma unroll
    for (int q = 0; q < VPL; ++q) {
        uint64_t sel = __ballot(rk[q] >= tau && rk[q] != 0);
        while (sel) {
            const int l = __builtin_ctzll(sel);             // wave-uniform
            sel &= sel - 1;
            const uint64_t x =
                ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(rk[q] >> 32), l) << 32) |
                (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)rk[q], l);
            const int slot = count_ge<VPL>(rk, x) - 1;       // keys above x
            if (lane == slot) mine = q * kWave + l;
        }
    }
    return mine;
}

// ---------------------------------------------------------------------------------------
// softmax router: select on l = logit + bias; gates = softmax over the selected logits
// ---------------------------------------------------------------------------------------
// STATS: also the block's part of the mean router probability, p = softmax of l over all E
// experts (fp32: max, exp, wave sum, divide).
template <int VPL, bool STATS>
__global__ __launch_bounds__(256) void route_softmax_kernel(
    const float* __restrict__ logits, const float* __restrict__ logit_bias, int T, int E,
    int k, int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate,
    float* __restrict__ prob_part) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int t = blockIdx.x * kRouteWaves + wave;
    const bool valid = t < T;
    if (!STATS && !valid) return;
    const float* row = logits + (size_t)(valid ? t : 0) * E;
    uint64_t rk[VPL];
    float lv[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        int e = v * kWave + lane;
        rk[v] = 0;
        lv[v] = -INFINITY;
        if (e < E) {
            float l = row[e];
            if (logit_bias) l = l + logit_bias[e];
            rk[v] = rank_key(l, e);
            lv[v] = l;
        }
    }
    if (STATS) {
        float m = lv[0];
#pragma unroll
        for (int v = 1; v < VPL; ++v) m = fmaxf(m, lv[v]);
        m = wave_max_f32(m);
        float p[VPL], den = 0.0f;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            p[v] = v * kWave + lane < E ? expf(lv[v] - m) : 0.0f;
            den += p[v];
        }
        den = wave_sum_f32(den);
#pragma unroll
        for (int v = 0; v < VPL; ++v) p[v] = p[v] / den;
        stats_block_sum<VPL>(p, valid, E, lane, wave, prob_part);
        if (!valid) return;
    }
    int e = wave_topk<VPL>(rk, k, lane);
    float l = 0.0f;
    if (lane < k) {
        l = row[e];
        if (logit_bias) l = l + logit_bias[e];
    }
    float l0 = __shfl(l, 0);
    float num = lane < k ? expf(l - l0) : 0.0f;
    float den = wave_sum_f32(num);
    if (lane < k) {
        topk_idx[(size_t)t * k + lane] = e;
        topk_gate[(size_t)t * k + lane] = num / den;
    }
}

// s = fp32(1 / (1 + exp(-l))), evaluated in double and rounded once.
MOE_DEVICE float sigmoid_rounded(float l) {
    return (float)(1.0 / (1.0 + exp(-(double)l)));
}

// ---------------------------------------------------------------------------------------
// sigmoid + group-limited router (DeepSeek-V3 style)
// ---------------------------------------------------------------------------------------
// STATS: also the block's part of the mean router probability, p = s / sum_e s over all E
// experts (s = the sigmoid score without the selection bias; fp32 wave sum, divide).
template <int VPL, bool STATS>
__global__ __launch_bounds__(256) void route_sigmoid_group_kernel(
    const float* __restrict__ logits, const float* __restrict__ logit_bias,
    const float* __restrict__ sel_bias, int T, int E, int k, int n_groups, int topk_groups,
    float route_scale, int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate,
    float* __restrict__ prob_part) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int t = blockIdx.x * kRouteWaves + wave;
    const bool valid = t < T;
    if (!STATS && !valid) return;
    const float* row = logits + (size_t)(valid ? t : 0) * E;
    const int per = E / n_groups;
    float key[VPL], sv[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        int e = v * kWave + lane;
        key[v] = 0.0f;
        sv[v] = 0.0f;
        if (e < E) {
            float l = row[e];
            if (logit_bias) l = l + logit_bias[e];
            float s = sigmoid_rounded(l);
            sv[v] = s;
            key[v] = sel_bias ? s + sel_bias[e] : s;
        }
    }
    if (STATS) {
        float den = 0.0f;
#pragma unroll
        for (int v = 0; v < VPL; ++v) den += sv[v];
        den = wave_sum_f32(den);
        float p[VPL];
#pragma unroll
        for (int v = 0; v < VPL; ++v) p[v] = sv[v] / den;
        stats_block_sum<VPL>(p, valid, E, lane, wave, prob_part);
        if (!valid) return;
    }
    uint64_t kept_mask;           // bit g: group g is kept (the same in every lane)
    if (per == 32 && E == VPL * kWave) {
        // groups are the 32-lane halves of the key registers (group 2 v + lane / 32 in v).
        // A group's score needs only the values of its two largest keys: the largest order
        // key m1 (a butterfly of 32-bit maxima inside each half), and m1 again when it occurs
        // twice in the group, else the largest of the others (a second butterfly).
        uint64_t gk[VPL];
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            const uint32_t ok = float_order_key(key[v]);
            uint32_t m1 = ok;
#pragma unroll
            for (int off = 1; off < 32; off <<= 1) m1 = max(m1, (uint32_t)__shfl_xor((int)m1, off));
            const uint64_t eq = __ballot(ok == m1);
            const int twice = __popc(lane < 32 ? (uint32_t)eq : (uint32_t)(eq >> 32)) >= 2;
            uint32_t m2 = ok == m1 ? 0u : ok;
#pragma unroll
            for (int off = 1; off < 32; off <<= 1) m2 = max(m2, (uint32_t)__shfl_xor((int)m2, off));
            if (twice) m2 = m1;
            gk[v] = rank_key(float_from_order_key(m1) + float_from_order_key(m2),
                             2 * v + lane / 32);
        }
        // group g's key sits in register g / 2 of lane 32 (g % 2). Lane l ranks group l % 8:
        // it is kept when fewer than topk_groups groups rank above it (score desc, then
        // group asc)
        uint64_t gkey[2 * VPL];
#pragma unroll
        for (int g = 0; g < 2 * VPL; ++g) {
            const uint64_t x = gk[g / 2];
            const int src = (g % 2) * 32;
            gkey[g] = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(x >> 32), src) << 32) |
                      (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, src);
        }
        const int myg = lane % (2 * VPL);
        uint64_t mine = gkey[0];
#pragma unroll
        for (int g = 1; g < 2 * VPL; ++g) mine = myg == g ? gkey[g] : mine;
        int above = 0;
#pragma unroll
        for (int h = 0; h < 2 * VPL; ++h) above += gkey[h] > mine;
        kept_mask = __ballot(lane < 2 * VPL && above < topk_groups);
    } else {
    // group score = sum of the two largest keys of the group; lane g keeps group g's score
    uint64_t my_group_rk = 0;
    for (int g = 0; g < n_groups; ++g) {
        uint64_t rk[VPL];
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            int e = v * kWave + lane;
            rk[v] = (e < E && e / per == g) ? rank_key(key[v], e) : 0;
        }
        uint64_t b1 = 0;
#pragma unroll
        for (int v = 0; v < VPL; ++v) b1 = rk[v] > b1 ? rk[v] : b1;
        b1 = wave_max_u64(b1);
        uint64_t b2 = 0;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            uint64_t r = rk[v] == b1 ? 0 : rk[v];
            b2 = r > b2 ? r : b2;
        }
        b2 = wave_max_u64(b2);
        float score = rank_key_value(b1) + rank_key_value(b2);
        if (lane == g) my_group_rk = rank_key(score, g);
    }
    // keep the topk_groups best groups; lane g learns whether group g is kept
    int kept = 0;
    for (int i = 0; i < topk_groups; ++i) {
        uint64_t best = wave_max_u64(my_group_rk);
        if (lane == rank_key_index(best)) {
            kept = 1;
            my_group_rk = 0;
        }
    }
    kept_mask = __ballot(kept);
    }
    uint64_t rk[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        int e = v * kWave + lane;
        int g = (e < E ? e : 0) / per;
        const bool keep = (kept_mask >> g) & 1u;
        rk[v] = (e < E && keep) ? rank_key(key[v], e) : 0;
    }
    int e = wave_topk<VPL>(rk, k, lane);
    float s = 0.0f;
    if (lane < k) {
        float l = row[e];
        if (logit_bias) l = l + logit_bias[e];
        s = sigmoid_rounded(l);
    }
    float den = wave_sum_f32(s);
    if (lane < k) {
        topk_idx[(size_t)t * k + lane] = e;
        topk_gate[(size_t)t * k + lane] = route_scale * s / den;
    }
}

// ---------------------------------------------------------------------------------------
// router GEMM, fp32 operands: logits[t, e] = sum_h x[t, h] w[e, h] (fp32 FMA)
// One wavefront per token row; lanes stride over h, each lane keeps E partial sums in
// chunks of 8 experts, reduced across the wavefront.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_logits_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ w, int T, int H, int E,
    float* __restrict__ logits) {
    const int lane = threadIdx.x % kWave;
    const int t = blockIdx.x * 4 + threadIdx.x / kWave;
    if (t >= T) return;
    const float* xr = x + (size_t)t * H;
    for (int e0 = 0; e0 < E; e0 += 8) {
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int h = lane; h < H; h += kWave) {
            float xv = xr[h];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (e0 + i < E) acc[i] = fmaf(xv, w[(size_t)(e0 + i) * H + h], acc[i]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float v = wave_sum_f32(acc[i]);
            if (lane == 0 && e0 + i < E) logits[(size_t)t * E + e0 + i] = v;
        }
    }
}

// ---------------------------------------------------------------------------------------
// router GEMM, bf16 operands on MFMA 16x16x32 (fp32 accumulate).
// Block: 64 tokens x 64 experts, 4 x S waves: wave (tg, kq) owns tokens [16 tg, 16 tg + 16)
// x all 64 experts (4 MFMA column tiles) over the K range kq * H / S .. (kq + 1) * H / S.
// The S partial tiles are summed through LDS in a fixed order (deterministic). Operands are
// read straight from global memory (K contiguous, 16 B per lane): x is read once per
// 64-expert column block and w (E x H, a few MB) stays in L2; each step issues the loads of
// kRouterU K chunks before their MFMAs. Splitting K raises the waves per CU (latency hiding)
// without adding traffic.
// ---------------------------------------------------------------------------------------
constexpr int kRouterU = 8;      // 32-wide K chunks per load batch

template <int S>
__global__ __launch_bounds__(256 * S) void router_logits_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int T, int H, int E,
    float* __restrict__ logits) {
    __shared__ float red[(S > 1 ? S - 1 : 1) * 4 * 64 * 16];
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int tg = wave % 4, kq = wave / 4;
    const int t0 = blockIdx.x * 64 + tg * 16;
    const int e_base = blockIdx.y * 64;
    int tr = t0 + (lane % 16);
    tr = tr < T ? tr : T - 1;
    const uint16_t* xa = x + (size_t)tr * H + 8 * (lane / 16);
    const uint16_t* wb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        int er = e_base + 16 * j + (lane % 16);
        er = er < E ? er : E - 1;
        wb[j] = w + (size_t)er * H + 8 * (lane / 16);
    }
    f32x4_t acc[4] = {};
    const int hq = H / S;
    for (int h = kq * hq; h < (kq + 1) * hq; h += 32 * kRouterU) {
        bf16x8_t a[kRouterU], b[kRouterU][4];
#pragma unroll
        for (int u = 0; u < kRouterU; ++u) {
            a[u] = *(const bf16x8_t*)(xa + h + 32 * u);
#pragma unroll
            for (int j = 0; j < 4; ++j) b[u][j] = *(const bf16x8_t*)(wb[j] + h + 32 * u);
        }
#pragma unroll
        for (int u = 0; u < kRouterU; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b[u][j], acc[j], 0, 0, 0);
    }
    if (S > 1) {
        if (kq > 0) {
            float* dst = red + (((kq - 1) * 4 + tg) * 64 + lane) * 16;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[j * 4 + i] = acc[j][i];
        }
        __syncthreads();
        if (kq > 0) return;
#pragma unroll
        for (int q = 1; q < S; ++q) {
            const float* p = red + (((q - 1) * 4 + tg) * 64 + lane) * 16;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[j][i] += p[j * 4 + i];
        }
    }
    // 16x16 output: lane holds rows 4*(lane/16)+i, column lane%16
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        int e = e_base + 16 * j + (lane % 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int t = t0 + 4 * (lane / 16) + i;
            if (t < T && e < E) logits[(size_t)t * E + e] = acc[j][i];
        }
    }
}

// ---------------------------------------------------------------------------------------
// Backward of the gates to the logits (one wavefront per token). The expert choice carries
// no gradient; lane j < k holds slot j. With dg_j = dL/dg_j:
//   softmax: dl_j = g_j (dg_j - sum_i g_i dg_i)
//   sigmoid: s_j = sigmoid(l_j + bias), S = sum_i s_i, g_j = c s_j / S,
//            dl_j = (c / S) (dg_j - sum_i dg_i g_i / c) s_j (1 - s_j)
// Unselected experts get 0. dl is written in bf16 (the router GEMMs' operand) and, when
// asked, in fp32.
// ---------------------------------------------------------------------------------------
template <int VPL>
__global__ __launch_bounds__(256) void route_backward_kernel(
    const float* __restrict__ logits, const float* __restrict__ logit_bias,
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_gate,
    const float* __restrict__ dgate_perm, const int32_t* __restrict__ pos, int T, int E,
    int k, int router, float route_scale, uint16_t* __restrict__ dl_bf16,
    float* __restrict__ dl_f32) {
    const int lane = threadIdx.x % kWave;
    const int t = blockIdx.x * kRouteWaves + threadIdx.x / kWave;
    if (t >= T) return;
    const bool mine = lane < k;
    const int e = mine ? topk_idx[(size_t)t * k + lane] : 0;
    const float g = mine ? topk_gate[(size_t)t * k + lane] : 0.0f;
    const float dg = mine ? dgate_perm[pos[(size_t)t * k + lane]] : 0.0f;
    const float dot = wave_sum_f32(g * dg);
    float dl = 0.0f;
    if (router == 0) {
        dl = g * (dg - dot);
    } else {
        float sv = 0.0f;
        if (mine) {
            const float l = logits[(size_t)t * E + e] + (logit_bias ? logit_bias[e] : 0.0f);
            sv = sigmoid_rounded(l);
        }
        const float ssum = wave_sum_f32(sv);
        dl = (route_scale / ssum) * (dg - dot / route_scale) * sv * (1.0f - sv);
    }
    // row t: every expert column, 0 unless selected (k <= 32 distinct experts)
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const int c = v * kWave + lane;
        float val = 0.0f;
        for (int j = 0; j < k; ++j) {
            const int ej = __shfl(e, j);
            const float dj = __shfl(dl, j);
            if (ej == c) val = dj;
        }
        if (c < E) {
            dl_bf16[(size_t)t * E + c] = f32_to_bf16(val);
            if (dl_f32) dl_f32[(size_t)t * E + c] = val;
        }
    }
}

}  // namespace

hipError_t launch_router_logits(int act_dtype, const void* x, const void* w_router, int T,
                                int H, int E, float* logits, hipStream_t s) {
    if (act_dtype == 0) {
        router_logits_f32_kernel<<<(T + 3) / 4, 256, 0, s>>>((const float*)x,
                                                             (const float*)w_router, T, H, E,
                                                             logits);
    } else {
        dim3 grid((T + 63) / 64, (E + 63) / 64);
        const uint16_t* xb = (const uint16_t*)x;
        const uint16_t* wb = (const uint16_t*)w_router;
        if (H % (4 * 32 * kRouterU) == 0)
            router_logits_bf16_kernel<4><<<grid, 1024, 0, s>>>(xb, wb, T, H, E, logits);
        else if (H % (2 * 32 * kRouterU) == 0)
            router_logits_bf16_kernel<2><<<grid, 512, 0, s>>>(xb, wb, T, H, E, logits);
        else
            router_logits_bf16_kernel<1><<<grid, 256, 0, s>>>(xb, wb, T, H, E, logits);
    }
    return hipGetLastError();
}

template <int VPL>
static void route_launch(int router, const float* logits, const float* logit_bias,
                         const float* sel_bias, int T, int E, int k, int n_groups,
                         int topk_groups, float route_scale, int32_t* topk_idx,
                         float* topk_gate, float* prob_part, hipStream_t s) {
    int blocks = (T + kRouteWaves - 1) / kRouteWaves;
    if (router == 0) {
        if (prob_part)
            route_softmax_kernel<VPL, true><<<blocks, 256, 0, s>>>(logits, logit_bias, T, E, k,
                                                                   topk_idx, topk_gate, prob_part);
        else
            route_softmax_kernel<VPL, false><<<blocks, 256, 0, s>>>(logits, logit_bias, T, E, k,
                                                                    topk_idx, topk_gate, nullptr);
    } else {
        if (prob_part)
            route_sigmoid_group_kernel<VPL, true><<<blocks, 256, 0, s>>>(
                logits, logit_bias, sel_bias, T, E, k, n_groups, topk_groups, route_scale,
                topk_idx, topk_gate, prob_part);
        else
            route_sigmoid_group_kernel<VPL, false><<<blocks, 256, 0, s>>>(
                logits, logit_bias, sel_bias, T, E, k, n_groups, topk_groups, route_scale,
                topk_idx, topk_gate, nullptr);
    }
}

// Deterministic column sums: out[blockIdx.y, c] = scale * sum of rows
// [blockIdx.y * rpb, min((blockIdx.y + 1) * rpb, R)) of in[R, C], added in row order.
__global__ __launch_bounds__(256) void colsum_kernel(const float* __restrict__ in, int R, int C,
                                                     int rpb, float inv,
                                                     float* __restrict__ out) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= C) return;
    const int r0 = blockIdx.y * rpb;
    const int r1 = r0 + rpb < R ? r0 + rpb : R;
    float acc = 0.0f;
    int r = r0;
    for (; r + 8 <= r1; r += 8) {      // eight loads in flight, then the adds in row order
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = in[(size_t)(r + u) * C + c];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += v[u];
    }
    for (; r < r1; ++r) acc += in[(size_t)r * C + c];
    out[(size_t)blockIdx.y * C + c] = acc * inv;
}

constexpr int kStatsRpb = 16;       // first-level rows per column-sum block

hipError_t route_dispatch(int router, const float* logits, const float* logit_bias,
                          const float* sel_bias, int T, int E, int k, int n_groups,
                          int topk_groups, float route_scale, int32_t* topk_idx,
                          float* topk_gate, float* prob_part, hipStream_t s) {
    int vpl = (E + kWave - 1) / kWave;
#define MOE_ROUTE_CASE(V)                                                                   \
    if (vpl <= V) {                                                                         \
        route_launch<V>(router, logits, logit_bias, sel_bias, T, E, k, n_groups,            \
                        topk_groups, route_scale, topk_idx, topk_gate, prob_part, s);       \
        return hipGetLastError();                                                           \
    }
    MOE_ROUTE_CASE(1)
    MOE_ROUTE_CASE(2)
    MOE_ROUTE_CASE(4)
    MOE_ROUTE_CASE(8)
    MOE_ROUTE_CASE(16)
#undef MOE_ROUTE_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_route(int router, const float* logits, const float* logit_bias,
                        const float* sel_bias, int T, int E, int k, int n_groups,
                        int topk_groups, float route_scale, int32_t* topk_idx,
                        float* topk_gate, hipStream_t s) {
    return route_dispatch(router, logits, logit_bias, sel_bias, T, E, k, n_groups, topk_groups,
                          route_scale, topk_idx, topk_gate, nullptr, s);
}

size_t route_stats_ws_bytes(int T, int E) {
    const size_t R = (size_t)(T + kRouteWaves - 1) / kRouteWaves;
    const size_t R2 = (R + kStatsRpb - 1) / kStatsRpb;
    return ((R + R2) * (size_t)E * sizeof(float) + 255) / 256 * 256;
}

hipError_t launch_route_stats(int router, const float* logits, const float* logit_bias,
                              const float* sel_bias, int T, int E, int k, int n_groups,
                              int topk_groups, float route_scale, int32_t* topk_idx,
                              float* topk_gate, float* prob_mean, void* ws, hipStream_t s) {
    const int R = (T + kRouteWaves - 1) / kRouteWaves;
    const int R2 = (R + kStatsRpb - 1) / kStatsRpb;
    float* part = (float*)ws;
    float* part2 = part + (size_t)R * E;
    hipError_t e = route_dispatch(router, logits, logit_bias, sel_bias, T, E, k, n_groups,
                                  topk_groups, route_scale, topk_idx, topk_gate, part, s);
    if (e != hipSuccess) return e;
    const unsigned cb = (unsigned)((E + 255) / 256);
    colsum_kernel<<<dim3(cb, (unsigned)R2), 256, 0, s>>>(part, R, E, kStatsRpb, 1.0f, part2);
    colsum_kernel<<<dim3(cb, 1), 256, 0, s>>>(part2, R2, E, R2, 1.0f / (float)T, prob_mean);
    return hipGetLastError();
}

}  // namespace moe

namespace moe {

hipError_t launch_route_backward(int router, const float* logits, const float* logit_bias,
                                 const int32_t* topk_idx, const float* topk_gate,
                                 const float* dgate_perm, const int32_t* pos, int T, int E,
                                 int k, float route_scale, uint16_t* dl_bf16, float* dl_f32,
                                 hipStream_t s) {
    const int blocks = (T + kRouteWaves - 1) / kRouteWaves;
    const int vpl = (E + kWave - 1) / kWave;
#define MOE_RB_CASE(V)                                                                      \
    if (vpl <= V) {                                                                         \
        route_backward_kernel<V><<<blocks, 256, 0, s>>>(logits, logit_bias, topk_idx,      \
                                                        topk_gate, dgate_perm, pos, T, E,  \
                                                        k, router, route_scale, dl_bf16,   \
                                                        dl_f32);                           \
        return hipGetLastError();                                                           \
    }
    MOE_RB_CASE(1)
    MOE_RB_CASE(2)
    MOE_RB_CASE(4)
    MOE_RB_CASE(8)
    MOE_RB_CASE(16)
#undef MOE_RB_CASE
    return hipErrorInvalidValue;
}

}  // namespace moe

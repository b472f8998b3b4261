/*
 * moe_oracle.c -- plain, slow CPU oracle for one token-choice Mixture-of-Experts layer.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the bench's CPU-baseline
 * leg may load this library. It shares no code, header, table or constant with the GPU
 * library, and it never sees a value the GPU library produced.
 *
 * What it computes follows the per-token loop of the study notes
 * "Megatron-Core MoE -- 大规模稀疏专家并行实践" (case 1, 实践案例 / 案例 1): score every
 * expert with the router, keep the top-k experts, and add gate(e) * Expert_e(x) for each
 * kept expert. Everything is accumulated in double precision from the exact input values
 * (fp32, bf16 and e4m3 values are all exact in double); a result is rounded only where a
 * stored fp32 value is part of the definition (logits, routing keys, gates, fp8 scales).
 *
 * Readings where the pages are silent (the router form, softmax renormalisation, the
 * sigmoid + group-limited router, tie-breaking, SwiGLU, the shared expert, e4m3 block
 * quantisation) are stated at each function.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no fast-math).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_E4M3 = 2, ORC_MXFP8 = 3 };
enum { ORC_SOFTMAX_TOPK = 0, ORC_SIGMOID_GROUP_TOPK = 1 };

/* ------------------------------------------------------------------------------------ */
/* Number formats                                                                       */
/* ------------------------------------------------------------------------------------ */

static double bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;           /* bf16 is the top half of an fp32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, no
 * infinities, S.1111.111 is NaN, largest finite magnitude 448, subnormal step 2^-9.
 * FP8 E4M3 is the format the pages name for low-precision expert GEMMs
 * ("万亿参数MoE模型训练的技术挑战", section 2.1). */
double orc_e4m3_value(uint8_t code) {
    int sign = code >> 7, ex = (code >> 3) & 15, man = code & 7;
    double mag;
    if (ex == 15 && man == 7) return NAN;
    if (ex == 0) mag = ldexp((double)man, -9);            /* (man/8) * 2^(1-7) */
    else mag = ldexp(1.0 + man / 8.0, ex - 7);
    return sign ? -mag : mag;
}

static double g_e4m3_mag[127];   /* magnitudes of codes 0..126, strictly increasing */
static double g_e4m3_val[256];
static double g_e8m0_val[256];        /* E8M0 scale code S -> 2^(S - 127) */
static int g_tables_ready = 0;

static void init_tables(void) {
    if (g_tables_ready) return;
    for (int c = 0; c < 256; ++c) g_e4m3_val[c] = orc_e4m3_value((uint8_t)c);
    for (int c = 0; c < 256; ++c) g_e8m0_val[c] = ldexp(1.0, c - 127);
    for (int c = 0; c < 127; ++c) g_e4m3_mag[c] = orc_e4m3_value((uint8_t)c);
    g_tables_ready = 1;
}

/* Round v to the nearest e4m3 value; a tie goes to the even code (even mantissa);
 * magnitudes at or above 448 saturate to 448. The sign of v (also of -0.0) is kept. */
uint8_t orc_e4m3_encode(float v) {
    init_tables();
    double a = fabs((double)v);
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    int c;
    if (a >= 448.0) {
        c = 126;
    } else {
        /* largest c with mag[c] <= a */
        int lo = 0, hi = 126;
        while (lo < hi) {
            int mid = (lo + hi + 1) / 2;
            if (g_e4m3_mag[mid] <= a) lo = mid; else hi = mid - 1;
        }
        c = lo;
        double below = a - g_e4m3_mag[c], above = g_e4m3_mag[c + 1] - a;
        if (above < below || (above == below && ((c + 1) % 2) == 0)) c = c + 1;
    }
    return (uint8_t)(sign | c);
}

/* Block scale of one quantisation block: fp32(amax / 448), and 1 for an all-zero block. */
static float block_scale(double amax) {
    if (amax == 0.0) return 1.0f;
    return (float)amax / 448.0f;
}

static double load(const void* p, int dtype, int64_t i) {
    switch (dtype) {
    case ORC_F32: return (double)((const float*)p)[i];
    case ORC_BF16: return bf16_value(((const uint16_t*)p)[i]);
    default: return NAN;
    }
}

/* Quantise rows of an fp32/bf16 matrix [rows, cols] to e4m3 with one fp32 scale per
 * 1 x 128 block along the row: s = fp32(amax/448), q = e4m3(fp32(v / s)). */
void orc_quant_rows(const void* v, int dtype, int64_t rows, int cols, uint8_t* q, float* s) {
    init_tables();
    int nb = cols / 128;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int b = 0; b < nb; ++b) {
            double amax = 0.0;
            for (int c = b * 128; c < b * 128 + 128; ++c) {
                double a = fabs(load(v, dtype, r * cols + c));
                if (a > amax) amax = a;
            }
            float sc = block_scale(amax);
            s[r * nb + b] = sc;
            for (int c = b * 128; c < b * 128 + 128; ++c) {
                float val = (float)load(v, dtype, r * cols + c);
                q[r * cols + c] = orc_e4m3_encode(val / sc);
            }
        }
    }
}

/* MX block quantisation: the MXFP8 format of the OCP Microscaling specification with E4M3
 * elements (named on the pages as MXFP8), one block per 32 consecutive values of a row.
 * Shared exponent X = floor(log2(amax)) - 8 (8: the exponent of E4M3's largest normal,
 * 448 = 1.75 * 2^8), clamped to [-127, 127] and stored as the E8M0 code X + 127; elements
 * q = e4m3(v / 2^X), nearest even, saturating at 448 (a block's largest value lands in
 * [256, 512), so only values of [448, 512) saturate). An all-zero block has X = -127. */
static int mx_exponent(double amax) {
    int X = -127;
    if (amax > 0.0) {
        int e;
        frexp(amax, &e);                      /* amax = m 2^e, m in [0.5, 1) */
        X = e - 1 - 8;
        if (X < -127) X = -127;
        if (X > 127) X = 127;
    }
    return X;
}

void orc_mx_quant(const void* v, int dtype, int64_t rows, int cols, uint8_t* q, uint8_t* s) {
    init_tables();
    int nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int b = 0; b < nb; ++b) {
            double amax = 0.0;
            for (int c = b * 32; c < b * 32 + 32; ++c) {
                double a = fabs(load(v, dtype, r * cols + c));
                if (a > amax) amax = a;
            }
            int X = mx_exponent(amax);
            s[r * nb + b] = (uint8_t)(X + 127);
            for (int c = b * 32; c < b * 32 + 32; ++c)
                q[r * cols + c] = orc_e4m3_encode((float)ldexp(load(v, dtype, r * cols + c), -X));
        }
    }
}

/* Quantise nmat matrices [rows, cols] to e4m3 with one fp32 scale per 128 x 128 block;
 * scales are laid out [nmat, rows/128, cols/128]. */
void orc_quant_weight(const void* w, int dtype, int64_t nmat, int rows, int cols,
                      uint8_t* q, float* s) {
    init_tables();
    int nbr = rows / 128, nbc = cols / 128;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t m = 0; m < nmat; ++m) {
        for (int br = 0; br < nbr; ++br) {
            for (int bc = 0; bc < nbc; ++bc) {
                double amax = 0.0;
                for (int r = br * 128; r < br * 128 + 128; ++r)
                    for (int c = bc * 128; c < bc * 128 + 128; ++c) {
                        double a = fabs(load(w, dtype, (m * rows + r) * (int64_t)cols + c));
                        if (a > amax) amax = a;
                    }
                float sc = block_scale(amax);
                s[(m * nbr + br) * nbc + bc] = sc;
                for (int r = br * 128; r < br * 128 + 128; ++r)
                    for (int c = bc * 128; c < bc * 128 + 128; ++c) {
                        int64_t i = (m * rows + r) * (int64_t)cols + c;
                        q[i] = orc_e4m3_encode((float)load(w, dtype, i) / sc);
                    }
            }
        }
    }
}

/* Value of element (r, c) of matrix m of a stacked weight [nmat, rows, cols]. For e4m3 the
 * value is the code's value times its 128 x 128 block scale (fp32, [nmat, rows/128,
 * cols/128]); for MXFP8, times 2^(S - 127) with S the E8M0 code of its 1 x 32 block along
 * the row ([nmat, rows, cols/32] bytes). */
typedef struct {
    const void* p;
    int dtype;
    const void* scales;
    int rows, cols;
} wmat;

static inline double wval(const wmat* w, int64_t m, int r, int c) {
    int64_t i = ((int64_t)m * w->rows + r) * (int64_t)w->cols + c;
    if (w->dtype == ORC_E4M3) {
        int nbr = w->rows / 128, nbc = w->cols / 128;
        double sc = ((const float*)w->scales)[((int64_t)m * nbr + r / 128) * nbc + c / 128];
        return g_e4m3_val[((const uint8_t*)w->p)[i]] * sc;
    }
    if (w->dtype == ORC_MXFP8) {
        uint8_t e8 = ((const uint8_t*)w->scales)[((int64_t)m * w->rows + r) * (w->cols / 32) + c / 32];
        return g_e4m3_val[((const uint8_t*)w->p)[i]] * g_e8m0_val[e8];
    }
    return load(w->p, w->dtype, i);
}

/* fp8 "quantise then dequantise" of one row of n values given as fp32, 1 x 128 blocks. */
static void fake_quant_row(const float* v, int n, double* out) {
    for (int b = 0; b < n / 128; ++b) {
        double amax = 0.0;
        for (int c = b * 128; c < b * 128 + 128; ++c)
            if (fabs((double)v[c]) > amax) amax = fabs((double)v[c]);
        float sc = block_scale(amax);
        for (int c = b * 128; c < b * 128 + 128; ++c)
            out[c] = g_e4m3_val[orc_e4m3_encode(v[c] / sc)] * (double)sc;
    }
}

/* ------------------------------------------------------------------------------------ */
/* Router scores: the scoring step of the per-token loop (study notes, 实践案例 案例 1)     */
/* ------------------------------------------------------------------------------------ */

/* logits[t, e] = fp32( sum_h x[t,h] * w_router[e,h] ), a linear router without bias
 * (the pages name the router only; the linear form is the plainest reading). */
void orc_router_logits(const void* x, const void* wr, int dtype, int T, int H, int E,
                       float* logits) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h)
                acc += load(x, dtype, (int64_t)t * H + h) * load(wr, dtype, (int64_t)e * H + h);
            logits[(int64_t)t * E + e] = (float)acc;
        }
    }
}

/* ------------------------------------------------------------------------------------ */
/* Top-k selection and gates: the selection step of that loop (案例 1)                  */
/* ------------------------------------------------------------------------------------ */

/* a ranks before b when its key is larger, or when the keys are equal and its index is
 * lower. -0.0 and +0.0 compare equal, so they tie. */
static int ranks_before(float key_a, int a, float key_b, int b) {
    if (key_a > key_b) return 1;
    if (key_a < key_b) return 0;
    return a < b;
}

/* Pick the k best entries of key[0..n) (skipping entries with allowed[i] == 0) in rank
 * order: repeated selection of the best remaining entry. */
static void select_topk(const float* key, const int* allowed, int n, int k, int* out) {
    char taken[4096];
    memset(taken, 0, (size_t)n);
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int i = 0; i < n; ++i) {
            if (taken[i] || (allowed && !allowed[i])) continue;
            if (best < 0 || ranks_before(key[i], i, key[best], best)) best = i;
        }
        out[j] = best;
        taken[best] = 1;
    }
}

/* Routing of every token.
 *   l[e] = fp32(logits[t,e] + logit_bias[e])           (logit_bias may be NULL)
 * Softmax router: keys are l; gates are the softmax over the k kept logits,
 *   g_j = exp(l[S_j] - l[S_0]) / sum_i exp(l[S_i] - l[S_0]),
 *   which equals the full softmax renormalised over the kept set.
 * Sigmoid group router:
 *   s[e] = fp32(1 / (1 + exp(-l[e]))) evaluated in double, key[e] = fp32(s[e] + sel_bias[e]);
 *   group score = fp32(sum of the two largest keys among the E/G contiguous experts of
 *   the group); keep the topk_groups best groups (score desc, group index asc); then the k
 *   best experts of the kept groups by key; g_j = route_scale * s[S_j] / sum_i s[S_i].
 * Slot order is rank order: key descending, ties to the lower expert index.
 * score_out (optional, [T,E]) receives s for the sigmoid router. */
void orc_route(const float* logits, const float* logit_bias, const float* sel_bias,
               int T, int E, int k, int router, int n_groups, int topk_groups,
               double route_scale, int32_t* topk_idx, float* topk_gate, float* score_out) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        float l[4096], s[4096], key[4096];
        int allowed[4096], sel[4096];
        for (int e = 0; e < E; ++e) {
            float v = logits[(int64_t)t * E + e];
            l[e] = logit_bias ? v + logit_bias[e] : v;
        }
        if (router == ORC_SOFTMAX_TOPK) {
            select_topk(l, NULL, E, k, sel);
            double den = 0.0, num[4096];
            for (int j = 0; j < k; ++j) {
                num[j] = exp((double)l[sel[j]] - (double)l[sel[0]]);
                den += num[j];
            }
            for (int j = 0; j < k; ++j) {
                topk_idx[(int64_t)t * k + j] = sel[j];
                topk_gate[(int64_t)t * k + j] = (float)(num[j] / den);
            }
        } else {
            for (int e = 0; e < E; ++e) {
                s[e] = (float)(1.0 / (1.0 + exp(-(double)l[e])));
                key[e] = sel_bias ? s[e] + sel_bias[e] : s[e];
                if (score_out) score_out[(int64_t)t * E + e] = s[e];
            }
            int per = E / n_groups;
            float gscore[4096];
            int gsel[4096], top2[2];
            for (int g = 0; g < n_groups; ++g) {
                select_topk(key + g * per, NULL, per, 2, top2);
                gscore[g] = key[g * per + top2[0]] + key[g * per + top2[1]];
            }
            select_topk(gscore, NULL, n_groups, topk_groups, gsel);
            for (int e = 0; e < E; ++e) allowed[e] = 0;
            for (int i = 0; i < topk_groups; ++i)
                for (int e = gsel[i] * per; e < (gsel[i] + 1) * per; ++e) allowed[e] = 1;
            select_topk(key, allowed, E, k, sel);
            double den = 0.0;
            for (int j = 0; j < k; ++j) den += (double)s[sel[j]];
            for (int j = 0; j < k; ++j) {
                topk_idx[(int64_t)t * k + j] = sel[j];
                topk_gate[(int64_t)t * k + j] = (float)(route_scale * (double)s[sel[j]] / den);
            }
        }
    }
}

/* ------------------------------------------------------------------------------------ */
/* Permutation metadata: group the T*k (token, slot) assignments by expert              */
/* ------------------------------------------------------------------------------------ */

/* Counting sort of the assignments by expert, stable in token order; dropless, so every
 * assignment gets a row and there are exactly T*k rows.
 *   counts[e] = number of assignments to e; offsets = exclusive prefix sum (E+1 entries);
 *   pos[t*k+j] = row of assignment (t, j); src[row] = t; gate_perm[row] = topk_gate[t*k+j]. */
void orc_permute(const int32_t* topk_idx, const float* topk_gate, int T, int k, int E,
                 int32_t* counts, int32_t* offsets, int32_t* pos, int32_t* src,
                 float* gate_perm) {
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t a = 0; a < (int64_t)T * k; ++a) counts[topk_idx[a]] += 1;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t* next = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    for (int e = 0; e < E; ++e) next[e] = offsets[e];
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            int e = topk_idx[(int64_t)t * k + j];
            int32_t row = next[e]++;
            pos[(int64_t)t * k + j] = row;
            if (src) src[row] = t;
            if (gate_perm && topk_gate) gate_perm[row] = topk_gate[(int64_t)t * k + j];
        }
    }
    free(next);
}

/* Token-dropping permutation with an expert capacity of cap assignments (the capacity
 * factor of the study notes, 案例 3 / 踩过的坑: an expert with more assignments than slots
 * overflows and the surplus is dropped). Each expert accepts the assignments routed to it in
 * token order (t, then slot j) while it has a free slot; later ones are dropped, pos = -1.
 * counts = the demand per expert; offsets = exclusive prefix sum of the accepted counts. */
void orc_permute_capacity(const int32_t* topk_idx, const float* topk_gate, int T, int k, int E,
                          int cap, int32_t* counts, int32_t* offsets, int32_t* pos,
                          int32_t* src, float* gate_perm) {
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t a = 0; a < (int64_t)T * k; ++a) counts[topk_idx[a]] += 1;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + (counts[e] < cap ? counts[e] : cap);
    int32_t* taken = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            int64_t a = (int64_t)t * k + j;
            int e = topk_idx[a];
            if (taken[e] < cap) {
                int32_t row = offsets[e] + taken[e]++;
                pos[a] = row;
                src[row] = t;
                gate_perm[row] = topk_gate[a];
            } else {
                pos[a] = -1;
            }
        }
    }
    free(taken);
}

/* ------------------------------------------------------------------------------------ */
/* Expert MLP (step "gate(e) * Expert_e(x)")                                            */
/* ------------------------------------------------------------------------------------ */

/* MXFP8 "quantise then dequantise" of one row of n values given as fp32, 1 x 32 blocks
 * (the block rule of orc_mx_quant). */
static void fake_mx_row(const float* v, int n, double* out) {
    for (int b = 0; b < n / 32; ++b) {
        double amax = 0.0;
        for (int c = b * 32; c < b * 32 + 32; ++c)
            if (fabs((double)v[c]) > amax) amax = fabs((double)v[c]);
        int X = mx_exponent(amax);
        for (int c = b * 32; c < b * 32 + 32; ++c)
            out[c] = ldexp(g_e4m3_val[orc_e4m3_encode((float)ldexp((double)v[c], -X))], X);
    }
}

/* SwiGLU expert without biases: Expert(x) = W2 (silu(W_gate x) * (W_up x)),
 * silu(u) = u / (1 + exp(-u)); W13 holds W_gate in rows 0..F-1 and W_up in rows F..2F-1. */
static double silu(double u) { return u / (1.0 + exp(-u)); }

/* Hidden activation of one expert for one input row:
 *   z = W13_m x (2F values), h = silu(z_gate) * z_up, a = g * h.
 * Folding g into the activation before the down projection is the pages' memory-efficient
 * permutation ("使用 Megatron Core 大规模训练混合专家模型（MoE）", section 2.2): the gate is
 * absorbed into the activations, so W2 (g h) is computed instead of g (W2 h). */
static void expert_hidden(const wmat* w13, int64_t m, const double* x, int H, int F,
                          double g, double* z, double* a) {
    for (int r = 0; r < 2 * F; ++r) {
        double acc = 0.0;
        for (int h = 0; h < H; ++h) acc += wval(w13, m, r, h) * x[h];
        z[r] = acc;
    }
    for (int f = 0; f < F; ++f) a[f] = g * (silu(z[f]) * z[F + f]);
}

static void expert_down(const wmat* w2, int64_t m, const double* a, int H, int F, double* y) {
    for (int r = 0; r < H; ++r) {
        double acc = 0.0;
        for (int f = 0; f < F; ++f) acc += wval(w2, m, r, f) * a[f];
        y[r] = acc;
    }
}

/* In fp8 modes the activation entering the down projection is quantised after the gate
 * fold: it is rounded to fp32, then to e4m3 with an fp32 scale per 1 x 128 block
 * (mode 1) or with an E8M0 scale per 1 x 32 block (mode 2, MXFP8). */
static void quantise_act(double* a, int F, float* tmp, int mode) {
    for (int f = 0; f < F; ++f) tmp[f] = (float)a[f];
    if (mode == 2) fake_mx_row(tmp, F, a);
    else fake_quant_row(tmp, F, a);
}

/* Load one activation row as doubles: fp32/bf16 values, e4m3 codes times their 1 x 128
 * block scales (fp32), or MXFP8 codes times 2^(S - 127) of their 1 x 32 block. */
static void load_row(const void* x, int dtype, const void* scales, int64_t row, int H,
                     double* out) {
    if (dtype == ORC_E4M3) {
        const uint8_t* q = (const uint8_t*)x + row * H;
        const float* sc = (const float*)scales;
        for (int h = 0; h < H; ++h)
            out[h] = g_e4m3_val[q[h]] * (double)sc[row * (H / 128) + h / 128];
    } else if (dtype == ORC_MXFP8) {
        const uint8_t* q = (const uint8_t*)x + row * H;
        const uint8_t* sc = (const uint8_t*)scales;
        for (int h = 0; h < H; ++h)
            out[h] = g_e4m3_val[q[h]] * g_e8m0_val[sc[row * (H / 32) + h / 32]];
    } else {
        for (int h = 0; h < H; ++h) out[h] = load(x, dtype, row * H + h);
    }
}

/* The expert math of selected rows of the expert-grouped buffer x_perm [A, H].
 * Row r belongs to the expert e with offsets[e] <= r < offsets[e+1] (offsets == NULL means
 * one expert owning every row, as for the shared expert) and carries gate gate_perm[r]
 * (NULL means gate 1). Outputs per selected row: z [2F] (optional), the activation fed to the
 * down projection [F] (after the fp8 round trip when quant_act), and y_perm [H]. */
void orc_expert_rows(int H, int F, int E, const void* x_perm, int x_dtype,
                     const void* x_scales, const int32_t* offsets, const float* gate_perm,
                     const void* w13, const void* w2, int w_dtype, const void* w13_scales,
                     const void* w2_scales, int quant_act, const int64_t* rows,
                     int64_t n_rows, double* z_out, double* act_out, double* y_out) {
    init_tables();
    wmat W13 = {w13, w_dtype, w13_scales, 2 * F, H};
    wmat W2 = {w2, w_dtype, w2_scales, H, F};
#pragma omp parallel
    {
        double* x = (double*)malloc(sizeof(double) * (size_t)H);
        double* z = (double*)malloc(sizeof(double) * (size_t)(2 * F));
        double* a = (double*)malloc(sizeof(double) * (size_t)F);
        float* tmp = (float*)malloc(sizeof(float) * (size_t)F);
#pragma omp for schedule(dynamic)
        for (int64_t i = 0; i < n_rows; ++i) {
            int64_t r = rows[i];
            int e = 0;
            if (offsets)
                while (e + 1 < E && offsets[e + 1] <= r) ++e;
            double g = gate_perm ? (double)gate_perm[r] : 1.0;
            load_row(x_perm, x_dtype, x_scales, r, H, x);
            expert_hidden(&W13, e, x, H, F, g, z, a);
            if (quant_act) quantise_act(a, F, tmp, quant_act);
            if (z_out) memcpy(z_out + i * 2 * F, z, sizeof(double) * (size_t)(2 * F));
            memcpy(act_out + i * F, a, sizeof(double) * (size_t)F);
            expert_down(&W2, e, a, H, F, y_out + i * H);
        }
        free(x); free(z); free(a); free(tmp);
    }
}

/* The whole layer for selected tokens, literally the per-token loop:
 *   y = 0; for each kept expert e (slot order): y += Expert_e applied with gate g_e;
 *   plus the always-on shared expert with weight 1 when shared_F > 0.
 * fold = 1 computes W2 (g h); fold = 0 computes g (W2 h) (the unfolded form, kept to check
 * that the fold is a pure rearrangement). fp8 = 1: x is quantised per 1 x 128 block, the
 * weights are e4m3 codes with 128 x 128 block scales, and the folded activation is
 * quantised per 1 x 128 block before the down projection. fp8 = 2 (MXFP8): the same with
 * 1 x 32 blocks and E8M0 scales for x, the activation and the weights (w_dtype MXFP8). */
void orc_layer_tokens(int T, int H, int E, int k, int F, int shared_F, const void* x_in,
                      int x_dtype, int fp8, const int32_t* topk_idx, const float* topk_gate,
                      const void* w13, const void* w2, int w_dtype, const void* w13_scales,
                      const void* w2_scales, const void* ws13, const void* ws2,
                      const void* ws13_scales, const void* ws2_scales, int fold,
                      const int64_t* tokens, int64_t n_tokens, double* y_out) {
    (void)T;
    init_tables();
    wmat W13 = {w13, w_dtype, w13_scales, 2 * F, H};
    wmat W2 = {w2, w_dtype, w2_scales, H, F};
    wmat S13 = {ws13, w_dtype, ws13_scales, 2 * shared_F, H};
    wmat S2 = {ws2, w_dtype, ws2_scales, H, shared_F};
    int Fm = F > shared_F ? F : shared_F;
#pragma omp parallel
    {
        double* x = (double*)malloc(sizeof(double) * (size_t)H);
        double* z = (double*)malloc(sizeof(double) * (size_t)(2 * Fm));
        double* a = (double*)malloc(sizeof(double) * (size_t)Fm);
        double* ye = (double*)malloc(sizeof(double) * (size_t)H);
        float* tmp = (float*)malloc(sizeof(float) * (size_t)(H > Fm ? H : Fm));
#pragma omp for schedule(dynamic)
        for (int64_t i = 0; i < n_tokens; ++i) {
            int64_t t = tokens[i];
            double* y = y_out + i * H;
            if (fp8) {
                for (int h = 0; h < H; ++h) tmp[h] = (float)load(x_in, x_dtype, t * H + h);
                if (fp8 == 2) fake_mx_row(tmp, H, x);
                else fake_quant_row(tmp, H, x);
            } else {
                load_row(x_in, x_dtype, NULL, t, H, x);
            }
            for (int h = 0; h < H; ++h) y[h] = 0.0;
            for (int j = 0; j < k; ++j) {
                int e = topk_idx[t * k + j];
                if (e < 0) continue;                  /* slot dropped by an expert capacity */
                double g = (double)topk_gate[t * k + j];
                expert_hidden(&W13, e, x, H, F, fold ? g : 1.0, z, a);
                if (fp8) quantise_act(a, F, tmp, fp8);
                expert_down(&W2, e, a, H, F, ye);
                for (int h = 0; h < H; ++h) y[h] += fold ? ye[h] : g * ye[h];
            }
            if (shared_F > 0) {
                expert_hidden(&S13, 0, x, H, shared_F, 1.0, z, a);
                if (fp8) quantise_act(a, shared_F, tmp, fp8);
                expert_down(&S2, 0, a, H, shared_F, ye);
                for (int h = 0; h < H; ++h) y[h] += ye[h];
            }
        }
        free(x); free(z); free(a); free(ye); free(tmp);
    }
}

/* ------------------------------------------------------------------------------------ */
/* Backward of the expert MLP with the gate fold (weight and data gradients kept apart) */
/* ------------------------------------------------------------------------------------ */

/* For rows r of one expert with saved z = W13 x (2F) and gate g, and upstream dy_perm [H]:
 *   da = W2^T dy                      (F)      data gradient through the down projection
 *   h  = silu(z_g) z_u,  dg = sum_f da[f] h[f]
 *   dh = g da
 *   dz_g = dh z_u silu'(z_g),  dz_u = dh silu(z_g)
 *   dx = W13^T dz                     (H)      data gradient through the gate/up projection
 * and the weight gradients are sums over the expert's rows:
 *   dW2[i, f]  = sum_r dy[r, i] a[r, f]       with a = g h (the folded activation)
 *   dW13[i, h] = sum_r dz[r, i] x[r, h].
 * silu'(u) = s (1 + u (1 - s)), s = 1 / (1 + exp(-u)).
 * All operands are read as given (bf16 or fp32) and combined in double. */
static double dsilu(double u) {
    double s = 1.0 / (1.0 + exp(-u));
    return s * (1.0 + u * (1.0 - s));
}

/* Data gradients of selected rows: dx_out [n, H], dg_out [n]. z is the saved [A, 2F]. */
void orc_expert_bwd_rows(int H, int F, int E, const void* dy_perm, const void* z, int dtype,
                         const int32_t* offsets, const float* gate_perm, const void* w13,
                         const void* w2, const int64_t* rows, int64_t n_rows,
                         double* dx_out, double* dg_out) {
#pragma omp parallel
    {
        double* dy = (double*)malloc(sizeof(double) * (size_t)H);
        double* zz = (double*)malloc(sizeof(double) * (size_t)(2 * F));
        double* da = (double*)malloc(sizeof(double) * (size_t)F);
        double* dz = (double*)malloc(sizeof(double) * (size_t)(2 * F));
        wmat W13 = {w13, dtype, NULL, 2 * F, H};
        wmat W2 = {w2, dtype, NULL, H, F};
#pragma omp for schedule(dynamic)
        for (int64_t i = 0; i < n_rows; ++i) {
            int64_t r = rows[i];
            int e = 0;
            if (offsets)
                while (e + 1 < E && offsets[e + 1] <= r) ++e;
            double g = gate_perm ? (double)gate_perm[r] : 1.0;
            load_row(dy_perm, dtype, NULL, r, H, dy);
            load_row(z, dtype, NULL, r, 2 * F, zz);
            for (int f = 0; f < F; ++f) {
                double acc = 0.0;
                for (int h = 0; h < H; ++h) acc += wval(&W2, e, h, f) * dy[h];
                da[f] = acc;
            }
            double dg = 0.0;
            for (int f = 0; f < F; ++f) {
                double u = zz[f], v = zz[F + f];
                dg += da[f] * silu(u) * v;
                double dh = g * da[f];
                dz[f] = dh * v * dsilu(u);
                dz[F + f] = dh * silu(u);
            }
            dg_out[i] = dg;
            for (int h = 0; h < H; ++h) {
                double acc = 0.0;
                for (int c = 0; c < 2 * F; ++c) acc += wval(&W13, e, c, h) * dz[c];
                dx_out[i * H + h] = acc;
            }
        }
        free(dy); free(zz); free(da); free(dz);
    }
}

/* dz rows [M, 2F] for rows [r0, r0+M) of one expert (helper of the weight gradients). */
static void expert_dz(int H, int F, const void* dy_perm, const void* z, int dtype, int e,
                      const float* gate_perm, const void* w2, int64_t r0, int64_t M,
                      double* dz) {
    wmat W2 = {w2, dtype, NULL, H, F};
#pragma omp parallel
    {
        double* dy = (double*)malloc(sizeof(double) * (size_t)H);
        double* zz = (double*)malloc(sizeof(double) * (size_t)(2 * F));
        double* da = (double*)malloc(sizeof(double) * (size_t)F);
#pragma omp for schedule(dynamic)
        for (int64_t i = 0; i < M; ++i) {
            int64_t r = r0 + i;
            double g = gate_perm ? (double)gate_perm[r] : 1.0;
            load_row(dy_perm, dtype, NULL, r, H, dy);
            load_row(z, dtype, NULL, r, 2 * F, zz);
            for (int f = 0; f < F; ++f) {
                double acc = 0.0;
                for (int h = 0; h < H; ++h) acc += wval(&W2, e, h, f) * dy[h];
                da[f] = acc;
            }
            for (int f = 0; f < F; ++f) {
                double u = zz[f], v = zz[F + f];
                double dh = g * da[f];
                dz[i * 2 * F + f] = dh * v * dsilu(u);
                dz[i * 2 * F + F + f] = dh * silu(u);
            }
        }
        free(dy); free(zz); free(da);
    }
}

/* Weight gradients of one expert e (rows offsets[e] .. offsets[e+1]) at selected entries:
 *   dw13_out[i] = dW13_e[w13_r[i], w13_c[i]],  dw2_out[i] = dW2_e[w2_r[i], w2_c[i]].
 * act is the saved folded activation [A, F]; x_perm the saved input [A, H]. */
void orc_expert_wgrad_entries(int H, int F, const void* dy_perm, const void* z,
                              const void* act, const void* x_perm, int dtype,
                              const int32_t* offsets, int e, const float* gate_perm,
                              const void* w2, const int32_t* w13_r, const int32_t* w13_c,
                              int64_t n13, double* dw13_out, const int32_t* w2_r,
                              const int32_t* w2_c, int64_t n2, double* dw2_out) {
    int64_t r0 = offsets ? offsets[e] : 0;
    int64_t M = offsets ? offsets[e + 1] - offsets[e] : 0;
    double* dz = (double*)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1) * (size_t)(2 * F));
    if (M > 0) expert_dz(H, F, dy_perm, z, dtype, e, gate_perm, w2, r0, M, dz);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n13; ++i) {
        double acc = 0.0;
        for (int64_t m = 0; m < M; ++m)
            acc += dz[m * 2 * F + w13_r[i]] * load(x_perm, dtype, (r0 + m) * H + w13_c[i]);
        dw13_out[i] = acc;
    }
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n2; ++i) {
        double acc = 0.0;
        for (int64_t m = 0; m < M; ++m)
            acc += load(dy_perm, dtype, (r0 + m) * H + w2_r[i]) *
                   load(act, dtype, (r0 + m) * F + w2_c[i]);
        dw2_out[i] = acc;
    }
    free(dz);
}

/* ------------------------------------------------------------------------------------ */
/* Unpermute / combine                                                                  */
/* ------------------------------------------------------------------------------------ */

/* y[t] = sum_j y_perm[pos[t*k+j]] (+ shared_y[t]): the token's expert outputs brought back
 * to token order and added; the gates are already inside y_perm (folded before the down
 * projection). Inputs fp32 or bf16 (shared_y may be NULL), output double. */
void orc_combine(const void* y_perm, const void* shared_y, int dtype, const int32_t* pos,
                 int T, int k, int H, double* y) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j) {
                int64_t r = pos[(int64_t)t * k + j];
                if (r >= 0) acc += load(y_perm, dtype, r * H + h);   /* < 0: dropped slot */
            }
            if (shared_y) acc += load(shared_y, dtype, (int64_t)t * H + h);
            y[(int64_t)t * H + h] = acc;
        }
    }
}

/* Host threads of the oracle's parallel loops (timing of the CPU baseline only; results do
 * not depend on the thread count: every output is written by one thread, in a fixed order). */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int orc_max_threads(void) { return omp_get_max_threads(); }

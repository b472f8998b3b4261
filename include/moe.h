/*
 * moe.h -- C ABI of the MI355X (gfx950) forward pass of one token-choice
 * Mixture-of-Experts layer on one GPU's share of tokens:
 *
 *   router scores -> top-k experts and gates -> permute (group the token copies by
 *   expert) -> SwiGLU experts as one grouped GEMM (gate folded into the activation)
 *   -> unpermute / combine back to token order,   y = sum_e g_e * Expert_e(x).
 *
 * The steps follow the per-token loop in the study notes "Megatron-Core MoE --
 * 大规模稀疏专家并行实践" (实践案例, 案例 1) and the optimisations named in the
 * technical summary "使用 Megatron Core 大规模训练混合专家模型（MoE）" (section 2.2
 * memory-efficient permutation; section 2.4 grouped GEMM, fused routing/permutation and
 * sync-free kernels).
 *
 * Conventions (every entry point):
 *  - Pointers are DEVICE pointers owned by the caller, except `cfg` and `bytes`, which are
 *    host pointers read (written) during the call only. Device pointers must be 16-byte
 *    aligned (the kernels load and store 16-byte vectors; the library does not check). The library never allocates or
 *    frees device memory; scratch comes from the caller's workspace `ws` of `ws_bytes`
 *    bytes, sized by moe_workspace_size().
 *  - Work is enqueued on `stream` and the call returns at once. The library never
 *    synchronises a stream or the device and never copies device -> host: expert counts
 *    and offsets stay on the device. The backward calls (moe_grouped_gemm_swiglu_bwd,
 *    moe_layer_backward, moe_layer_backward_saved) run their expert weight gradients on
 *    two side streams of the library's, forked from `stream` and joined back to it with
 *    events (the weight gradients overlap the data gradients), so all of a call's work is
 *    still ordered on `stream`.
 *  - Arguments are validated on the host before anything is enqueued; on an invalid
 *    argument nothing is launched and MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED or
 *    MOE_ERR_WORKSPACE is returned. A failed launch returns MOE_ERR_HIP. Expert indices
 *    are not validated on the device: topk_idx must come from moe_route or lie in [0, E).
 *  - Every output is overwritten, never accumulated into. Results are deterministic:
 *    bit-identical across runs. No floating-point atomics are used; the one split-K (the
 *    bf16 router GEMM inside moe_layer_forward, up to 8 K ranges) writes one partial sum
 *    per range and adds them in a fixed range order.
 *  - The library holds no state between calls except the instrumentation switch of
 *    moe_set_stage_events (per host thread; it changes no result) and, per device, the
 *    backward's two side streams and five events (created on the first backward call on
 *    that device, default priority, kept until the process ends; they carry no data).
 *  - Layouts: every matrix keeps K (its last index) contiguous, so each expert GEMM is
 *    C = A B^T. A matrix [R, C] is either row-major (MOE_LAYOUT_ROWS) or K-blocked
 *    (MOE_LAYOUT_KBLOCK): stored as [C * eb / 64][R][64 bytes] (eb = element bytes), i.e.
 *    the 64-byte K slice j of row r is at byte (j * R + r) * 64, so one K slice of
 *    consecutive rows is one contiguous run. Stacked weights [E, N, K] are K-blocked per
 *    expert. moe_config.a_layout selects the layout of the expert-grouped activations
 *    (x_perm, act, a shared expert's act) and w_layout that of the expert weights
 *    (w13, w2, ws13, ws2); everything else (x, y, y_perm, z, scales) is row-major.
 *    fp8 scale tensors are row-major over blocks: fp32 for MOE_E4M3, one E8M0 byte per
 *    block for MOE_MXFP8 (scale arguments are therefore `void*`).
 *  - Calls on different streams may overlap if their outputs and workspaces are disjoint.
 */
#ifndef MOE_AMD_H
#define MOE_AMD_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, k > E, ... */
    MOE_ERR_UNSUPPORTED = 2,   /* valid but not implemented (dtype mix, H % 128 != 0 ...) */
    MOE_ERR_WORKSPACE = 3,     /* ws_bytes smaller than moe_workspace_size() */
    MOE_ERR_HIP = 4            /* a HIP launch failed */
} moe_status;

/* MOE_MXFP8: the MXFP8 format of the OCP Microscaling (MX) specification, named among the
 * low-precision recipes of "使用 Megatron Core 大规模训练混合专家模型（MoE）" (section 3, key
 * contributions; FP8 expert GEMMs in section 2.4): OCP E4M3 elements in blocks of 32
 * consecutive values along K, each block with one E8M0 scale byte S (the power of two
 * 2^(S - 127)). Quantising a block with largest magnitude amax: X = floor(log2 amax) - 8
 * (8 = exponent of E4M3's largest normal), clamped to [-127, 127], X = -127 for an all-zero
 * block; S = X + 127; q = e4m3_rne_saturate(v * 2^-X). */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_E4M3 = 2, MOE_MXFP8 = 3 } moe_dtype;

typedef enum { MOE_LAYOUT_ROWS = 0, MOE_LAYOUT_KBLOCK = 1 } moe_layout;

typedef enum {
    /* select on the logits (ties to the lower expert index); gates = softmax over the k
     * selected logits (the full softmax renormalised over the selected set) */
    MOE_ROUTER_SOFTMAX_TOPK = 0,
    /* s = sigmoid(logit) (evaluated in double, rounded once to fp32); key = s + sel_bias;
     * group score = sum of the two largest keys of each of n_groups contiguous expert
     * groups; keep topk_groups groups; top-k experts by key inside them;
     * gates = route_scale * s / sum(s over the selected) (the bias selects only) */
    MOE_ROUTER_SIGMOID_GROUP_TOPK = 1
} moe_router;

typedef enum {
    MOE_OP_PERMUTE = 0,
    MOE_OP_GROUPED_GEMM = 1,
    MOE_OP_LAYER_FORWARD = 2,
    MOE_OP_GROUPED_GEMM_BWD = 3,
    MOE_OP_LAYER_BACKWARD = 4,
    MOE_OP_ROUTE_STATS = 5,
    /* not a workspace: the size of the `saved` buffer of moe_layer_forward_train and
     * moe_layer_backward_saved */
    MOE_OP_LAYER_SAVED = 6
} moe_op;

/* Layer shape and numerics. Host memory, read only during a call. */
typedef struct {
    int32_t T;            /* tokens on this GPU */
    int32_t H;            /* hidden size */
    int32_t E;            /* routed experts (1 .. 1024) */
    int32_t k;            /* experts per token (1 .. min(E, 32)) */
    int32_t F;            /* SwiGLU width of one routed expert */
    int32_t n_groups;     /* expert groups for the group-limited router (1 = none) */
    int32_t topk_groups;  /* groups kept per token */
    int32_t router;       /* moe_router */
    float route_scale;    /* gate multiplier (1 for softmax, 2.5 DeepSeek-V3 style) */
    int32_t act_dtype;    /* MOE_F32 or MOE_BF16: x, router weight, y_perm, y */
    int32_t w_dtype;      /* expert GEMM operands: MOE_F32 (with act F32), MOE_BF16,
                             MOE_E4M3 (with act BF16: 1x128 activation scales, 128x128
                             weight scales, fp32 accumulation) or MOE_MXFP8 (with act BF16
                             and row-major activations: 1x32 E8M0 scales along K for the
                             activations and the weights, fp32 accumulation; K-blocked
                             weight codes take scales packed by moe_pack_mx_scales).
                             With the fp8 dtypes every one-byte activation matrix must stay
                             below 4 GiB: (T*k + T) * max(H, F, shared_F) < 2^32, else
                             MOE_ERR_UNSUPPORTED */
    int32_t shared_F;     /* width of the always-on shared expert, 0 = none */
    int32_t a_layout;     /* moe_layout of x_perm / act in the standalone calls (bf16, e4m3) */
    int32_t w_layout;     /* moe_layout of the expert weights (bf16, e4m3) */
    float capacity_factor;/* 0: dropless (every assignment is computed). > 0: token-dropping
                             routing with an expert capacity of
                             C = ceil(capacity_factor * T * k / E) assignments (evaluated in
                             double); each expert keeps its first C assignments in token
                             order and drops the rest (the capacity factor / overflowing
                             expert slots of the study notes, 案例 3 and 踩过的坑). The
                             backward entry points require 0. */
} moe_config;

/* Name of a status code (static string; never NULL). */
const char* moe_status_string(int status);

/* Workspace bytes needed by entry point `op` for `cfg`. Host only, no HIP call. */
int moe_workspace_size(const moe_config* cfg, int op, size_t* bytes);

/* Router scores (the scoring step of the per-token loop in the study notes
 * "Megatron-Core MoE -- 大规模稀疏专家并行实践", 实践案例 案例 1): a linear router without bias,
 *   logits[t, e] = sum_h x[t, h] * w_router[e, h],  fp32 accumulation and output.
 * x [T, H] and w_router [E, H] are in cfg->act_dtype; logits [T, E] fp32. */
int moe_router_logits(const moe_config* cfg, const void* x, const void* w_router,
                      float* logits, hipStream_t stream);

/* Top-k expert selection and gates (the selection step of the same loop, 案例 1), one
 * wavefront per token.
 *   l[e] = fp32(logits[t, e] + logit_bias[e])    (logit_bias [E] fp32, may be NULL)
 * then cfg->router (see moe_router). sel_bias [E] fp32 is used by the sigmoid router and
 * may be NULL there (zero bias). Slots are in rank order: key descending, ties to the
 * lower expert index (-0.0 ties +0.0).
 * Outputs: topk_idx [T, k] int32, topk_gate [T, k] fp32. */
int moe_route(const moe_config* cfg, const float* logits, const float* logit_bias,
              const float* sel_bias, int32_t* topk_idx, float* topk_gate,
              hipStream_t stream);

/* moe_route plus the load-balancing statistics of the routing, computed in the same kernel
 * (the expert-utilisation view the study notes ask for before tuning capacity and the
 * auxiliary loss, 案例 3; the per-expert assignment counts come from moe_permute):
 *   prob_mean[e] = (1/T) sum_t p[t, e]                                      [E] fp32
 * with p the router's normalised probabilities of token t over all E experts, from
 * l = fp32(logits + logit_bias): the softmax router's p = softmax(l); the sigmoid router's
 * p = s / sum_e s with s = sigmoid(l) as in moe_route (the selection bias excluded).
 * p is evaluated in fp32 per token; the sums run in a fixed order (per 4-token block, then
 * over blocks), so the result is deterministic. No loss formula is applied: counts and
 * prob_mean are the inputs of the usual balance losses. Workspace:
 * moe_workspace_size(cfg, MOE_OP_ROUTE_STATS). topk_idx / topk_gate as moe_route. */
int moe_route_stats(const moe_config* cfg, const float* logits, const float* logit_bias,
                    const float* sel_bias, int32_t* topk_idx, float* topk_gate,
                    float* prob_mean, void* ws, size_t ws_bytes, hipStream_t stream);

/* Permute: the routing metadata that says which token goes to which expert (indices,
 * counts, offsets: the study notes, 实践案例 案例 1) and the copy of x grouped by expert, as
 * the fused routing/permutation and sync-free kernels of the technical summary (section
 * 2.4): computed on the device without any host synchronisation. Dropless: exactly
 * A = T*k rows.
 *   counts[e]   = number of (t, j) with topk_idx[t, j] == e              [E]    int32
 *   offsets     = exclusive prefix sum of counts (offsets[E] = A)          [E+1]  int32
 *   pos[t*k+j]  = row of assignment (t, j); rows of one expert are in ascending token
 *                 order (a stable counting sort)                           [A]    int32
 * With cfg->capacity_factor > 0 (capacity C, see moe_config): counts stay the demand, but
 * offsets scan the kept counts min(counts[e], C), so offsets[E] = A - dropped; an
 * assignment whose rank in its expert (token order) is >= C gets pos = -1 and no row, and
 * src / gate_perm / x_perm are written for rows [0, offsets[E]) only.
 *   src[row]    = token of a row                                           [A]    int32
 *   gate_perm[row] = topk_gate of the assignment                           [A]    fp32
 *   x_perm[pos[t*k+j], :] = x[t, :]                                        [A, H]
 * With cfg->w_dtype == MOE_E4M3, x (bf16) is quantised per 1 x 128 block
 * (s = fp32(amax / 448), q = e4m3_rne_saturate(fp32(x / s))): x_perm holds the e4m3
 * codes and x_perm_scales [A, H/128] the scales; x_q [T, H] / x_q_scales [T, H/128]
 * optionally (may be NULL) receive the quantised x in token order (for a shared expert;
 * with a K-blocked x_perm they also let each token be quantised once and then gathered).
 * With MOE_MXFP8, the same with 1 x 32 blocks: x_perm_scales [A, H/32] and x_q_scales
 * [T, H/32] hold E8M0 bytes (a_layout must be row-major).
 * Otherwise x_perm has cfg->act_dtype and the scale pointers must be NULL.
 * x_perm is in cfg->a_layout; a K-blocked x_perm is written by a gather over src so that
 * every store is a contiguous kilobyte. */
int moe_permute(const moe_config* cfg, const void* x, const int32_t* topk_idx,
                const float* topk_gate, int32_t* counts, int32_t* offsets, int32_t* pos,
                int32_t* src, float* gate_perm, void* x_perm, void* x_perm_scales,
                void* x_q, void* x_q_scales, void* ws, size_t ws_bytes,
                hipStream_t stream);

/* moe_permute without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments, outputs and results as moe_permute, bit for bit, but its scratch (the
 * per-chunk expert histograms, ceil(T*k / 512) * E int32) lives in a 4 MiB device array
 * inside the library that each GPU holds until the process ends. Sizes whose scratch exceeds
 * 4 MiB (ceil(T*k / 512) * E > 1048576) return MOE_ERR_WORKSPACE and launch nothing. Every
 * call overwrites the part it uses (nothing needs to start at zero). Calls that overlap on one
 * GPU (several streams or host threads at once) share that array and race: serialise them.
 * The stream must belong to the current device. Allocates nothing, ever. */
int moe_permute_noalloc(const moe_config* cfg, const void* x, const int32_t* topk_idx,
                        const float* topk_gate, int32_t* counts, int32_t* offsets,
                        int32_t* pos, int32_t* src, float* gate_perm, void* x_perm,
                        void* x_perm_scales, void* x_q, void* x_q_scales, hipStream_t stream);

/* SwiGLU experts as one grouped GEMM over the expert-grouped rows (ragged per-expert M).
 * For expert e and its rows R_e = [offsets[e], offsets[e+1]):
 *   Z   = x_perm[R_e] W13_e^T                     [M_e, 2F]  (fp32 accumulation)
 *   act = gate_perm[r] * silu(Z[:, :F]) * Z[:, F:] [M_e, F]   (gate folded in: the
 *         memory-efficient permutation of the technical summary, section 2.2)
 *   y_perm[R_e] = act W2_e^T                       [M_e, H]
 * w13 [E, 2F, H] (rows 0..F-1 gate, F..2F-1 up), w2 [E, H, F]. With MOE_E4M3 weights,
 * w13_scales [E, 2F/128, H/128] and w2_scales [E, H/128, F/128] are the 128 x 128 block
 * scales, x_perm is e4m3 with x_perm_scales [A, H/128], and act is stored as e4m3 with
 * act_scales [A, F/128] (quantised per 1 x 128 after the fold). With MOE_MXFP8 every
 * operand has E8M0 bytes per 1 x 32 block along K instead: x_perm_scales [A, H/32],
 * w13_scales [E, 2F, H/32], w2_scales [E, H, F/32], act_scales [A, F/32] (act quantised per
 * 1 x 32 after the fold), and the shared expert's likewise; with K-blocked weights
 * (w_layout) the weight scales are in the order of moe_pack_mx_scales. Otherwise all scale pointers
 * must be NULL and act has cfg->act_dtype. y_perm has cfg->act_dtype.
 * Shared expert (cfg->shared_F > 0): the same SwiGLU with weight 1 applied to every token
 * of x_shared [T, H] (e4m3 + x_shared_scales in fp8 mode), weights ws13 [2*shared_F, H],
 * ws2 [H, shared_F] (+ scales), output shared_y [T, H] in cfg->act_dtype. Pass NULL for
 * all shared arguments when shared_F == 0.
 * z_out [A, 2F] (optional, NULL = not saved): Z rounded to cfg->act_dtype, for a backward. */
int moe_grouped_gemm_swiglu(const moe_config* cfg, const void* x_perm,
                            const void* x_perm_scales, const int32_t* offsets,
                            const float* gate_perm, const void* w13, const void* w13_scales,
                            const void* w2, const void* w2_scales, const void* x_shared,
                            const void* x_shared_scales, const void* ws13,
                            const void* ws13_scales, const void* ws2,
                            const void* ws2_scales, void* act, void* act_scales,
                            void* y_perm, void* shared_y, void* z_out, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/* The two halves of moe_grouped_gemm_swiglu as separate calls (same arguments and
 * layouts), for callers that schedule or time them apart -- e.g. the data- and
 * weight-gradient split of a backward.
 * moe_grouped_gemm_up:   act (and optionally z_out) from x_perm and w13; with a shared
 *                        expert, shared_act [T, shared_F] (+ shared_act_scales
 *                        [T, shared_F/128] in e4m3 mode, [T, shared_F/32] E8M0 in
 *                        MXFP8 mode) from x_shared and ws13.
 * moe_grouped_gemm_down: y_perm from act and w2; with a shared expert, shared_y from
 *                        shared_act and ws2.
 * Both need a workspace of moe_workspace_size(cfg, MOE_OP_GROUPED_GEMM) bytes. */
int moe_grouped_gemm_up(const moe_config* cfg, const void* x_perm, const void* x_perm_scales,
                        const int32_t* offsets, const float* gate_perm, const void* w13,
                        const void* w13_scales, const void* x_shared,
                        const void* x_shared_scales, const void* ws13,
                        const void* ws13_scales, void* act, void* act_scales,
                        void* shared_act, void* shared_act_scales, void* z_out, void* ws,
                        size_t ws_bytes, hipStream_t stream);
int moe_grouped_gemm_down(const moe_config* cfg, const void* act, const void* act_scales,
                          const int32_t* offsets, const void* w2, const void* w2_scales,
                          const void* shared_act, const void* shared_act_scales,
                          const void* ws2, const void* ws2_scales, void* y_perm,
                          void* shared_y, void* ws, size_t ws_bytes, hipStream_t stream);

/* Unpermute / combine (the weighted sum over the selected experts that ends the per-token
 * loop of the study notes, 实践案例 案例 1; the weights were folded in before the down
 * projection, the memory-efficient permutation of the technical summary, section 2.2):
 * y[t, :] = sum_{j<k} y_perm[pos[t*k+j], :] (+ shared_y[t, :]), where a
 * slot with pos < 0 (dropped by an expert capacity) contributes nothing,
 * summed in fp32 in slot order and rounded once to cfg->act_dtype. The gates were folded
 * in before the down projection, so no weight is applied here. A gather: no atomics.
 * shared_y may be NULL. */
int moe_unpermute_combine(const moe_config* cfg, const void* y_perm, const int32_t* pos,
                          const void* shared_y, void* y, hipStream_t stream);

/* The whole layer, i.e. the per-token loop of the study notes (实践案例 案例 1) run for all T
 * tokens at once with the fused routing/permutation, grouped GEMM and sync-free kernels of
 * the technical summary (section 2.4): router GEMM (skipped when logits_in != NULL), route,
 * permute, grouped GEMM with the shared expert, combine. x [T, H] and w_router [E, H] in
 * act_dtype; weights
 * as in moe_grouped_gemm_swiglu (in cfg->w_layout); y [T, H] in act_dtype. The expert-grouped
 * activations live in the workspace, row-major whatever cfg->a_layout says (cfg->a_layout
 * applies to the stand-alone calls only). For bf16, the router's split-K partial sums use the
 * workspace's y_perm region before the down projection writes it.
 * Optional outputs (NULL = skip): logits_out [T, E] (the router's logits, or a copy of
 * logits_in when that is given), topk_idx_out [T, k], topk_gate_out [T, k], counts_out [E]
 * (the demand per expert, before any capacity).
 * With cfg->capacity_factor > 0, dropped assignments (see moe_permute) add nothing to y. */
int moe_layer_forward(const moe_config* cfg, const void* x, const void* w_router,
                      const float* logit_bias, const float* sel_bias, const float* logits_in,
                      const void* w13, const void* w13_scales, const void* w2,
                      const void* w2_scales, const void* ws13, const void* ws13_scales,
                      const void* ws2, const void* ws2_scales, void* y, float* logits_out,
                      int32_t* topk_idx_out, float* topk_gate_out, int32_t* counts_out,
                      void* ws, size_t ws_bytes, hipStream_t stream);

/* Stage timing of moe_layer_forward (instrumentation; computes nothing). Not from the
 * pages: it lets a caller time each kernel of the layer on the stream it runs on. This is
 * the library's only state: a per-host-thread switch and the 7 event handles it was given
 * (thread-local, so threads do not see each other's setting). It never changes a result.
 * events: MOE_N_STAGE_EVENTS hipEvent_t handles that the caller created (with timing) and
 * keeps alive. Until the next call on the same host thread, every moe_layer_forward on that
 * thread records events[i] on its stream when stage i starts and events[6] when the last one
 * ends; stages: 0 router logits (no kernel when logits_in is given), 1 top-k routing,
 * 2 permutation, 3 grouped GEMM up (gate/up + SwiGLU), 4 grouped GEMM down, 5 combine.
 * events == NULL turns recording off. n_events other than MOE_N_STAGE_EVENTS, or a NULL
 * handle, gives MOE_ERR_INVALID_ARG and leaves the previous setting. */
#define MOE_N_STAGE_EVENTS 7
int moe_set_stage_events(void* const* events, int32_t n_events);

/* Backward of the grouped expert MLP with the gate fold (bf16 operands, fp32
 * accumulation), data and weight gradients as separate grouped GEMMs (the W/D split of the
 * technical summary, section 2.3). Per expert rows R_e = [offsets[e], offsets[e+1]), with
 * h = silu(Z_g) * Z_u from the saved z and g = gate_perm[r]:
 *   dA      = dy_perm W2_e                    dg[r] = sum_f dA[r, f] h[r, f]
 *   dZ_g    = g dA Z_u silu'(Z_g)             dZ_u  = g dA silu(Z_g)
 *   dx_perm = dZ W13_e                        [M_e, H]
 *   dW2_e   = dy_perm[R_e]^T act[R_e]         [H, F]
 *   dW13_e  = dZ[R_e]^T x_perm[R_e]           [2F, H]
 * All tensors bf16 (cfg->act_dtype == MOE_BF16, a_layout = 0; cfg->w_dtype is not used:
 * the backward runs on the bf16 weights), row-major except the weights, which follow
 * cfg->w_layout (row-major, or K-blocked as the forward takes them, so one copy serves
 * both): dy_perm [A, H], x_perm [A, H], z [A, 2F] and act [A, F] (the forward's saved Z and
 * g * h), w13 [E, 2F, H], w2 [E, H, F]. The results do not depend on the weight layout.
 * Outputs (row-major) dx_perm [A, H], dw13 [E, 2F, H], dw2 [E, H, F] bf16 and
 * dgate_perm [A] fp32 (may be NULL). gate_perm may be NULL (gate 1 for every row: a shared
 * expert is one group whose offsets are {0, T}). Experts with no rows get zero weight
 * gradients. Deterministic: dg is summed per tile, then over tiles in a fixed order.
 * Workspace: moe_workspace_size(cfg, MOE_OP_GROUPED_GEMM_BWD). */
int moe_grouped_gemm_swiglu_bwd(const moe_config* cfg, const void* dy_perm,
                                const void* x_perm, const void* z, const void* act,
                                const float* gate_perm, const int32_t* offsets, const void* w13,
                                const void* w2, void* dx_perm, void* dw13, void* dw2,
                                float* dgate_perm, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/* Backward of the whole layer (bf16 operands, fp32 accumulation, bf16 gradients): the
 * forward of the study notes' case 1 (y = sum_j g_j Expert_{e_j}(x) + shared(x), gate folded
 * into the activation as in the technical summary, section 2.2) differentiated by the chain
 * rule, data and weight gradients as separate GEMMs (section 2.3). The expert selection is a
 * choice and carries no gradient; logit_bias and sel_bias are constants.
 * Inputs are the forward's: x [T, H], w_router [E, H], logits [T, E] (fp32, before
 * logit_bias), logit_bias [E] or NULL, topk_idx / topk_gate [T, k] (moe_route's outputs),
 * w13 [E, 2F, H], w2 [E, H, F], ws13 / ws2 (shared expert, NULL when shared_F == 0), and
 * dy [T, H]. Z and act are recomputed (one extra GEMM1), so nothing of the forward's
 * workspace is needed. Gates to logits:
 *   softmax: dl_j = g_j (dg_j - sum_i g_i dg_i)
 *   sigmoid: dl_j = (c / S) (dg_j - sum_i dg_i g_i / c) s_j (1 - s_j),  S = sum_i s_i,
 * zero for unselected experts; dW_r = dl^T x, and dx collects the experts' rows (combine),
 * the shared expert and dl W_r. Outputs (all overwritten): dx [T, H], dw_router [E, H],
 * dw13, dw2 (zero for experts without rows), dws13, dws2 (NULL without a shared expert) in
 * bf16, and dlogits_out [T, E] fp32 (optional, NULL = skip). dl passes through bf16 on its
 * way to the router GEMMs. Requires act_dtype = w_dtype = MOE_BF16, a_layout = 0 and
 * E % 128 == 0 (else MOE_ERR_UNSUPPORTED); the expert weights (w13, w2, ws13, ws2) follow
 * cfg->w_layout, the gradients are row-major, and the results do not depend on the weight
 * layout. Deterministic.
 * Workspace: moe_workspace_size(cfg, MOE_OP_LAYER_BACKWARD). */
int moe_layer_backward(const moe_config* cfg, const void* x, const void* w_router,
                       const float* logits, const float* logit_bias, const int32_t* topk_idx,
                       const float* topk_gate, const void* w13, const void* w2,
                       const void* ws13, const void* ws2, const void* dy, void* dx,
                       void* dw_router, void* dw13, void* dw2, void* dws13, void* dws2,
                       float* dlogits_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* The training pair: a forward that keeps GEMM1's outputs, and the backward that uses them
 * instead of recomputing GEMM1. The technical summary on large-scale MoE training with
 * Megatron Core (section 2.2, fine-grained recomputation) weighs activation memory against
 * recomputation; moe_layer_backward recomputes the whole GEMM1, this pair keeps it:
 * Z [T*k, 2F] and act [T*k, F] of the routed rows in expert order, and the shared expert's
 * Z [T, 2 shared_F] and act [T, shared_F], bf16 row-major, in one caller-owned buffer of
 * moe_workspace_size(cfg, MOE_OP_LAYER_SAVED) bytes (about 0.9 GB for T = 8192, k = 8,
 * F = shared_F = 2048). Its layout is private to the pair; contents live until the caller
 * overwrites them.
 * moe_layer_forward_train: moe_layer_forward for act_dtype = w_dtype = MOE_BF16, a_layout 0,
 * no capacity (else MOE_ERR_UNSUPPORTED), any w_layout; same arguments without the fp8 scale
 * pointers, plus saved (NULL or too small: MOE_ERR_INVALID_ARG / MOE_ERR_WORKSPACE). y and
 * the optional outputs are bit-identical to moe_layer_forward's. Workspace:
 * moe_workspace_size(cfg, MOE_OP_LAYER_FORWARD).
 * moe_layer_backward_saved: moe_layer_backward with the buffer written by
 * moe_layer_forward_train for the same x, routing (topk_idx, topk_gate) and weights (the
 * backward's cfg may differ only in w_layout); every output is bit-identical to
 * moe_layer_backward's, and no GEMM1 is run. Workspace:
 * moe_workspace_size(cfg, MOE_OP_LAYER_BACKWARD). */
int moe_layer_forward_train(const moe_config* cfg, const void* x, const void* w_router,
                            const float* logit_bias, const float* sel_bias,
                            const float* logits_in, const void* w13, const void* w2,
                            const void* ws13, const void* ws2, void* y, float* logits_out,
                            int32_t* topk_idx_out, float* topk_gate_out, int32_t* counts_out,
                            void* saved, size_t saved_bytes, void* ws, size_t ws_bytes,
                            hipStream_t stream);
int moe_layer_backward_saved(const moe_config* cfg, const void* x, const void* w_router,
                             const float* logits, const float* logit_bias,
                             const int32_t* topk_idx, const float* topk_gate, const void* w13,
                             const void* w2, const void* ws13, const void* ws2,
                             const void* saved, size_t saved_bytes, const void* dy, void* dx,
                             void* dw_router, void* dw13, void* dw2, void* dws13, void* dws2,
                             float* dlogits_out, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/* Re-layout of n_mat row-major matrices [rows, cols] of elem_bytes-byte elements into the
 * K-blocked layout [n_mat][cols * elem_bytes / 64][rows][64 bytes] (see Layouts). A pure
 * data movement, for expert weights that are stored once and used by many calls; in and
 * out must not overlap. cols * elem_bytes must be a multiple of 64. */
int moe_pack_kblock(const void* in, int64_t n_mat, int32_t rows, int32_t cols,
                    int32_t elem_bytes, void* out, hipStream_t stream);

/* e4m3 block quantisation of n_mat matrices [rows, cols] (bf16 or fp32 input):
 * one fp32 scale per block_rows x block_cols block, s = fp32(amax / 448) (1 for an
 * all-zero block), q = e4m3_rne_saturate(fp32(v / s)) in the OCP E4M3 format.
 * block_rows is 1 (activations) or 128 (weights); block_cols is 128; rows and cols must be
 * multiples of the block. q [n_mat, rows, cols] uint8, scales
 * [n_mat, rows/block_rows, cols/128] fp32. (FP8 E4M3 for expert GEMMs: "万亿参数MoE模型
 * 训练的技术挑战", section 2.1.) */
int moe_quantize_e4m3(const void* in, int32_t in_dtype, int64_t n_mat, int32_t rows,
                      int32_t cols, int32_t block_rows, int32_t block_cols, uint8_t* q,
                      float* scales, hipStream_t stream);

/* MXFP8 quantisation (see MOE_MXFP8) of a row-major [rows, cols] matrix (bf16 or fp32
 * input; stacked weights [E, N, K] pass rows = E * N): 32-value blocks along each row.
 * q [rows, cols] uint8 e4m3 codes, scales [rows, cols/32] E8M0 bytes. cols must be a
 * multiple of 32. (MXFP8 recipe: "使用 Megatron Core 大规模训练混合专家模型（MoE）",
 * section 3.) */
int moe_quantize_mx(const void* in, int32_t in_dtype, int64_t rows, int32_t cols, uint8_t* q,
                    uint8_t* scales, hipStream_t stream);

/* Re-layout of MXFP8 weight scales for K-blocked weights: n_mat matrices of E8M0 bytes
 * [rows, cols] (cols = K/32, a multiple of 4) -> [n_mat][cols/4][rows][4 bytes], i.e. the four
 * block codes of one row's 128 K form a word and the words of consecutive rows are adjacent,
 * so that a GEMM tile's scales for one 128-K step are one contiguous run. Weights in
 * MOE_LAYOUT_KBLOCK (cfg->w_layout) take their MXFP8 scales in this order; in and out must
 * not overlap. A pure data movement, run once per weight set. */
int moe_pack_mx_scales(const uint8_t* in, int64_t n_mat, int32_t rows, int32_t cols,
                       uint8_t* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_AMD_H */

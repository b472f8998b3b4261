// Internal launch interface between the C ABI (api.cpp) and the kernel files.
// Every launcher enqueues on `stream`, performs no validation (the ABI has done it) and
// returns hipGetLastError() of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---- router ----------------------------------------------------------------------------
hipError_t launch_router_logits(int act_dtype, const void* x, const void* w_router, int T,
                                int H, int E, float* logits, hipStream_t s);

// bf16 router scores as a split-K MFMA GEMM (grouped_gemm.hip). router_gemm_ksplit gives the
// number of K ranges to use with scratch_bytes of partial-sum space (1: no partials, the
// kernel writes logits directly; 0: the shape is not supported, use launch_router_logits).
// part holds ksplit * T * E floats when ksplit > 1.
int router_gemm_ksplit(int T, int H, int E, size_t scratch_bytes);
hipError_t launch_router_gemm(const void* x, const void* w_router, int T, int H, int E,
                              int ksplit, float* part, float* logits, hipStream_t s);

hipError_t launch_route(int router, const float* logits, const float* logit_bias,
                        const float* sel_bias, int T, int E, int k, int n_groups,
                        int topk_groups, float route_scale, int32_t* topk_idx,
                        float* topk_gate, hipStream_t s);

// launch_route plus the load-balancing statistics: prob_mean[e] = (1/T) sum_t p[t, e] with p
// the router's normalised probabilities (softmax router: softmax of l over all E; sigmoid
// router: s / sum s), per-block sums reduced in a fixed order. Workspace:
// route_stats_ws_bytes(T, E).
size_t route_stats_ws_bytes(int T, int E);
hipError_t launch_route_stats(int router, const float* logits, const float* logit_bias,
                              const float* sel_bias, int T, int E, int k, int n_groups,
                              int topk_groups, float route_scale, int32_t* topk_idx,
                              float* topk_gate, float* prob_mean, void* ws, hipStream_t s);

// gates -> logits: dl [T, E] (bf16, and fp32 when dl_f32 != nullptr) from the gates'
// gradient in expert-grouped order (dgate_perm [T*k], read through pos)
hipError_t launch_route_backward(int router, const float* logits, const float* logit_bias,
                                 const int32_t* topk_idx, const float* topk_gate,
                                 const float* dgate_perm, const int32_t* pos, int T, int E,
                                 int k, float route_scale, uint16_t* dl_bf16, float* dl_f32,
                                 hipStream_t s);

// ---- permute ---------------------------------------------------------------------------
constexpr int kPermChunk = 512;   // assignments per counting block
size_t permute_ws_bytes(int T, int k, int E);
// With mode 3 and kblock -1 (the layer's MXFP8 path) x_q_scales are written blocked
// ([H/128][T][4]) and, when x_perm_scales != nullptr, gathered into expert order there (blocked
// [H/128][A][4], rows [0, offsets[E])).
hipError_t launch_permute(int mode /*0 f32, 1 bf16, 2 e4m3 from bf16, 3 MXFP8 from bf16*/,
                          int kblock /*1: x_perm K-blocked (not with MXFP8); -1: no x_perm
                                       (routing metadata, and in the fp8 modes the token-order
                                       x_q, only)*/,
                          int cap /*expert capacity: assignments of rank >= cap within their
                                    expert (token order) are dropped, pos = -1; INT_MAX =
                                    dropless*/,
                          const void* x,
                          const int32_t* topk_idx, const float* topk_gate, int T, int H,
                          int E, int k, int32_t* counts, int32_t* offsets, int32_t* pos,
                          int32_t* src, float* gate_perm, void* x_perm,
                          void* x_perm_scales, void* x_q, void* x_q_scales, void* ws,
                          hipStream_t s);

// ---- combine ---------------------------------------------------------------------------
hipError_t launch_combine(int act_dtype, const void* y_perm, const int32_t* pos,
                          const void* shared_y, int T, int H, int k, void* y, hipStream_t s);

// y += a over n bf16 values (n % 8 == 0), fp32 sum, one rounding
hipError_t launch_add_bf16(void* y, const void* a, int64_t n, hipStream_t s);

// ---- K-blocked re-layout: [n, rows, cols] -> [n][cols*eb/64][rows][64 bytes] ------------
hipError_t launch_pack_kblock(const void* in, int64_t n_mat, int rows, int cols, int elem_bytes,
                              void* out, hipStream_t s);

// ---- quantise --------------------------------------------------------------------------
hipError_t launch_quantize(const void* in, int in_dtype, int64_t n_mat, int rows, int cols,
                           int block_rows, uint8_t* q, float* scales, hipStream_t s);
// MXFP8: a row-major [rows, cols] matrix (cols % 32 == 0) in 1 x 32 blocks along the rows ->
// e4m3 codes q and one E8M0 code per block, row-major [rows, cols/32] or, with blocked (cols
// % 128 == 0), in the blocked scale order [cols/128][rows][4 bytes]
hipError_t launch_quantize_mx(const void* in, int in_dtype, int64_t rows, int cols,
                              int blocked, uint8_t* q, uint8_t* scales, hipStream_t s);
// MXFP8 scale bytes [n, rows, cols] (cols % 4 == 0) -> blocked [n][cols/4][rows][4 bytes]
hipError_t launch_pack_mx_scales(const uint8_t* in, int64_t n_mat, int rows, int cols,
                                 uint8_t* out, hipStream_t s);

// ---- grouped GEMM ----------------------------------------------------------------------
// One expert segment of a grouped GEMM launch: `groups` groups whose rows are
// [offsets[g], offsets[g+1]) of `a` (offsets == nullptr: one group of `rows` rows).
struct Segment {
    const void* a;             // [rows_total, K] activations (dtype of the launch)
    const void* a_scales;      // e4m3: fp32 [rows_total, K/128]; MXFP8: E8M0 [rows_total, K/32]
    const int32_t* offsets;    // [groups+1] device, or nullptr
    int groups;
    int rows;                  // rows when offsets == nullptr
    const float* gate;         // per-row gate (GEMM1 fold), nullptr = 1
    const void* w;             // [groups, N, K]
    const void* w_scales;      // e4m3: fp32 [groups, N/128, K/128]; MXFP8: E8M0 [groups, N, K/32]
    void* out;                 // GEMM1: act [rows, N/2]; GEMM2: y [rows, N]
    void* out_scales;          // GEMM1 act scales: e4m3 fp32 [rows, N/2/128]; MXFP8 E8M0
                               // [rows, N/2/32]
    void* z_out;               // GEMM1 optional: Z [rows, N] in the activation dtype
    int rows_total;            // rows of `a` (and of `out`)
    int a_kblock;              // 1: `a` is K-blocked ([K*eb/64][rows_total][64 bytes])
    int w_kblock;              // 1: each group's [N, K] weight is K-blocked
    int out_kblock;            // 1: GEMM1's `out` (act) is K-blocked
    const int32_t* a_rows;     // nullptr, or: row r reads row a_rows[r] of a row-major `a`
                               // (and of a_scales): the permutation fused into the A loads
    // MXFP8 scale layouts (0 = row-major [rows, K/32] bytes; 1 = blocked [K/128][rows][4])
    int a_sc_blocked;          // a_scales blocked, with a_sc_rows rows
    int a_sc_rows;
    int a_sc_direct;           // 1: a_scales row r belongs to launch row r even when a_rows
                               //    gathers the codes (scales permuted beforehand)
    int w_sc_blocked;          // each group's w_scales blocked ([K/128][N][4])
    int out_sc_blocked;        // GEMM1's out_scales blocked, rows_total rows
};

struct GemmPlan {
    int bm;                    // M tile of the chosen kernel
    size_t ws_bytes;           // tile-schedule workspace
};

// kind: 0 = GEMM1 (gate/up + SwiGLU * gate), 1 = GEMM2 (plain).  dtype: moe_dtype of the
// operands (F32, BF16, E4M3, MXFP8; MXFP8 needs row-major scales, K % 128 == 0 and for
// GEMM1 N % 256 == 0). N = output columns of the GEMM before the SwiGLU pairing.
// Tile list of one segment (groups with device-resident row offsets) for M tiles of `bm`
// rows, written to ws: *(int*)ws = count, (int4*)(ws + 256) = {group, first row, rows,
// group's first global row}.
hipError_t launch_schedule(const int32_t* offsets, int groups, int bm, void* ws, hipStream_t s);
size_t schedule_ws_bytes(int max_rows, int groups, int bm);

// ---- grouped GEMM backward (bf16) ----------------------------------------------------
size_t bwd_ws_bytes(int T, int k, int E, int H, int F);
// The weight gradients run on the library's side streams; join = false leaves them unjoined
// for a caller that joins once after several launches (bwd_side_join), holding
// bwd_side_lock() .. bwd_side_unlock() around the whole sequence. w_kblock: w13 and w2 are
// K-blocked per expert (the forward's weight layout), else row-major. use_side = false runs
// every launch on s (no side streams, nothing to join).
// Rows of x [T, row_bytes] to their expert-order positions (pos [T * k], from
// launch_permute; row-major out, row_bytes a multiple of 16): the permute's row copy alone.
hipError_t launch_gather_rows(const void* x, const int32_t* pos, int T, int k, int row_bytes,
                              void* out, hipStream_t s);
// Expert-order copies left to the backward (the permute's pos and src; nullptr = the caller
// filled that buffer): x (-> x_perm, gathered on dW13's stream while dA runs) and dY
// (-> dy_perm, gathered on dW2's stream; dA then reads dY's rows through src).
struct BwdGather {
    const void* x;
    const void* dy;
    const int32_t* pos;
    const int32_t* src;
    int T, k;
};
hipError_t launch_grouped_gemm_bwd(const void* dy_perm, const void* x_perm, const void* z,
                                   const void* act, const float* gate_perm,
                                   const int32_t* offsets, const void* w13, const void* w2,
                                   int A, int E, int H, int F, void* dx_perm, void* dw13,
                                   void* dw2, float* dgate_perm, void* ws, hipStream_t s,
                                   bool join = true, bool w_kblock = false,
                                   bool use_side = true, const BwdGather* gx = nullptr);
hipError_t bwd_side_join(hipStream_t s);
void bwd_side_lock();
void bwd_side_unlock();

// offsets {0, T} of a single group of T rows
hipError_t launch_offsets2(int32_t* offs, int T, hipStream_t s);

// Router backward GEMMs (bf16): dW_r = dl^T x [E, H] and dx_r = dl W_r [T, H] from
// dl [T, E]; E and H multiples of 128. Workspace: router_bwd_ws_bytes(T).
size_t router_bwd_ws_bytes(int T);
hipError_t launch_router_bwd(const void* dl, const void* x, const void* w_router, int T, int E,
                             int H, void* dw_router, void* dx_router, void* ws, hipStream_t s);

GemmPlan grouped_gemm_plan(int kind, int dtype, int max_rows_total, int groups_total, int N,
                           int K);
hipError_t launch_grouped_gemm(int kind, int dtype, const Segment* segs, int nseg,
                               int max_rows_total, int N, int K, void* ws, hipStream_t s);

}  // namespace moe

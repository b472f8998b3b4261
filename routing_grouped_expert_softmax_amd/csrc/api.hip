// C ABI of the MoE-layer forward: host-side validation, workspace carving, launches.
// Every entry point validates before it enqueues anything, never allocates device memory,
// never synchronises and never copies device -> host.
#include <limits.h>
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/moe.h"
#include "kernels.h"

// Layout of the layer's internal activations (x_perm, act): row-major (0) measured as fast
// in the grouped GEMMs as K-blocked (1) and makes the permute a one-read, k-write scatter.
#ifndef MOE_LAYER_ACT_KBLOCK
#define MOE_LAYER_ACT_KBLOCK 0
#endif
#ifndef MOE_LAYER_FUSED_GATHER
#define MOE_LAYER_FUSED_GATHER 1
#endif

namespace {

using moe::Segment;

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

size_t elem_bytes(int dtype) { return dtype == MOE_F32 ? 4 : dtype == MOE_BF16 ? 2 : 1; }

// fp8 expert operands: e4m3 with fp32 block scales, or MXFP8 with E8M0 block scales
bool is_fp8(int w_dtype) { return w_dtype == MOE_E4M3 || w_dtype == MOE_MXFP8; }

// Bytes of the block scales of a [rows, cols] fp8 activation: fp32 per 1 x 128 (e4m3) or one
// E8M0 byte per 1 x 32 (MXFP8)
size_t act_scale_bytes(int w_dtype, size_t rows, size_t cols) {
    return w_dtype == MOE_MXFP8 ? rows * (cols / 32) : rows * (cols / 128) * 4;
}

// Validation of the configuration itself (shapes and numerics).
int check_cfg(const moe_config* c) {
    if (!c) return MOE_ERR_INVALID_ARG;
    if (c->T < 1 || c->H < 1 || c->E < 1 || c->k < 1 || c->F < 1 || c->shared_F < 0)
        return MOE_ERR_INVALID_ARG;
    if (c->k > c->E) return MOE_ERR_INVALID_ARG;
    if (c->E > 1024 || c->k > 32) return MOE_ERR_UNSUPPORTED;
    if ((int64_t)c->T * c->k > (int64_t)1 << 30) return MOE_ERR_UNSUPPORTED;
    if (c->router == MOE_ROUTER_SOFTMAX_TOPK) {
        if (c->n_groups != 1 || c->topk_groups != 1) return MOE_ERR_INVALID_ARG;
    } else if (c->router == MOE_ROUTER_SIGMOID_GROUP_TOPK) {
        if (c->n_groups < 1 || c->topk_groups < 1 || c->topk_groups > c->n_groups)
            return MOE_ERR_INVALID_ARG;
        if (c->E % c->n_groups != 0) return MOE_ERR_INVALID_ARG;
        int per = c->E / c->n_groups;
        if (per < 2 || per * c->topk_groups < c->k) return MOE_ERR_INVALID_ARG;
        if (c->n_groups > 64) return MOE_ERR_UNSUPPORTED;
    } else {
        return MOE_ERR_INVALID_ARG;
    }
    if (!(c->route_scale > 0.0f) || c->route_scale != c->route_scale) return MOE_ERR_INVALID_ARG;
    if (!(c->capacity_factor >= 0.0f) || !isfinite(c->capacity_factor)) return MOE_ERR_INVALID_ARG;
    if ((c->a_layout != MOE_LAYOUT_ROWS && c->a_layout != MOE_LAYOUT_KBLOCK) ||
        (c->w_layout != MOE_LAYOUT_ROWS && c->w_layout != MOE_LAYOUT_KBLOCK))
        return MOE_ERR_INVALID_ARG;
    if (c->act_dtype == MOE_F32 && (c->a_layout || c->w_layout)) return MOE_ERR_UNSUPPORTED;
    if (c->act_dtype == MOE_F32) {
        if (c->w_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
        if (c->H % 64 || c->F % 32 || (c->shared_F && c->shared_F % 32)) return MOE_ERR_UNSUPPORTED;
    } else if (c->act_dtype == MOE_BF16) {
        if (c->w_dtype != MOE_BF16 && !is_fp8(c->w_dtype)) return MOE_ERR_UNSUPPORTED;
        if (c->w_dtype == MOE_MXFP8 && c->a_layout) return MOE_ERR_UNSUPPORTED;
        if (c->H % 256 || c->F % 128 || (c->shared_F && c->shared_F % 128))
            return MOE_ERR_UNSUPPORTED;
        // the fp8 GEMMs address their one-byte activation rows with 32-bit offsets from the
        // activation base: every fp8 activation matrix (x_perm / act with T*k rows, x_q /
        // the shared act with T rows) must stay below 4 GiB
        if (is_fp8(c->w_dtype)) {
            const int64_t rows = (int64_t)c->T * c->k + c->T;
            int64_t width = c->H > c->F ? c->H : c->F;
            if (c->shared_F > width) width = c->shared_F;
            if (rows * width >= ((int64_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
        }
    } else {
        return MOE_ERR_INVALID_ARG;
    }
    return MOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Expert capacity in assignments: ceil(capacity_factor * T * k / E), evaluated in double;
// INT_MAX when capacity_factor == 0 (dropless).
int capacity_of(const moe_config* c) {
    if (c->capacity_factor == 0.0f) return INT_MAX;
    const double cap = ceil((double)c->capacity_factor * ((double)c->T * (double)c->k) / (double)c->E);
    return cap >= (double)c->T * c->k ? c->T * c->k : (int)cap;
}

// Stage events of moe_layer_forward (instrumentation): per host thread, caller-owned handles.
thread_local hipEvent_t g_stage_ev[MOE_N_STAGE_EVENTS];
thread_local bool g_stage_on = false;

hipError_t stage_mark(int i, hipStream_t s) {
    return g_stage_on ? hipEventRecord(g_stage_ev[i], s) : hipSuccess;
}

// ---- workspace layouts -------------------------------------------------------------------
struct Carve {
    char* base;
    size_t off = 0;
    explicit Carve(void* p) : base((char*)p) {}
    void* take(size_t bytes) {
        void* p = base ? base + off : nullptr;
        off += align_up(bytes);
        return p;
    }
};

size_t sched_ws_bytes(const moe_config* c);

size_t gemm_ws_bytes(const moe_config* c) {
    size_t shared = 0;
    if (c->shared_F) {
        const bool q8 = is_fp8(c->w_dtype);
        const size_t eb = q8 ? 1 : elem_bytes(c->act_dtype);
        shared += align_up((size_t)c->T * c->shared_F * eb);                // shared act
        if (q8) shared += align_up(act_scale_bytes(c->w_dtype, c->T, c->shared_F));   // scales
    }
    return align_up(sched_ws_bytes(c)) + shared;
}

struct LayerWs {
    float* logits;
    int32_t* idx;
    float* gate;
    int32_t* counts;
    int32_t* offsets;
    int32_t* pos;
    int32_t* src;
    float* gate_perm;
    void* x_perm;
    void* x_perm_scales;
    void* x_q;
    void* x_q_scales;
    void* act;
    void* act_scales;
    void* y_perm;
    void* shared_y;
    void* scratch;       // permute / grouped-GEMM scratch (used one after the other)
    size_t total;
};

LayerWs carve_layer(const moe_config* c, void* ws) {
    LayerWs L = {};
    Carve cv(ws);
    const size_t T = c->T, H = c->H, E = c->E, k = c->k, F = c->F, A = T * k;
    const bool fp8 = is_fp8(c->w_dtype);
    const int wd = c->w_dtype;
    const size_t ab = elem_bytes(c->act_dtype);
    const size_t gb = fp8 ? 1 : ab;       // GEMM operand bytes
    L.logits = (float*)cv.take(T * E * 4);
    L.idx = (int32_t*)cv.take(A * 4);
    L.gate = (float*)cv.take(A * 4);
    L.counts = (int32_t*)cv.take(E * 4);
    L.offsets = (int32_t*)cv.take((E + 1) * 4);
    L.pos = (int32_t*)cv.take(A * 4);
    L.src = (int32_t*)cv.take(A * 4);
    L.gate_perm = (float*)cv.take(A * 4);
    L.x_perm = cv.take(A * H * gb);
    L.x_perm_scales = fp8 ? cv.take(act_scale_bytes(wd, A, H)) : nullptr;
    L.x_q = fp8 ? cv.take(T * H) : nullptr;                // token-order fp8 x (the
    L.x_q_scales = fp8 ? cv.take(act_scale_bytes(wd, T, H)) : nullptr;   // gather's source)
    L.act = cv.take(A * F * gb);
    L.act_scales = fp8 ? cv.take(act_scale_bytes(wd, A, F)) : nullptr;
    L.y_perm = cv.take(A * H * ab);
    L.shared_y = c->shared_F ? cv.take(T * H * ab) : nullptr;
    size_t p = moe::permute_ws_bytes(c->T, c->k, c->E);
    size_t g = gemm_ws_bytes(c);
    L.scratch = cv.take(p > g ? p : g);
    L.total = cv.off;
    return L;
}

// Workspace of the whole-layer backward: the routing metadata, the expert-grouped x and dY,
// the recomputed Z and act (routed and shared), the data gradients before they are
// combined, dl, and the scratch of every launch.
struct LayerBwdWs {
    int32_t *counts, *offsets, *pos, *src, *offs_one;
    float *gate_perm, *dgate_perm;
    void *x_perm, *dy_perm, *z, *act, *zs, *acts, *dx_perm, *dxs, *dxr, *dl;
    void *perm_scratch, *sched, *bws, *bws_s, *rws;
    size_t total;
};

size_t sched_ws_bytes(const moe_config* c);

LayerBwdWs carve_layer_bwd(const moe_config* c, void* ws) {
    LayerBwdWs L = {};
    Carve cv(ws);
    const size_t T = c->T, H = c->H, E = c->E, k = c->k, F = c->F, sF = c->shared_F, A = T * k;
    L.counts = (int32_t*)cv.take(E * 4);
    L.offsets = (int32_t*)cv.take((E + 1) * 4);
    L.pos = (int32_t*)cv.take(A * 4);
    L.src = (int32_t*)cv.take(A * 4);
    L.gate_perm = (float*)cv.take(A * 4);
    L.offs_one = (int32_t*)cv.take(2 * 4);
    L.dgate_perm = (float*)cv.take(A * 4);
    L.x_perm = cv.take(A * H * 2);
    L.dy_perm = cv.take(A * H * 2);
    L.z = cv.take(A * 2 * F * 2);
    L.act = cv.take(A * F * 2);
    L.zs = sF ? cv.take(T * 2 * sF * 2) : nullptr;
    L.acts = sF ? cv.take(T * sF * 2) : nullptr;
    L.dx_perm = cv.take(A * H * 2);
    L.dxs = sF ? cv.take(T * H * 2) : nullptr;
    L.dxr = cv.take(T * H * 2);
    L.dl = cv.take(T * E * 2);
    L.perm_scratch = cv.take(moe::permute_ws_bytes(c->T, c->k, c->E));
    L.sched = cv.take(sched_ws_bytes(c));
    L.bws = cv.take(moe::bwd_ws_bytes(c->T, c->k, c->E, c->H, c->F));
    L.bws_s = sF ? cv.take(moe::bwd_ws_bytes(c->T, 1, 1, c->H, c->shared_F)) : nullptr;
    L.rws = cv.take(moe::router_bwd_ws_bytes(c->T));
    L.total = cv.off;
    return L;
}

int check_layer_bwd(const moe_config* c) {
    if (c->act_dtype != MOE_BF16 || c->w_dtype != MOE_BF16 || c->a_layout)
        return MOE_ERR_UNSUPPORTED;
    if (c->capacity_factor != 0.0f) return MOE_ERR_UNSUPPORTED;     // dropless only
    if (c->E % 128) return MOE_ERR_UNSUPPORTED;          // router GEMM tiles
    return MOE_OK;
}

// The GEMM1 outputs a training forward keeps for the backward: Z and act of the routed rows
// (expert order) and of the shared expert, bf16 row-major.
struct SavedActs {
    void *z, *act, *zs, *acts;
    size_t total;
};

SavedActs carve_saved(const moe_config* c, void* p) {
    SavedActs S = {};
    Carve cv(p);
    const size_t T = c->T, F = c->F, sF = c->shared_F, A = T * c->k;
    S.z = cv.take(A * 2 * F * 2);
    S.act = cv.take(A * F * 2);
    S.zs = sF ? cv.take(T * 2 * sF * 2) : nullptr;
    S.acts = sF ? cv.take(T * sF * 2) : nullptr;
    S.total = cv.off;
    return S;
}

// A forward that saves its activations runs the bf16 layer without dropping (the backward's
// conditions, any weight layout).
int check_saved(const moe_config* c) {
    if (c->act_dtype != MOE_BF16 || c->w_dtype != MOE_BF16 || c->a_layout)
        return MOE_ERR_UNSUPPORTED;
    if (c->capacity_factor != 0.0f) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

size_t sched_ws_bytes(const moe_config* c) {
    const int dt = c->w_dtype;
    const int seg_groups = c->E + (c->shared_F ? 1 : 0);
    const int rows = c->T * c->k + (c->shared_F ? c->T : 0);
    size_t s1 = moe::grouped_gemm_plan(0, dt, rows, seg_groups, 2 * c->F, c->H).ws_bytes;
    size_t s2 = moe::grouped_gemm_plan(1, dt, rows, seg_groups, c->H, c->F).ws_bytes;
    return s1 > s2 ? s1 : s2;
}

// GEMM1 of the experts (gate/up projection + SwiGLU with the gate folded in): routed
// experts as segment 0 and, when shared_F == F, the shared expert as segment 1 of the same
// launch; a shared expert of another width gets its own launch.
int run_up(const moe_config* c, int a_kb, const void* x_perm, const void* x_perm_scales,
           const int32_t* offsets, const float* gate_perm, const void* w13,
           const void* w13_scales, const void* x_shared, const void* x_shared_scales,
           const void* ws13, const void* ws13_scales, void* act, void* act_scales,
           void* shared_act, void* shared_act_scales, void* z_out, void* sched,
           hipStream_t stream, const int32_t* a_rows = nullptr, bool mx_blocked = false,
           void* shared_z_out = nullptr) {
    const int dt = c->w_dtype;
    const int A = c->T * c->k;
    Segment r1 = {x_perm, x_perm_scales, offsets, c->E, 0, gate_perm, w13, w13_scales,
                  act, act_scales, z_out, A, a_kb, c->w_layout, a_kb, a_rows};
    Segment s1 = {x_shared, x_shared_scales, nullptr, 1, c->T, nullptr, ws13, ws13_scales,
                  shared_act, shared_act_scales, shared_z_out, c->T, 0, c->w_layout, a_kb};
    if (dt == MOE_MXFP8) {
        // K-blocked weights carry blocked scales; the layer keeps its activation scales
        // blocked too, the routed ones already in expert order
        r1.w_sc_blocked = s1.w_sc_blocked = c->w_layout;
        if (mx_blocked) {
            r1.a_sc_blocked = 1; r1.a_sc_rows = A; r1.a_sc_direct = 1; r1.out_sc_blocked = 1;
            s1.a_sc_blocked = 1; s1.a_sc_rows = c->T; s1.out_sc_blocked = 1;
        }
    }
    if (!c->shared_F)
        return hip_status(moe::launch_grouped_gemm(0, dt, &r1, 1, A, 2 * c->F, c->H, sched, stream));
    if (c->shared_F == c->F) {
        Segment g[2] = {r1, s1};
        return hip_status(moe::launch_grouped_gemm(0, dt, g, 2, A + c->T, 2 * c->F, c->H, sched,
                                                   stream));
    }
    hipError_t e = moe::launch_grouped_gemm(0, dt, &r1, 1, A, 2 * c->F, c->H, sched, stream);
    if (e == hipSuccess)
        e = moe::launch_grouped_gemm(0, dt, &s1, 1, c->T, 2 * c->shared_F, c->H, sched, stream);
    return hip_status(e);
}

// GEMM2 of the experts (down projection), same segment layout as run_up.
int run_down(const moe_config* c, int a_kb, const void* act, const void* act_scales,
             const int32_t* offsets, const void* w2, const void* w2_scales,
             const void* shared_act, const void* shared_act_scales, const void* ws2,
             const void* ws2_scales, void* y_perm, void* shared_y, void* sched,
             hipStream_t stream, bool mx_blocked = false) {
    const int dt = c->w_dtype;
    const int A = c->T * c->k;
    Segment r2 = {act, act_scales, offsets, c->E, 0, nullptr, w2, w2_scales, y_perm, nullptr,
                  nullptr, A, a_kb, c->w_layout, 0};
    Segment s2 = {shared_act, shared_act_scales, nullptr, 1, c->T, nullptr, ws2, ws2_scales,
                  shared_y, nullptr, nullptr, c->T, a_kb, c->w_layout, 0};
    if (dt == MOE_MXFP8) {
        r2.w_sc_blocked = s2.w_sc_blocked = c->w_layout;
        if (mx_blocked) {
            r2.a_sc_blocked = 1; r2.a_sc_rows = A;
            s2.a_sc_blocked = 1; s2.a_sc_rows = c->T;
        }
    }
    if (!c->shared_F)
        return hip_status(moe::launch_grouped_gemm(1, dt, &r2, 1, A, c->H, c->F, sched, stream));
    if (c->shared_F == c->F) {
        Segment g[2] = {r2, s2};
        return hip_status(moe::launch_grouped_gemm(1, dt, g, 2, A + c->T, c->H, c->F, sched,
                                                   stream));
    }
    hipError_t e = moe::launch_grouped_gemm(1, dt, &r2, 1, A, c->H, c->F, sched, stream);
    if (e == hipSuccess)
        e = moe::launch_grouped_gemm(1, dt, &s2, 1, c->T, c->H, c->shared_F, sched, stream);
    return hip_status(e);
}

// Both GEMMs; the shared expert's activation lives in the workspace after the schedule.
int run_experts(const moe_config* c, int a_kb, const void* x_perm, const void* x_perm_scales,
                const int32_t* offsets, const float* gate_perm, const void* w13,
                const void* w13_scales, const void* w2, const void* w2_scales,
                const void* x_shared, const void* x_shared_scales, const void* ws13,
                const void* ws13_scales, const void* ws2, const void* ws2_scales, void* act,
                void* act_scales, void* y_perm, void* shared_y, void* z_out, void* ws,
                hipStream_t stream, int mid_mark = -1, const int32_t* a_rows = nullptr,
                bool mx_blocked = false, void* shared_act_out = nullptr,
                void* shared_z_out = nullptr) {
    Carve cv(ws);
    void* sched = cv.take(sched_ws_bytes(c));
    void* sh_act = nullptr;
    void* sh_act_scales = nullptr;
    if (c->shared_F) {
        const bool fp8 = is_fp8(c->w_dtype);
        sh_act = cv.take((size_t)c->T * c->shared_F * (fp8 ? 1 : elem_bytes(c->act_dtype)));
        if (fp8) sh_act_scales = cv.take(act_scale_bytes(c->w_dtype, c->T, c->shared_F));
        if (shared_act_out) sh_act = shared_act_out;
    }
    int st = run_up(c, a_kb, x_perm, x_perm_scales, offsets, gate_perm, w13, w13_scales, x_shared,
                    x_shared_scales, ws13, ws13_scales, act, act_scales, sh_act, sh_act_scales,
                    z_out, sched, stream, a_rows, mx_blocked, shared_z_out);
    if (st) return st;
    if (mid_mark >= 0 && stage_mark(mid_mark, stream) != hipSuccess) return MOE_ERR_HIP;
    return run_down(c, a_kb, act, act_scales, offsets, w2, w2_scales, sh_act, sh_act_scales, ws2,
                    ws2_scales, y_perm, shared_y, sched, stream, mx_blocked);
}

// ---- the no-allocation permute's scratch -------------------------------------------------
// The per-chunk expert histograms of the permute (its only scratch) in a file-scope device
// array instead of the caller's workspace. Every GPU the library runs on holds its own copy
// until the process ends. In host code `scratch` is a host-side stand-in: its device address
// comes from hipGetSymbolAddress, looked up once per device with that device current, and
// only that address is handed to kernels.
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) int32_t scratch[kNoAllocScratchBytes / sizeof(int32_t)];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on the first call on a device).
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
    switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: unsupported shape or dtype";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP launch failed";
    default: return "unknown moe status";
    }
}

int moe_workspace_size(const moe_config* cfg, int op, size_t* bytes) {
    if (!bytes) return MOE_ERR_INVALID_ARG;
    int st = check_cfg(cfg);
    if (st) return st;
    switch (op) {
    case MOE_OP_PERMUTE: *bytes = moe::permute_ws_bytes(cfg->T, cfg->k, cfg->E); break;
    case MOE_OP_GROUPED_GEMM: *bytes = gemm_ws_bytes(cfg); break;
    case MOE_OP_LAYER_FORWARD: *bytes = carve_layer(cfg, nullptr).total; break;
    case MOE_OP_GROUPED_GEMM_BWD:
        if (cfg->act_dtype != MOE_BF16 || cfg->a_layout) return MOE_ERR_UNSUPPORTED;
        if (cfg->capacity_factor != 0.0f) return MOE_ERR_UNSUPPORTED;
        *bytes = moe::bwd_ws_bytes(cfg->T, cfg->k, cfg->E, cfg->H, cfg->F);
        break;
    case MOE_OP_ROUTE_STATS: *bytes = moe::route_stats_ws_bytes(cfg->T, cfg->E); break;
    case MOE_OP_LAYER_BACKWARD:
        st = check_layer_bwd(cfg);
        if (st) return st;
        *bytes = carve_layer_bwd(cfg, nullptr).total;
        break;
    case MOE_OP_LAYER_SAVED:
        st = check_saved(cfg);
        if (st) return st;
        *bytes = carve_saved(cfg, nullptr).total;
        break;
    default: return MOE_ERR_INVALID_ARG;
    }
    return MOE_OK;
}

int moe_router_logits(const moe_config* cfg, const void* x, const void* w_router,
                      float* logits, hipStream_t stream) {
    int st = check_cfg(cfg);
    if (st) return st;
    if (!x || !w_router || !logits) return MOE_ERR_INVALID_ARG;
    // bf16: the MFMA router GEMM without a K split (no partial-sum space here)
    if (cfg->act_dtype == MOE_BF16 && moe::router_gemm_ksplit(cfg->T, cfg->H, cfg->E, 0) == 1)
        return hip_status(moe::launch_router_gemm(x, w_router, cfg->T, cfg->H, cfg->E, 1,
                                                  nullptr, logits, stream));
    return hip_status(moe::launch_router_logits(cfg->act_dtype, x, w_router, cfg->T, cfg->H,
                                                cfg->E, logits, stream));
}

int moe_route(const moe_config* cfg, const float* logits, const float* logit_bias,
              const float* sel_bias, int32_t* topk_idx, float* topk_gate, hipStream_t stream) {
    int st = check_cfg(cfg);
    if (st) return st;
    if (!logits || !topk_idx || !topk_gate) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_route(cfg->router, logits, logit_bias, sel_bias, cfg->T,
                                        cfg->E, cfg->k, cfg->n_groups, cfg->topk_groups,
                                        cfg->route_scale, topk_idx, topk_gate, stream));
}

int moe_route_stats(const moe_config* cfg, const float* logits, const float* logit_bias,
                    const float* sel_bias, int32_t* topk_idx, float* topk_gate,
                    float* prob_mean, void* ws, size_t ws_bytes, hipStream_t stream) {
    int st = check_cfg(cfg);
    if (st) return st;
    if (!logits || !topk_idx || !topk_gate || !prob_mean || !ws) return MOE_ERR_INVALID_ARG;
    if (ws_bytes < moe::route_stats_ws_bytes(cfg->T, cfg->E)) return MOE_ERR_WORKSPACE;
    return hip_status(moe::launch_route_stats(cfg->router, logits, logit_bias, sel_bias, cfg->T,
                                              cfg->E, cfg->k, cfg->n_groups, cfg->topk_groups,
                                              cfg->route_scale, topk_idx, topk_gate, prob_mean,
                                              ws, stream));
}

int moe_permute(const moe_config* cfg, const void* x, const int32_t* topk_idx,
                const float* topk_gate, int32_t* counts, int32_t* offsets, int32_t* pos,
                int32_t* src, float* gate_perm, void* x_perm, void* x_perm_scales, void* x_q,
                void* x_q_scales, void* ws, size_t ws_bytes, hipStream_t stream) {
    int st = check_cfg(cfg);
    if (st) return st;
    if (!x || !topk_idx || !topk_gate || !counts || !offsets || !pos || !src || !gate_perm ||
        !x_perm || !ws)
        return MOE_ERR_INVALID_ARG;
    const bool fp8 = is_fp8(cfg->w_dtype);
    if (fp8 != (x_perm_scales != nullptr)) return MOE_ERR_INVALID_ARG;
    if (!fp8 && (x_q || x_q_scales)) return MOE_ERR_INVALID_ARG;
    if ((x_q == nullptr) != (x_q_scales == nullptr)) return MOE_ERR_INVALID_ARG;
    if (ws_bytes < moe::permute_ws_bytes(cfg->T, cfg->k, cfg->E)) return MOE_ERR_WORKSPACE;
    const int mode = cfg->w_dtype == MOE_MXFP8 ? 3 : fp8 ? 2 : (cfg->act_dtype == MOE_F32 ? 0 : 1);
    return hip_status(moe::launch_permute(mode, cfg->a_layout, capacity_of(cfg), x, topk_idx,
                                          topk_gate, cfg->T,
                                          cfg->H, cfg->E, cfg->k, counts, offsets, pos, src,
                                          gate_perm, x_perm, x_perm_scales, x_q, x_q_scales, ws,
                                          stream));
}

int moe_permute_noalloc(const moe_config* cfg, const void* x, const int32_t* topk_idx,
                        const float* topk_gate, int32_t* counts, int32_t* offsets,
                        int32_t* pos, int32_t* src, float* gate_perm, void* x_perm,
                        void* x_perm_scales, void* x_q, void* x_q_scales, hipStream_t stream) {
    int st = check_cfg(cfg);
    if (st) return st;
    if (!x || !topk_idx || !topk_gate || !counts || !offsets || !pos || !src || !gate_perm ||
        !x_perm)
        return MOE_ERR_INVALID_ARG;
    const bool fp8 = is_fp8(cfg->w_dtype);
    if (fp8 != (x_perm_scales != nullptr)) return MOE_ERR_INVALID_ARG;
    if (!fp8 && (x_q || x_q_scales)) return MOE_ERR_INVALID_ARG;
    if ((x_q == nullptr) != (x_q_scales == nullptr)) return MOE_ERR_INVALID_ARG;
    if (moe::permute_ws_bytes(cfg->T, cfg->k, cfg->E) > kNoAllocScratchBytes)
        return MOE_ERR_WORKSPACE;
    void* sp = nullptr;
    st = scratch_address(&sp);
    if (st) return st;
    const int mode = cfg->w_dtype == MOE_MXFP8 ? 3 : fp8 ? 2 : (cfg->act_dtype == MOE_F32 ? 0 : 1);
    return hip_status(moe::launch_permute(mode, cfg->a_layout, capacity_of(cfg), x, topk_idx,
                                          topk_gate, cfg->T, cfg->H, cfg->E, cfg->k, counts,
                                          offsets, pos, src, gate_perm, x_perm, x_perm_scales,
                                          x_q, x_q_scales, sp, stream));
}

int moe_grouped_gemm_swiglu(const moe_config* cfg, const void* x_perm,
                            const void* x_perm_scales, const int32_t* offsets,
                            const float* gate_perm, const void* w13, const void* w13_scales,
                            const void* w2, const void* w2_scales, const void* x_shared,
                            const void* x_shared_scales, const void* ws13,
                            const void* ws13_scales, const void* ws2,
                            const void* ws2_scales, void* act, void* act_scales,
                            void* y_perm, void* shared_y, void* z_out, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
    int st = check_cfg(cfg);
    if (st) return st;
    if (!x_perm || !offsets || !gate_perm || !w13 || !w2 || !act || !y_perm || !ws)
        return MOE_ERR_INVALID_ARG;
    const bool fp8 = is_fp8(cfg->w_dtype);
    if (fp8) {
        if (!x_perm_scales || !w13_scales || !w2_scales || !act_scales || z_out)
            return MOE_ERR_INVALID_ARG;
        if (cfg->shared_F && (!x_shared_scales || !ws13_scales || !ws2_scales))
            return MOE_ERR_INVALID_ARG;
        if (!cfg->shared_F && (x_shared_scales || ws13_scales || ws2_scales))
            return MOE_ERR_INVALID_ARG;
    } else if (x_perm_scales || w13_scales || w2_scales || act_scales || x_shared_scales ||
               ws13_scales || ws2_scales) {
        return MOE_ERR_INVALID_ARG;
    }
    if (cfg->shared_F) {
        if (!x_shared || !ws13 || !ws2 || !shared_y) return MOE_ERR_INVALID_ARG;
    } else if (x_shared || ws13 || ws2 || shared_y) {
        return MOE_ERR_INVALID_ARG;
    }
    if (ws_bytes < gemm_ws_bytes(cfg)) return MOE_ERR_WORKSPACE;
    return run_experts(cfg, cfg->a_layout, x_perm, x_perm_scales, offsets, gate_perm, w13, w13_scales, w2,
                       w2_scales, x_shared, x_shared_scales, ws13, ws13_scales, ws2,
                       ws2_scales, act, act_scales, y_perm, shared_y, z_out, ws, stream);
}

// Scale pointers of one GEMM half: required exactly in the fp8 modes (out_scales only when
// the half writes fp8, i.e. GEMM1's act).
static int check_gemm_dtypes(const moe_config* cfg, bool e4m3_out, const void* a_scales,
                             const void* w_scales, const void* out_scales,
                             const void* sh_a_scales, const void* sh_w_scales,
                             const void* sh_out_scales) {
    if (is_fp8(cfg->w_dtype)) {
        if (!a_scales || !w_scales) return MOE_ERR_INVALID_ARG;
        if (e4m3_out != (out_scales != nullptr)) return MOE_ERR_INVALID_ARG;
        if (cfg->shared_F && (!sh_a_scales || !sh_w_scales)) return MOE_ERR_INVALID_ARG;
        if (cfg->shared_F && e4m3_out != (sh_out_scales != nullptr)) return MOE_ERR_INVALID_ARG;
        if (!cfg->shared_F && (sh_a_scales || sh_w_scales || sh_out_scales))
            return MOE_ERR_INVALID_ARG;
        return MOE_OK;
    }
    if (a_scales || w_scales || out_scales || sh_a_scales || sh_w_scales || sh_out_scales)
        return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

int moe_grouped_gemm_up(const moe_config* cfg, const void* x_perm, const void* x_perm_scales,
                        const int32_t* offsets, const float* gate_perm, const void* w13,
                        const void* w13_scales, const void* x_shared,
                        const void* x_shared_scales, const void* ws13,
                        const void* ws13_scales, void* act, void* act_scales,
                        void* shared_act, void* shared_act_scales, void* z_out, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
    int st = check_cfg(cfg);
    if (st) return st;
    if (!x_perm || !offsets || !gate_perm || !w13 || !act || !ws) return MOE_ERR_INVALID_ARG;
    if (cfg->shared_F) {
        if (!x_shared || !ws13 || !shared_act) return MOE_ERR_INVALID_ARG;
    } else if (x_shared || ws13 || shared_act) {
        return MOE_ERR_INVALID_ARG;
    }
    st = check_gemm_dtypes(cfg, true, x_perm_scales, w13_scales, act_scales, x_shared_scales,
                           ws13_scales, shared_act_scales);
    if (!st && is_fp8(cfg->w_dtype) && z_out) st = MOE_ERR_INVALID_ARG;
    if (st) return st;
    if (ws_bytes < sched_ws_bytes(cfg)) return MOE_ERR_WORKSPACE;
    return run_up(cfg, cfg->a_layout, x_perm, x_perm_scales, offsets, gate_perm, w13, w13_scales, x_shared,
                  x_shared_scales, ws13, ws13_scales, act, act_scales, shared_act,
                  shared_act_scales, z_out, ws, stream);
}

int moe_grouped_gemm_down(const moe_config* cfg, const void* act, const void* act_scales,
                          const int32_t* offsets, const void* w2, const void* w2_scales,
                          const void* shared_act, const void* shared_act_scales,
                          const void* ws2, const void* ws2_scales, void* y_perm,
                          void* shared_y, void* ws, size_t ws_bytes, hipStream_t stream) {
    int st = check_cfg(cfg);
    if (st) return st;
    if (!act || !offsets || !w2 || !y_perm || !ws) return MOE_ERR_INVALID_ARG;
    if (cfg->shared_F) {
        if (!shared_act || !ws2 || !shared_y) return MOE_ERR_INVALID_ARG;
    } else if (shared_act || ws2 || shared_y) {
        return MOE_ERR_INVALID_ARG;
    }
    st = check_gemm_dtypes(cfg, false, act_scales, w2_scales, nullptr, shared_act_scales,
                           ws2_scales, nullptr);
    if (st) return st;
    if (ws_bytes < sched_ws_bytes(cfg)) return MOE_ERR_WORKSPACE;
    return run_down(cfg, cfg->a_layout, act, act_scales, offsets, w2, w2_scales, shared_act,
                    shared_act_scales, ws2, ws2_scales, y_perm, shared_y, ws, stream);
}

int moe_unpermute_combine(const moe_config* cfg, const void* y_perm, const int32_t* pos,
                          const void* shared_y, void* y, hipStream_t stream) {
    int st = check_cfg(cfg);
    if (st) return st;
    if (!y_perm || !pos || !y) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_combine(cfg->act_dtype, y_perm, pos, shared_y, cfg->T,
                                          cfg->H, cfg->k, y, stream));
}

// The layer forward; sv != NULL: GEMM1 writes act and Z (routed and shared) into the saved
// buffer instead of act alone into the workspace (moe_layer_forward_train).
static int layer_forward_impl(const moe_config* cfg, const void* x, const void* w_router,
                              const float* logit_bias, const float* sel_bias,
                              const float* logits_in, const void* w13, const void* w13_scales,
                              const void* w2, const void* w2_scales, const void* ws13,
                              const void* ws13_scales, const void* ws2, const void* ws2_scales,
                              void* y, float* logits_out, int32_t* topk_idx_out,
                              float* topk_gate_out, int32_t* counts_out, void* ws,
                              size_t ws_bytes, hipStream_t stream, const SavedActs* sv) {
    int st = check_cfg(cfg);
    if (st) return st;
    if (!x || !w13 || !w2 || !y || !ws) return MOE_ERR_INVALID_ARG;
    if (!logits_in && !w_router) return MOE_ERR_INVALID_ARG;
    const bool fp8 = is_fp8(cfg->w_dtype);
    if (fp8 && (!w13_scales || !w2_scales)) return MOE_ERR_INVALID_ARG;
    if (!fp8 && (w13_scales || w2_scales || ws13_scales || ws2_scales)) return MOE_ERR_INVALID_ARG;
    if (cfg->shared_F && (!ws13 || !ws2)) return MOE_ERR_INVALID_ARG;
    if (fp8 && cfg->shared_F && (!ws13_scales || !ws2_scales)) return MOE_ERR_INVALID_ARG;
    LayerWs L = carve_layer(cfg, nullptr);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    L = carve_layer(cfg, ws);
    float* logits = logits_out ? logits_out : L.logits;
    int32_t* idx = topk_idx_out ? topk_idx_out : L.idx;
    float* gate = topk_gate_out ? topk_gate_out : L.gate;
    int32_t* counts = counts_out ? counts_out : L.counts;
    hipError_t e = stage_mark(0, stream);
    const float* lg = logits_in;
    if (e == hipSuccess && lg && logits_out && logits_out != lg)
        e = hipMemcpyAsync(logits_out, lg, (size_t)cfg->T * cfg->E * 4, hipMemcpyDeviceToDevice,
                           stream);
    if (e == hipSuccess && !lg) {
        // bf16: split-K MFMA GEMM whose partial sums borrow the y_perm region (unused until
        // the down projection)
        const size_t yp_bytes = (size_t)cfg->T * cfg->k * cfg->H * elem_bytes(cfg->act_dtype);
        const int ks = cfg->act_dtype == MOE_BF16
                           ? moe::router_gemm_ksplit(cfg->T, cfg->H, cfg->E, yp_bytes)
                           : 0;
        if (ks > 0)
            e = moe::launch_router_gemm(x, w_router, cfg->T, cfg->H, cfg->E, ks,
                                        (float*)L.y_perm, logits, stream);
        else
            e = moe::launch_router_logits(cfg->act_dtype, x, w_router, cfg->T, cfg->H,
                                          cfg->E, logits, stream);
        lg = logits;
    }
    if (e == hipSuccess) e = stage_mark(1, stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
    e = moe::launch_route(cfg->router, lg, logit_bias, sel_bias, cfg->T, cfg->E, cfg->k,
                          cfg->n_groups, cfg->topk_groups, cfg->route_scale, idx, gate, stream);
    if (e == hipSuccess) e = stage_mark(2, stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
    const int mode = cfg->w_dtype == MOE_MXFP8 ? 3 : fp8 ? 2 : (cfg->act_dtype == MOE_F32 ? 0 : 1);
    // layout of the internal activations (x_perm, act, the shared expert's act)
    const int a_kb = cfg->act_dtype == MOE_F32 ? 0 : MOE_LAYER_ACT_KBLOCK;
    // bf16 / fp8 with row-major activations: no x_perm copy; GEMM1 gathers its A rows
    // straight from x (fp8: from the token-order codes x_q and their scales) through src
    const bool gather = MOE_LAYER_FUSED_GATHER && cfg->act_dtype != MOE_F32 && a_kb == 0;
    e = moe::launch_permute(mode, gather ? -1 : a_kb, capacity_of(cfg), x, idx, gate, cfg->T,
                            cfg->H, cfg->E,
                            cfg->k, counts, L.offsets, L.pos, L.src, L.gate_perm, L.x_perm,
                            L.x_perm_scales, L.x_q, L.x_q_scales, L.scratch, stream);
    if (e == hipSuccess) e = stage_mark(3, stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
    const void* xs = fp8 ? L.x_q : x;
    const void* a1 = gather ? xs : L.x_perm;
    // MXFP8: scales blocked throughout, the routed rows' scales permuted to expert order by
    // the permute (so a tile's scale words are adjacent); the codes are gathered from x_q
    const bool mx = cfg->w_dtype == MOE_MXFP8;
    const void* a1_scales = gather && !mx ? (fp8 ? L.x_q_scales : nullptr) : L.x_perm_scales;
    st = run_experts(cfg, a_kb, a1, a1_scales, L.offsets, L.gate_perm, w13, w13_scales,
                     w2, w2_scales, cfg->shared_F ? xs : nullptr, fp8 ? L.x_q_scales : nullptr,
                     ws13, ws13_scales, ws2, ws2_scales, sv ? sv->act : L.act, L.act_scales,
                     L.y_perm, L.shared_y, sv ? sv->z : nullptr, L.scratch, stream, 4,
                     gather ? L.src : nullptr, mx, sv ? sv->acts : nullptr,
                     sv ? sv->zs : nullptr);
    if (st) return st;
    e = stage_mark(5, stream);
    if (e == hipSuccess)
        e = moe::launch_combine(cfg->act_dtype, L.y_perm, L.pos, L.shared_y, cfg->T, cfg->H,
                                cfg->k, y, stream);
    if (e == hipSuccess) e = stage_mark(6, stream);
    return hip_status(e);
}

int moe_layer_forward(const moe_config* cfg, const void* x, const void* w_router,
                      const float* logit_bias, const float* sel_bias, const float* logits_in,
                      const void* w13, const void* w13_scales, const void* w2,
                      const void* w2_scales, const void* ws13, const void* ws13_scales,
                      const void* ws2, const void* ws2_scales, void* y, float* logits_out,
                      int32_t* topk_idx_out, float* topk_gate_out, int32_t* counts_out,
                      void* ws, size_t ws_bytes, hipStream_t stream) {
    return layer_forward_impl(cfg, x, w_router, logit_bias, sel_bias, logits_in, w13,
                              w13_scales, w2, w2_scales, ws13, ws13_scales, ws2, ws2_scales, y,
                              logits_out, topk_idx_out, topk_gate_out, counts_out, ws, ws_bytes,
                              stream, nullptr);
}

int moe_layer_forward_train(const moe_config* cfg, const void* x, const void* w_router,
                            const float* logit_bias, const float* sel_bias,
                            const float* logits_in, const void* w13, const void* w2,
                            const void* ws13, const void* ws2, void* y, float* logits_out,
                            int32_t* topk_idx_out, float* topk_gate_out, int32_t* counts_out,
                            void* saved, size_t saved_bytes, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
    int st = check_cfg(cfg);
    if (st) return st;
    st = check_saved(cfg);
    if (st) return st;
    if (!saved) return MOE_ERR_INVALID_ARG;
    SavedActs sv = carve_saved(cfg, nullptr);
    if (saved_bytes < sv.total) return MOE_ERR_WORKSPACE;
    sv = carve_saved(cfg, saved);
    return layer_forward_impl(cfg, x, w_router, logit_bias, sel_bias, logits_in, w13, nullptr,
                              w2, nullptr, ws13, nullptr, ws2, nullptr, y, logits_out,
                              topk_idx_out, topk_gate_out, counts_out, ws, ws_bytes, stream,
                              &sv);
}

int moe_set_stage_events(void* const* events, int32_t n_events) {
    if (!events) {
        g_stage_on = false;
        return MOE_OK;
    }
    if (n_events != MOE_N_STAGE_EVENTS) return MOE_ERR_INVALID_ARG;
    for (int i = 0; i < MOE_N_STAGE_EVENTS; ++i)
        if (!events[i]) return MOE_ERR_INVALID_ARG;
    for (int i = 0; i < MOE_N_STAGE_EVENTS; ++i) g_stage_ev[i] = (hipEvent_t)events[i];
    g_stage_on = true;
    return MOE_OK;
}

int moe_grouped_gemm_swiglu_bwd(const moe_config* cfg, const void* dy_perm, const void* x_perm,
                                const void* z, const void* act, const float* gate_perm,
                                const int32_t* offsets, const void* w13, const void* w2,
                                void* dx_perm, void* dw13, void* dw2, float* dgate_perm,
                                void* ws, size_t ws_bytes, hipStream_t stream) {
    int st = check_cfg(cfg);
    if (st) return st;
    if (cfg->act_dtype != MOE_BF16 || cfg->a_layout) return MOE_ERR_UNSUPPORTED;
    if (cfg->capacity_factor != 0.0f) return MOE_ERR_UNSUPPORTED;      // dropless only
    if (!dy_perm || !x_perm || !z || !act || !offsets || !w13 || !w2 || !dx_perm || !dw13 ||
        !dw2 || !ws)
        return MOE_ERR_INVALID_ARG;
    if (ws_bytes < moe::bwd_ws_bytes(cfg->T, cfg->k, cfg->E, cfg->H, cfg->F))
        return MOE_ERR_WORKSPACE;
    return hip_status(moe::launch_grouped_gemm_bwd(dy_perm, x_perm, z, act, gate_perm, offsets,
                                                   w13, w2, cfg->T * cfg->k, cfg->E, cfg->H,
                                                   cfg->F, dx_perm, dw13, dw2, dgate_perm, ws,
                                                   stream, true, cfg->w_layout != 0));
}

// The layer backward; sv != NULL: Z and act come from the saved buffer of a training forward
// instead of a recomputed GEMM1 (moe_layer_backward_saved).
static int layer_backward_impl(const moe_config* cfg, const void* x, const void* w_router,
                               const float* logits, const float* logit_bias,
                               const int32_t* topk_idx, const float* topk_gate, const void* w13,
                               const void* w2, const void* ws13, const void* ws2, const void* dy,
                               void* dx, void* dw_router, void* dw13, void* dw2, void* dws13,
                               void* dws2, float* dlogits_out, void* ws, size_t ws_bytes,
                               hipStream_t stream, const SavedActs* sv) {
    int st = check_cfg(cfg);
    if (st) return st;
    st = check_layer_bwd(cfg);
    if (st) return st;
    if (!x || !w_router || !logits || !topk_idx || !topk_gate || !w13 || !w2 || !dy || !dx ||
        !dw_router || !dw13 || !dw2 || !ws)
        return MOE_ERR_INVALID_ARG;
    if (cfg->shared_F) {
        if (!ws13 || !ws2 || !dws13 || !dws2) return MOE_ERR_INVALID_ARG;
    } else if (ws13 || ws2 || dws13 || dws2) {
        return MOE_ERR_INVALID_ARG;
    }
    LayerBwdWs L = carve_layer_bwd(cfg, nullptr);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    L = carve_layer_bwd(cfg, ws);
    const int T = cfg->T, H = cfg->H, E = cfg->E, k = cfg->k, F = cfg->F, sF = cfg->shared_F;
    const int A = T * k;
    // the routing metadata once, then the expert-grouped x and dY (the permute of dY is the
    // backward of the combine). Recomputing, x_perm comes first (GEMM1 reads it) and dY is
    // left to the grouped backward (gathered on dW2's side stream; dA reads dY's rows through
    // src); with saved activations dy_perm comes first and x_perm is left to the grouped
    // backward (gathered on dW13's side stream beside dA). Measured, each is the faster form
    // for its path.
    hipError_t e = moe::launch_permute(1, -1, INT_MAX, x, topk_idx, topk_gate, T, H, E, k,
                                       L.counts, L.offsets, L.pos, L.src, L.gate_perm, nullptr,
                                       nullptr, nullptr, nullptr, L.perm_scratch, stream);
    if (e == hipSuccess)
        e = sv ? moe::launch_gather_rows(dy, L.pos, T, k, H * 2, L.dy_perm, stream)
               : moe::launch_gather_rows(x, L.pos, T, k, H * 2, L.x_perm, stream);
    const moe::BwdGather gx = {sv ? x : nullptr, sv ? nullptr : dy, L.pos, L.src, T, k};
    // Z and act of GEMM1 (routed, then the shared expert): saved by the forward, or recomputed
    void* z = sv ? sv->z : L.z;
    void* act = sv ? sv->act : L.act;
    void* zs = sv ? sv->zs : L.zs;
    void* acts = sv ? sv->acts : L.acts;
    if (e == hipSuccess && !sv) {
        Segment r1 = {L.x_perm, nullptr, L.offsets, E, 0, L.gate_perm, w13, nullptr, L.act,
                      nullptr, L.z, A, 0, cfg->w_layout, 0, nullptr};
        e = moe::launch_grouped_gemm(0, MOE_BF16, &r1, 1, A, 2 * F, H, L.sched, stream);
    }
    if (e == hipSuccess) e = moe::launch_offsets2(L.offs_one, T, stream);
    if (e == hipSuccess && sF && !sv) {
        Segment s1 = {x, nullptr, nullptr, 1, T, nullptr, ws13, nullptr, L.acts, nullptr, L.zs,
                      T, 0, cfg->w_layout, 0, nullptr};
        e = moe::launch_grouped_gemm(0, MOE_BF16, &s1, 1, T, 2 * sF, H, L.sched, stream);
    }
    // expert gradients (routed: dgate through the fold; shared: gate 1). Their weight
    // gradients run on the library's side streams, joined once at the end: nothing after
    // them reads dW or writes what they read, so the shared expert, the router backward and
    // the combine need not wait for them.
    struct SideLock {
        SideLock() { moe::bwd_side_lock(); }
        ~SideLock() { moe::bwd_side_unlock(); }
    } side_lock;
    if (e == hipSuccess)
        e = moe::launch_grouped_gemm_bwd(L.dy_perm, L.x_perm, z, act, L.gate_perm, L.offsets,
                                         w13, w2, A, E, H, F, L.dx_perm, dw13, dw2,
                                         L.dgate_perm, L.bws, stream, false, cfg->w_layout != 0,
                                         true, &gx);
    if (e == hipSuccess && sF)
        e = moe::launch_grouped_gemm_bwd(dy, x, zs, acts, nullptr, L.offs_one, ws13, ws2, T, 1,
                                         H, sF, L.dxs, dws13, dws2, nullptr, L.bws_s, stream,
                                         false, cfg->w_layout != 0, false);
    // gates -> logits -> router weight and x
    if (e == hipSuccess)
        e = moe::launch_route_backward(cfg->router, logits, logit_bias, topk_idx, topk_gate,
                                       L.dgate_perm, L.pos, T, E, k, cfg->route_scale,
                                       (uint16_t*)L.dl, dlogits_out, stream);
    if (e == hipSuccess)
        e = moe::launch_router_bwd(L.dl, x, w_router, T, E, H, dw_router, L.dxr, L.rws, stream);
    // dx = combine of the experts' rows (+ the shared expert's) + the router's part
    if (e == hipSuccess)
        e = moe::launch_combine(MOE_BF16, L.dx_perm, L.pos, sF ? L.dxs : nullptr, T, H, k, dx,
                                stream);
    if (e == hipSuccess) e = moe::launch_add_bf16(dx, L.dxr, (int64_t)T * H, stream);
    // join the weight gradients (also after a failure, so no side work outlives the call)
    const hipError_t j = moe::bwd_side_join(stream);
    if (e == hipSuccess) e = j;
    return hip_status(e);
}

int moe_layer_backward(const moe_config* cfg, const void* x, const void* w_router,
                       const float* logits, const float* logit_bias, const int32_t* topk_idx,
                       const float* topk_gate, const void* w13, const void* w2,
                       const void* ws13, const void* ws2, const void* dy, void* dx,
                       void* dw_router, void* dw13, void* dw2, void* dws13, void* dws2,
                       float* dlogits_out, void* ws, size_t ws_bytes, hipStream_t stream) {
    return layer_backward_impl(cfg, x, w_router, logits, logit_bias, topk_idx, topk_gate, w13,
                               w2, ws13, ws2, dy, dx, dw_router, dw13, dw2, dws13, dws2,
                               dlogits_out, ws, ws_bytes, stream, nullptr);
}

int moe_layer_backward_saved(const moe_config* cfg, const void* x, const void* w_router,
                             const float* logits, const float* logit_bias,
                             const int32_t* topk_idx, const float* topk_gate, const void* w13,
                             const void* w2, const void* ws13, const void* ws2,
                             const void* saved, size_t saved_bytes, const void* dy, void* dx,
                             void* dw_router, void* dw13, void* dw2, void* dws13, void* dws2,
                             float* dlogits_out, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
    int st = check_cfg(cfg);
    if (st) return st;
    st = check_layer_bwd(cfg);
    if (st) return st;
    if (!saved) return MOE_ERR_INVALID_ARG;
    SavedActs sv = carve_saved(cfg, nullptr);
    if (saved_bytes < sv.total) return MOE_ERR_WORKSPACE;
    sv = carve_saved(cfg, const_cast<void*>(saved));
    return layer_backward_impl(cfg, x, w_router, logits, logit_bias, topk_idx, topk_gate, w13,
                               w2, ws13, ws2, dy, dx, dw_router, dw13, dw2, dws13, dws2,
                               dlogits_out, ws, ws_bytes, stream, &sv);
}

int moe_pack_kblock(const void* in, int64_t n_mat, int32_t rows, int32_t cols,
                    int32_t elem_bytes, void* out, hipStream_t stream) {
    if (!in || !out || in == out) return MOE_ERR_INVALID_ARG;
    if (n_mat < 1 || rows < 1 || cols < 1) return MOE_ERR_INVALID_ARG;
    if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4) return MOE_ERR_INVALID_ARG;
    if (((int64_t)cols * elem_bytes) % 64) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_pack_kblock(in, n_mat, rows, cols, elem_bytes, out, stream));
}

int moe_quantize_mx(const void* in, int32_t in_dtype, int64_t rows, int32_t cols, uint8_t* q,
                    uint8_t* scales, hipStream_t stream) {
    if (!in || !q || !scales) return MOE_ERR_INVALID_ARG;
    if (in_dtype != MOE_F32 && in_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
    if (rows < 1 || cols < 1 || cols % 32) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_quantize_mx(in, in_dtype, rows, cols, 0, q, scales, stream));
}

int moe_pack_mx_scales(const uint8_t* in, int64_t n_mat, int32_t rows, int32_t cols,
                       uint8_t* out, hipStream_t stream) {
    if (!in || !out || in == out) return MOE_ERR_INVALID_ARG;
    if (n_mat < 1 || rows < 1 || cols < 1 || cols % 4) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_pack_mx_scales(in, n_mat, rows, cols, out, stream));
}

int moe_quantize_e4m3(const void* in, int32_t in_dtype, int64_t n_mat, int32_t rows,
                      int32_t cols, int32_t block_rows, int32_t block_cols, uint8_t* q,
                      float* scales, hipStream_t stream) {
    if (!in || !q || !scales) return MOE_ERR_INVALID_ARG;
    if (in_dtype != MOE_F32 && in_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
    if (n_mat < 1 || rows < 1 || cols < 1) return MOE_ERR_INVALID_ARG;
    if (block_cols != 128 || (block_rows != 1 && block_rows != 128)) return MOE_ERR_UNSUPPORTED;
    if (cols % 128 || rows % block_rows) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_quantize(in, in_dtype, n_mat, rows, cols, block_rows, q,
                                           scales, stream));
}

}  // extern "C"

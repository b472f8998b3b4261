"""Python binding of libmoe_amd.so, the MI355X (gfx950) MoE-layer forward.

Argument marshalling only: every function checks dtypes, shapes, contiguity and device of
its torch tensors, passes their data pointers and the current HIP stream to the C entry
point of the same name (include/moe.h) and raises on a non-zero status. All computation
happens in the HIP kernels; there is no fallback of any kind, and importing this package
fails loudly when the library has not been built.

A config is any object with the attributes T, H, E, k, F, router, n_groups, topk_groups,
route_scale, act_dtype, w_dtype, shared_F (dtype codes: 0 fp32, 1 bf16, 2 e4m3) and
optionally a_layout, w_layout (0 row-major, 1 K-blocked; default 0). A K-blocked [R, C]
tensor keeps its torch shape [R, C]; only the order of its bytes differs
([C * eb / 64][R][64 bytes]).
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_amd.so")

F32, BF16, E4M3, MXFP8 = 0, 1, 2, 3
SOFTMAX_TOPK, SIGMOID_GROUP_TOPK = 0, 1
LAYOUT_ROWS, LAYOUT_KBLOCK = 0, 1
OP_PERMUTE, OP_GROUPED_GEMM, OP_LAYER_FORWARD, OP_GROUPED_GEMM_BWD, OP_LAYER_BACKWARD = \
    0, 1, 2, 3, 4
OP_ROUTE_STATS = 5
OP_LAYER_SAVED = 6

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python routing_grouped_expert_softmax_amd/build.py`"
        " (there is no fallback path)")


class MoeConfigC(C.Structure):
    _fields_ = [("T", C.c_int32), ("H", C.c_int32), ("E", C.c_int32), ("k", C.c_int32),
                ("F", C.c_int32), ("n_groups", C.c_int32), ("topk_groups", C.c_int32),
                ("router", C.c_int32), ("route_scale", C.c_float), ("act_dtype", C.c_int32),
                ("w_dtype", C.c_int32), ("shared_F", C.c_int32), ("a_layout", C.c_int32),
                ("w_layout", C.c_int32), ("capacity_factor", C.c_float)]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {_lib.moe_status_string(status).decode()}")
        self.status = status


P = C.c_void_p
I32 = C.c_int32
I64 = C.c_int64
SZ = C.c_size_t
CFG = C.POINTER(MoeConfigC)

_lib = C.CDLL(LIB_PATH)
_lib.moe_status_string.restype = C.c_char_p
_lib.moe_status_string.argtypes = [C.c_int]
_SIGS = {
    "moe_workspace_size": [CFG, C.c_int, C.POINTER(C.c_size_t)],
    "moe_router_logits": [CFG, P, P, P, P],
    "moe_route": [CFG, P, P, P, P, P, P],
    "moe_route_stats": [CFG, P, P, P, P, P, P, P, SZ, P],
    "moe_permute": [CFG, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P],
    "moe_permute_noalloc": [CFG, P, P, P, P, P, P, P, P, P, P, P, P, P],
    "moe_grouped_gemm_swiglu": [CFG, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                P, SZ, P],
    "moe_grouped_gemm_up": [CFG, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P],
    "moe_grouped_gemm_down": [CFG, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P],
    "moe_unpermute_combine": [CFG, P, P, P, P, P],
    "moe_layer_forward": [CFG, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P],
    "moe_grouped_gemm_swiglu_bwd": [CFG, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P],
    "moe_quantize_e4m3": [P, I32, I64, I32, I32, I32, I32, P, P, P],
    "moe_quantize_mx": [P, I32, I64, I32, P, P, P],
    "moe_pack_mx_scales": [P, I64, I32, I32, P, P],
    "moe_pack_kblock": [P, I64, I32, I32, I32, P, P],
    "moe_set_stage_events": [P, I32],
    "moe_layer_backward": [CFG, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P],
    "moe_layer_forward_train": [CFG] + [P] * 15 + [SZ, P, SZ, P],
    "moe_layer_backward_saved": [CFG] + [P] * 11 + [SZ] + [P] * 8 + [P, SZ, P],
}
for _name, _args in _SIGS.items():
    getattr(_lib, _name).argtypes = _args
    getattr(_lib, _name).restype = C.c_int

EXPORTED = ["moe_status_string"] + list(_SIGS)


def lib():
    return _lib


def status_string(status: int) -> str:
    return _lib.moe_status_string(status).decode()


def make_config(cfg) -> MoeConfigC:
    return MoeConfigC(cfg.T, cfg.H, cfg.E, cfg.k, cfg.F, cfg.n_groups, cfg.topk_groups,
                      cfg.router, float(cfg.route_scale), cfg.act_dtype, cfg.w_dtype,
                      cfg.shared_F, getattr(cfg, "a_layout", 0), getattr(cfg, "w_layout", 0),
                      float(getattr(cfg, "capacity_factor", 0.0)))


def _check(fn: str, status: int):
    if status != 0:
        raise MoeError(fn, status)


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _ptr(t, dtype=None, shape=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.data_ptr() % 16:
        raise ValueError(f"{name}: must be 16-byte aligned (the kernels move 16-byte vectors)")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    return C.c_void_p(t.data_ptr())


def torch_dtype(code: int):
    return {F32: torch.float32, BF16: torch.bfloat16, E4M3: torch.uint8, MXFP8: torch.uint8}[code]


def act_torch_dtype(cfg):
    return torch_dtype(cfg.act_dtype)


def is_fp8(cfg):
    return cfg.w_dtype in (E4M3, MXFP8)


def gemm_torch_dtype(cfg):
    return torch.uint8 if is_fp8(cfg) else act_torch_dtype(cfg)


def act_scale_spec(cfg, rows, cols):
    """(dtype, shape) of the block scales of an fp8 activation [rows, cols]."""
    if cfg.w_dtype == MXFP8:
        return torch.uint8, (rows, cols // 32)
    return torch.float32, (rows, cols // 128)


def weight_scale_spec(cfg, lead, rows, cols):
    """(dtype, shape) of the block scales of fp8 weights lead + [rows, cols]."""
    if cfg.w_dtype == MXFP8:
        return torch.uint8, tuple(lead) + (rows, cols // 32)
    return torch.float32, tuple(lead) + (rows // 128, cols // 128)


def _psc(t, spec, name):
    return _ptr(t, spec[0], spec[1], name)


def workspace_size(cfg, op: int) -> int:
    c = make_config(cfg)
    n = C.c_size_t(0)
    _check("moe_workspace_size", _lib.moe_workspace_size(C.byref(c), op, C.byref(n)))
    return n.value


def workspace(cfg, op: int, device="cuda"):
    return torch.empty(max(1, workspace_size(cfg, op)), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------------------

def router_logits(cfg, x, w_router, logits=None, stream=None):
    ad = act_torch_dtype(cfg)
    if logits is None:
        logits = torch.empty(cfg.T, cfg.E, dtype=torch.float32, device=x.device)
    c = make_config(cfg)
    _check("moe_router_logits", _lib.moe_router_logits(
        C.byref(c), _ptr(x, ad, (cfg.T, cfg.H), "x"),
        _ptr(w_router, ad, (cfg.E, cfg.H), "w_router"),
        _ptr(logits, torch.float32, (cfg.T, cfg.E), "logits"), _stream(stream)))
    return logits


def route(cfg, logits, logit_bias=None, sel_bias=None, topk_idx=None, topk_gate=None,
          stream=None):
    dev = logits.device
    if topk_idx is None:
        topk_idx = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device=dev)
    if topk_gate is None:
        topk_gate = torch.empty(cfg.T, cfg.k, dtype=torch.float32, device=dev)
    c = make_config(cfg)
    _check("moe_route", _lib.moe_route(
        C.byref(c), _ptr(logits, torch.float32, (cfg.T, cfg.E), "logits"),
        _ptr(logit_bias, torch.float32, (cfg.E,), "logit_bias"),
        _ptr(sel_bias, torch.float32, (cfg.E,), "sel_bias"),
        _ptr(topk_idx, torch.int32, (cfg.T, cfg.k), "topk_idx"),
        _ptr(topk_gate, torch.float32, (cfg.T, cfg.k), "topk_gate"), _stream(stream)))
    return topk_idx, topk_gate


def route_stats(cfg, logits, logit_bias=None, sel_bias=None, ws=None, stream=None):
    """moe_route with the fused load-balancing statistics -> (topk_idx, topk_gate,
    prob_mean [E])."""
    dev = logits.device
    topk_idx = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device=dev)
    topk_gate = torch.empty(cfg.T, cfg.k, dtype=torch.float32, device=dev)
    prob_mean = torch.empty(cfg.E, dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(cfg, OP_ROUTE_STATS, dev)
    c = make_config(cfg)
    _check("moe_route_stats", _lib.moe_route_stats(
        C.byref(c), _ptr(logits, torch.float32, (cfg.T, cfg.E), "logits"),
        _ptr(logit_bias, torch.float32, (cfg.E,), "logit_bias"),
        _ptr(sel_bias, torch.float32, (cfg.E,), "sel_bias"), _ptr(topk_idx), _ptr(topk_gate),
        _ptr(prob_mean), _ptr(ws), ws.numel(), _stream(stream)))
    return topk_idx, topk_gate, prob_mean


def permute(cfg, x, topk_idx, topk_gate, want_x_q=False, ws=None, out=None, stream=None):
    """moe_permute. `out` may pass the dict a previous call returned (same cfg), so that its
    buffers are overwritten instead of new ones allocated."""
    dev = x.device
    T, H, E, k = cfg.T, cfg.H, cfg.E, cfg.k
    A = T * k
    fp8 = is_fp8(cfg)
    xsd, xss = act_scale_spec(cfg, A, H)
    qsd, qss = act_scale_spec(cfg, T, H)
    out = out if out is not None else dict(
        counts=torch.empty(E, dtype=torch.int32, device=dev),
        offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
        pos=torch.empty(T, k, dtype=torch.int32, device=dev),
        src=torch.empty(A, dtype=torch.int32, device=dev),
        gate_perm=torch.empty(A, dtype=torch.float32, device=dev),
        x_perm=torch.empty(A, H, dtype=gemm_torch_dtype(cfg), device=dev),
        x_perm_scales=torch.empty(xss, dtype=xsd, device=dev) if fp8 else None,
        x_q=torch.empty(T, H, dtype=torch.uint8, device=dev) if (fp8 and want_x_q) else None,
        x_q_scales=torch.empty(qss, dtype=qsd, device=dev) if (fp8 and want_x_q) else None,
    )
    if ws is None:
        ws = workspace(cfg, OP_PERMUTE, dev)
    c = make_config(cfg)
    _check("moe_permute", _lib.moe_permute(
        C.byref(c), _ptr(x, act_torch_dtype(cfg), (T, H), "x"),
        _ptr(topk_idx, torch.int32, (T, k), "topk_idx"),
        _ptr(topk_gate, torch.float32, (T, k), "topk_gate"),
        _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["pos"]), _ptr(out["src"]),
        _ptr(out["gate_perm"]), _ptr(out["x_perm"]), _ptr(out["x_perm_scales"]),
        _ptr(out["x_q"]), _ptr(out["x_q_scales"]), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def permute_noalloc(cfg, x, topk_idx, topk_gate, want_x_q=False, out=None, stream=None):
    """moe_permute_noalloc: moe_permute with the library's own device scratch (no workspace).
    Returns the same dict as permute(); `out` may pass a previous result to overwrite."""
    dev = x.device
    T, H, E, k = cfg.T, cfg.H, cfg.E, cfg.k
    A = T * k
    fp8 = is_fp8(cfg)
    xsd, xss = act_scale_spec(cfg, A, H)
    qsd, qss = act_scale_spec(cfg, T, H)
    out = out if out is not None else dict(
        counts=torch.empty(E, dtype=torch.int32, device=dev),
        offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
        pos=torch.empty(T, k, dtype=torch.int32, device=dev),
        src=torch.empty(A, dtype=torch.int32, device=dev),
        gate_perm=torch.empty(A, dtype=torch.float32, device=dev),
        x_perm=torch.empty(A, H, dtype=gemm_torch_dtype(cfg), device=dev),
        x_perm_scales=torch.empty(xss, dtype=xsd, device=dev) if fp8 else None,
        x_q=torch.empty(T, H, dtype=torch.uint8, device=dev) if (fp8 and want_x_q) else None,
        x_q_scales=torch.empty(qss, dtype=qsd, device=dev) if (fp8 and want_x_q) else None,
    )
    c = make_config(cfg)
    _check("moe_permute_noalloc", _lib.moe_permute_noalloc(
        C.byref(c), _ptr(x, act_torch_dtype(cfg), (T, H), "x"),
        _ptr(topk_idx, torch.int32, (T, k), "topk_idx"),
        _ptr(topk_gate, torch.float32, (T, k), "topk_gate"),
        _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["pos"]), _ptr(out["src"]),
        _ptr(out["gate_perm"]), _ptr(out["x_perm"]), _ptr(out["x_perm_scales"]),
        _ptr(out["x_q"]), _ptr(out["x_q_scales"]), _stream(stream)))
    return out


def grouped_gemm_swiglu(cfg, x_perm, offsets, gate_perm, w13, w2, x_perm_scales=None,
                        w13_scales=None, w2_scales=None, x_shared=None, x_shared_scales=None,
                        ws13=None, ws13_scales=None, ws2=None, ws2_scales=None, save_z=False,
                        ws=None, out=None, stream=None):
    dev = x_perm.device
    T, H, E, k, F = cfg.T, cfg.H, cfg.E, cfg.k, cfg.F
    A = T * k
    gd = gemm_torch_dtype(cfg)
    ad = act_torch_dtype(cfg)
    fp8 = is_fp8(cfg)
    sF = cfg.shared_F
    if out is None:
        asd, ass = act_scale_spec(cfg, A, F)
        out = dict(
            act=torch.empty(A, F, dtype=gd, device=dev),
            act_scales=torch.empty(ass, dtype=asd, device=dev) if fp8 else None,
            y_perm=torch.empty(A, H, dtype=ad, device=dev),
            shared_y=torch.empty(T, H, dtype=ad, device=dev) if sF else None,
            z=torch.empty(A, 2 * F, dtype=ad, device=dev) if save_z else None,
        )
    if ws is None:
        ws = workspace(cfg, OP_GROUPED_GEMM, dev)
    c = make_config(cfg)
    _check("moe_grouped_gemm_swiglu", _lib.moe_grouped_gemm_swiglu(
        C.byref(c), _ptr(x_perm, gd, (A, H), "x_perm"),
        _psc(x_perm_scales, act_scale_spec(cfg, A, H), "x_perm_scales"),
        _ptr(offsets, torch.int32, (E + 1,), "offsets"),
        _ptr(gate_perm, torch.float32, (A,), "gate_perm"),
        _ptr(w13, gd, (E, 2 * F, H), "w13"),
        _psc(w13_scales, weight_scale_spec(cfg, (E,), 2 * F, H), "w13_scales"),
        _ptr(w2, gd, (E, H, F), "w2"),
        _psc(w2_scales, weight_scale_spec(cfg, (E,), H, F), "w2_scales"),
        _ptr(x_shared, gd, (T, H), "x_shared"),
        _psc(x_shared_scales, act_scale_spec(cfg, T, H), "x_shared_scales"),
        _ptr(ws13, gd, (2 * sF, H), "ws13"),
        _psc(ws13_scales, weight_scale_spec(cfg, (), 2 * sF, H), "ws13_scales"),
        _ptr(ws2, gd, (H, sF), "ws2"),
        _psc(ws2_scales, weight_scale_spec(cfg, (), H, sF), "ws2_scales"),
        _ptr(out["act"]), _ptr(out["act_scales"]), _ptr(out["y_perm"]), _ptr(out["shared_y"]),
        _ptr(out["z"]), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def grouped_gemm_up(cfg, x_perm, offsets, gate_perm, w13, act, x_perm_scales=None,
                    w13_scales=None, x_shared=None, x_shared_scales=None, ws13=None,
                    ws13_scales=None, act_scales=None, shared_act=None,
                    shared_act_scales=None, z=None, ws=None, stream=None):
    """GEMM1 (gate/up + SwiGLU, gate folded in) into caller-provided outputs."""
    T, H, E, k, F = cfg.T, cfg.H, cfg.E, cfg.k, cfg.F
    A = T * k
    gd, ad = gemm_torch_dtype(cfg), act_torch_dtype(cfg)
    sF = cfg.shared_F
    if ws is None:
        ws = workspace(cfg, OP_GROUPED_GEMM, x_perm.device)
    c = make_config(cfg)
    _check("moe_grouped_gemm_up", _lib.moe_grouped_gemm_up(
        C.byref(c), _ptr(x_perm, gd, (A, H), "x_perm"),
        _psc(x_perm_scales, act_scale_spec(cfg, A, H), "x_perm_scales"),
        _ptr(offsets, torch.int32, (E + 1,), "offsets"),
        _ptr(gate_perm, torch.float32, (A,), "gate_perm"),
        _ptr(w13, gd, (E, 2 * F, H), "w13"),
        _psc(w13_scales, weight_scale_spec(cfg, (E,), 2 * F, H), "w13_scales"),
        _ptr(x_shared, gd, (T, H), "x_shared"),
        _psc(x_shared_scales, act_scale_spec(cfg, T, H), "x_shared_scales"),
        _ptr(ws13, gd, (2 * sF, H), "ws13"),
        _psc(ws13_scales, weight_scale_spec(cfg, (), 2 * sF, H), "ws13_scales"),
        _ptr(act, gd, (A, F), "act"), _psc(act_scales, act_scale_spec(cfg, A, F), "act_scales"),
        _ptr(shared_act, gd, (T, sF), "shared_act"),
        _psc(shared_act_scales, act_scale_spec(cfg, T, sF), "shared_act_scales"),
        _ptr(z, ad, (A, 2 * F), "z"), _ptr(ws), ws.numel(), _stream(stream)))


def grouped_gemm_down(cfg, act, offsets, w2, y_perm, act_scales=None, w2_scales=None,
                      shared_act=None, shared_act_scales=None, ws2=None, ws2_scales=None,
                      shared_y=None, ws=None, stream=None):
    """GEMM2 (down projection) into caller-provided outputs."""
    T, H, E, k, F = cfg.T, cfg.H, cfg.E, cfg.k, cfg.F
    A = T * k
    gd, ad = gemm_torch_dtype(cfg), act_torch_dtype(cfg)
    sF = cfg.shared_F
    if ws is None:
        ws = workspace(cfg, OP_GROUPED_GEMM, act.device)
    c = make_config(cfg)
    _check("moe_grouped_gemm_down", _lib.moe_grouped_gemm_down(
        C.byref(c), _ptr(act, gd, (A, F), "act"),
        _psc(act_scales, act_scale_spec(cfg, A, F), "act_scales"),
        _ptr(offsets, torch.int32, (E + 1,), "offsets"),
        _ptr(w2, gd, (E, H, F), "w2"),
        _psc(w2_scales, weight_scale_spec(cfg, (E,), H, F), "w2_scales"),
        _ptr(shared_act, gd, (T, sF), "shared_act"),
        _psc(shared_act_scales, act_scale_spec(cfg, T, sF), "shared_act_scales"),
        _ptr(ws2, gd, (H, sF), "ws2"),
        _psc(ws2_scales, weight_scale_spec(cfg, (), H, sF), "ws2_scales"),
        _ptr(y_perm, ad, (A, H), "y_perm"), _ptr(shared_y, ad, (T, H), "shared_y"),
        _ptr(ws), ws.numel(), _stream(stream)))


def unpermute_combine(cfg, y_perm, pos, shared_y=None, y=None, stream=None):
    ad = act_torch_dtype(cfg)
    if y is None:
        y = torch.empty(cfg.T, cfg.H, dtype=ad, device=y_perm.device)
    c = make_config(cfg)
    _check("moe_unpermute_combine", _lib.moe_unpermute_combine(
        C.byref(c), _ptr(y_perm, ad, (cfg.T * cfg.k, cfg.H), "y_perm"),
        _ptr(pos, torch.int32, (cfg.T, cfg.k), "pos"),
        _ptr(shared_y, ad, (cfg.T, cfg.H), "shared_y"),
        _ptr(y, ad, (cfg.T, cfg.H), "y"), _stream(stream)))
    return y


def layer_forward(cfg, x, w_router, w13, w2, logit_bias=None, sel_bias=None, logits_in=None,
                  w13_scales=None, w2_scales=None, ws13=None, ws13_scales=None, ws2=None,
                  ws2_scales=None, y=None, want=(), ws=None, stream=None):
    """The whole layer. `want` may name any of 'logits', 'topk_idx', 'topk_gate', 'counts'
    to also return those intermediate results. Returns (y, extras dict)."""
    dev = x.device
    T, H, E, k, F = cfg.T, cfg.H, cfg.E, cfg.k, cfg.F
    ad = act_torch_dtype(cfg)
    gd = gemm_torch_dtype(cfg)
    sF = cfg.shared_F
    if y is None:
        y = torch.empty(T, H, dtype=ad, device=dev)
    extras = {}
    if "logits" in want:
        extras["logits"] = torch.empty(T, E, dtype=torch.float32, device=dev)
    if "topk_idx" in want:
        extras["topk_idx"] = torch.empty(T, k, dtype=torch.int32, device=dev)
    if "topk_gate" in want:
        extras["topk_gate"] = torch.empty(T, k, dtype=torch.float32, device=dev)
    if "counts" in want:
        extras["counts"] = torch.empty(E, dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(cfg, OP_LAYER_FORWARD, dev)
    c = make_config(cfg)
    _check("moe_layer_forward", _lib.moe_layer_forward(
        C.byref(c), _ptr(x, ad, (T, H), "x"), _ptr(w_router, ad, (E, H), "w_router"),
        _ptr(logit_bias, torch.float32, (E,), "logit_bias"),
        _ptr(sel_bias, torch.float32, (E,), "sel_bias"),
        _ptr(logits_in, torch.float32, (T, E), "logits_in"),
        _ptr(w13, gd, (E, 2 * F, H), "w13"),
        _psc(w13_scales, weight_scale_spec(cfg, (E,), 2 * F, H), "w13_scales"),
        _ptr(w2, gd, (E, H, F), "w2"),
        _psc(w2_scales, weight_scale_spec(cfg, (E,), H, F), "w2_scales"),
        _ptr(ws13, gd, (2 * sF, H), "ws13"),
        _psc(ws13_scales, weight_scale_spec(cfg, (), 2 * sF, H), "ws13_scales"),
        _ptr(ws2, gd, (H, sF), "ws2"),
        _psc(ws2_scales, weight_scale_spec(cfg, (), H, sF), "ws2_scales"),
        _ptr(y, ad, (T, H), "y"), _ptr(extras.get("logits")), _ptr(extras.get("topk_idx")),
        _ptr(extras.get("topk_gate")), _ptr(extras.get("counts")), _ptr(ws), ws.numel(),
        _stream(stream)))
    return y, extras


def layer_forward_train(cfg, x, w_router, w13, w2, logit_bias=None, sel_bias=None,
                        logits_in=None, ws13=None, ws2=None, y=None, want=(), saved=None,
                        ws=None, stream=None):
    """The bf16 layer forward that also keeps GEMM1's Z and act for layer_backward_saved
    (moe_layer_forward_train). Returns (y, extras dict as layer_forward, saved buffer)."""
    dev = x.device
    T, H, E, k, F, sF = cfg.T, cfg.H, cfg.E, cfg.k, cfg.F, cfg.shared_F
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    if y is None:
        y = torch.empty(T, H, dtype=bf, device=dev)
    shapes = dict(logits=((T, E), f32), topk_idx=((T, k), i32), topk_gate=((T, k), f32),
                  counts=((E,), i32))
    extras = {n: torch.empty(shapes[n][0], dtype=shapes[n][1], device=dev) for n in want}
    if saved is None:
        saved = workspace(cfg, OP_LAYER_SAVED, dev)
    if ws is None:
        ws = workspace(cfg, OP_LAYER_FORWARD, dev)
    c = make_config(cfg)
    _check("moe_layer_forward_train", _lib.moe_layer_forward_train(
        C.byref(c), _ptr(x, bf, (T, H), "x"), _ptr(w_router, bf, (E, H), "w_router"),
        _ptr(logit_bias, f32, (E,), "logit_bias"), _ptr(sel_bias, f32, (E,), "sel_bias"),
        _ptr(logits_in, f32, (T, E), "logits_in"), _ptr(w13, bf, (E, 2 * F, H), "w13"),
        _ptr(w2, bf, (E, H, F), "w2"), _ptr(ws13, bf, (2 * sF, H), "ws13"),
        _ptr(ws2, bf, (H, sF), "ws2"), _ptr(y, bf, (T, H), "y"), _ptr(extras.get("logits")),
        _ptr(extras.get("topk_idx")), _ptr(extras.get("topk_gate")),
        _ptr(extras.get("counts")), _ptr(saved, torch.uint8, name="saved"), saved.numel(), _ptr(ws),
        ws.numel(), _stream(stream)))
    return y, extras, saved


def grouped_gemm_swiglu_bwd(cfg, dy_perm, x_perm, z, act, gate_perm, offsets, w13, w2,
                            want_dgate=True, ws=None, stream=None):
    """Backward of the grouped expert MLP (moe_grouped_gemm_swiglu_bwd). gate_perm may be
    None (gate 1). Returns dict dx_perm, dw13, dw2, dgate_perm (None unless want_dgate)."""
    dev = dy_perm.device
    T, H, E, k, F = cfg.T, cfg.H, cfg.E, cfg.k, cfg.F
    A = T * k
    bf = torch.bfloat16
    out = dict(dx_perm=torch.empty(A, H, dtype=bf, device=dev),
               dw13=torch.empty(E, 2 * F, H, dtype=bf, device=dev),
               dw2=torch.empty(E, H, F, dtype=bf, device=dev),
               dgate_perm=torch.empty(A, dtype=torch.float32, device=dev) if want_dgate else None)
    if ws is None:
        ws = workspace(cfg, OP_GROUPED_GEMM_BWD, dev)
    c = make_config(cfg)
    _check("moe_grouped_gemm_swiglu_bwd", _lib.moe_grouped_gemm_swiglu_bwd(
        C.byref(c), _ptr(dy_perm, bf, (A, H), "dy_perm"), _ptr(x_perm, bf, (A, H), "x_perm"),
        _ptr(z, bf, (A, 2 * F), "z"), _ptr(act, bf, (A, F), "act"),
        _ptr(gate_perm, torch.float32, (A,), "gate_perm"),
        _ptr(offsets, torch.int32, (E + 1,), "offsets"), _ptr(w13, bf, (E, 2 * F, H), "w13"),
        _ptr(w2, bf, (E, H, F), "w2"), _ptr(out["dx_perm"]), _ptr(out["dw13"]),
        _ptr(out["dw2"]), _ptr(out["dgate_perm"]), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def layer_backward(cfg, x, w_router, logits, topk_idx, topk_gate, w13, w2, dy,
                   logit_bias=None, ws13=None, ws2=None, want_dlogits=False, ws=None,
                   stream=None):
    """Gradients of the whole layer (moe_layer_backward) for the forward's routing. Returns
    dict dx, dw_router, dw13, dw2, dws13, dws2 (None without a shared expert), dlogits
    (fp32, None unless want_dlogits)."""
    dev = x.device
    T, H, E, k, F, sF = cfg.T, cfg.H, cfg.E, cfg.k, cfg.F, cfg.shared_F
    bf, f32 = torch.bfloat16, torch.float32
    out = dict(dx=torch.empty(T, H, dtype=bf, device=dev),
               dw_router=torch.empty(E, H, dtype=bf, device=dev),
               dw13=torch.empty(E, 2 * F, H, dtype=bf, device=dev),
               dw2=torch.empty(E, H, F, dtype=bf, device=dev),
               dws13=torch.empty(2 * sF, H, dtype=bf, device=dev) if sF else None,
               dws2=torch.empty(H, sF, dtype=bf, device=dev) if sF else None,
               dlogits=torch.empty(T, E, dtype=f32, device=dev) if want_dlogits else None)
    if ws is None:
        ws = workspace(cfg, OP_LAYER_BACKWARD, dev)
    c = make_config(cfg)
    _check("moe_layer_backward", _lib.moe_layer_backward(
        C.byref(c), _ptr(x, bf, (T, H), "x"), _ptr(w_router, bf, (E, H), "w_router"),
        _ptr(logits, f32, (T, E), "logits"), _ptr(logit_bias, f32, (E,), "logit_bias"),
        _ptr(topk_idx, torch.int32, (T, k), "topk_idx"),
        _ptr(topk_gate, f32, (T, k), "topk_gate"), _ptr(w13, bf, (E, 2 * F, H), "w13"),
        _ptr(w2, bf, (E, H, F), "w2"), _ptr(ws13, bf, (2 * sF, H), "ws13"),
        _ptr(ws2, bf, (H, sF), "ws2"), _ptr(dy, bf, (T, H), "dy"), _ptr(out["dx"]),
        _ptr(out["dw_router"]), _ptr(out["dw13"]), _ptr(out["dw2"]), _ptr(out["dws13"]),
        _ptr(out["dws2"]), _ptr(out["dlogits"]), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def layer_backward_saved(cfg, x, w_router, logits, topk_idx, topk_gate, w13, w2, dy, saved,
                         logit_bias=None, ws13=None, ws2=None, want_dlogits=False, ws=None,
                         stream=None):
    """layer_backward with Z and act from layer_forward_train's saved buffer instead of a
    recomputed GEMM1 (moe_layer_backward_saved). Returns the same dict as layer_backward."""
    dev = x.device
    T, H, E, k, F, sF = cfg.T, cfg.H, cfg.E, cfg.k, cfg.F, cfg.shared_F
    bf, f32 = torch.bfloat16, torch.float32
    out = dict(dx=torch.empty(T, H, dtype=bf, device=dev),
               dw_router=torch.empty(E, H, dtype=bf, device=dev),
               dw13=torch.empty(E, 2 * F, H, dtype=bf, device=dev),
               dw2=torch.empty(E, H, F, dtype=bf, device=dev),
               dws13=torch.empty(2 * sF, H, dtype=bf, device=dev) if sF else None,
               dws2=torch.empty(H, sF, dtype=bf, device=dev) if sF else None,
               dlogits=torch.empty(T, E, dtype=f32, device=dev) if want_dlogits else None)
    if ws is None:
        ws = workspace(cfg, OP_LAYER_BACKWARD, dev)
    c = make_config(cfg)
    _check("moe_layer_backward_saved", _lib.moe_layer_backward_saved(
        C.byref(c), _ptr(x, bf, (T, H), "x"), _ptr(w_router, bf, (E, H), "w_router"),
        _ptr(logits, f32, (T, E), "logits"), _ptr(logit_bias, f32, (E,), "logit_bias"),
        _ptr(topk_idx, torch.int32, (T, k), "topk_idx"),
        _ptr(topk_gate, f32, (T, k), "topk_gate"), _ptr(w13, bf, (E, 2 * F, H), "w13"),
        _ptr(w2, bf, (E, H, F), "w2"), _ptr(ws13, bf, (2 * sF, H), "ws13"),
        _ptr(ws2, bf, (H, sF), "ws2"), _ptr(saved, torch.uint8, name="saved"), saved.numel(),
        _ptr(dy, bf, (T, H), "dy"), _ptr(out["dx"]), _ptr(out["dw_router"]),
        _ptr(out["dw13"]), _ptr(out["dw2"]), _ptr(out["dws13"]), _ptr(out["dws2"]),
        _ptr(out["dlogits"]), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def quantize_e4m3(t, block_rows: int, stream=None):
    """e4m3 block quantisation of [rows, cols] or [n, rows, cols] (bf16 or fp32) ->
    (codes uint8 of the same shape, fp32 scales [..., rows/block_rows, cols/128])."""
    dt = {torch.float32: F32, torch.bfloat16: BF16}[t.dtype]
    shape = tuple(t.shape)
    n, rows, cols = (1,) + shape if len(shape) == 2 else shape
    q = torch.empty(shape, dtype=torch.uint8, device=t.device)
    s = torch.empty(shape[:-2] + (rows // block_rows, cols // 128), dtype=torch.float32,
                    device=t.device)
    _check("moe_quantize_e4m3", _lib.moe_quantize_e4m3(
        _ptr(t, name="input"), dt, n, rows, cols, block_rows, 128, _ptr(q), _ptr(s),
        _stream(stream)))
    return q, s


def quantize_mx(t, stream=None):
    """MXFP8 quantisation along the last axis of a bf16 / fp32 tensor (32-value blocks) ->
    (codes uint8 of the same shape, E8M0 scale codes uint8 [..., cols/32])."""
    dt = {torch.float32: F32, torch.bfloat16: BF16}[t.dtype]
    shape = tuple(t.shape)
    cols = shape[-1]
    rows = t.numel() // cols
    q = torch.empty(shape, dtype=torch.uint8, device=t.device)
    s = torch.empty(shape[:-1] + (cols // 32,), dtype=torch.uint8, device=t.device)
    _check("moe_quantize_mx", _lib.moe_quantize_mx(
        _ptr(t, name="input"), dt, rows, cols, _ptr(q), _ptr(s), _stream(stream)))
    return q, s


def pack_mx_scales(s, stream=None):
    """MXFP8 weight scales [..., rows, cols] (uint8 E8M0, cols = K/32) -> the blocked order of
    K-blocked weights, [..., cols/4, rows, 4] stored in a tensor of the input's shape."""
    shape = tuple(s.shape)
    rows, cols = shape[-2], shape[-1]
    n = s.numel() // (rows * cols)
    out = torch.empty_like(s)
    _check("moe_pack_mx_scales", _lib.moe_pack_mx_scales(
        _ptr(s, torch.uint8, name="scales"), n, rows, cols, _ptr(out), _stream(stream)))
    return out


def pack_kblock(t, out=None, stream=None):
    """Row-major [rows, cols] or [n, rows, cols] -> the same shape in the K-blocked layout
    (moe_pack_kblock)."""
    shape = tuple(t.shape)
    n, rows, cols = (1,) + shape if len(shape) == 2 else shape
    if out is None:
        out = torch.empty_like(t)
    _ptr(out, t.dtype, shape, "out")
    _check("moe_pack_kblock", _lib.moe_pack_kblock(
        _ptr(t, name="input"), n, rows, cols, t.element_size(), _ptr(out), _stream(stream)))
    return out


N_STAGE_EVENTS = 7
STAGES = ("router_logits", "route", "permute", "grouped_gemm_up", "grouped_gemm_down",
          "combine")


def set_stage_events(events):
    """Make later layer_forward calls on this thread record the given torch.cuda.Event
    objects (7, with timing) on their stream at each stage boundary (moe_set_stage_events);
    None stops. The events must outlive their use."""
    if events is None:
        _check("moe_set_stage_events", _lib.moe_set_stage_events(None, 0))
        return
    if len(events) != N_STAGE_EVENTS:
        raise ValueError(f"need {N_STAGE_EVENTS} events, got {len(events)}")
    for ev in events:
        if not ev.cuda_event:       # torch creates the HIP event on its first record
            ev.record()
    arr = (C.c_void_p * N_STAGE_EVENTS)(*[ev.cuda_event for ev in events])
    _check("moe_set_stage_events", _lib.moe_set_stage_events(arr, N_STAGE_EVENTS))

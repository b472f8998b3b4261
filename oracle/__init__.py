"""CPU oracle for one token-choice MoE layer -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check in __graft_entry__ and the CPU-baseline leg of bench.py may
import this package. The product library never imports it, and nothing here imports the
product package.

The arithmetic lives in moe_oracle.c (plain loops, double precision); this module compiles
it with gcc when no up-to-date build exists and wraps each entry point with numpy arrays.
Which part of the pages each function follows is stated in the C source.

Parity status: every function here is pinned by tests under tests/ (marked "not gpu")
against library routines, closed forms, brute force on tiny inputs, the OCP e4m3
specification, or (layer_backward) torch.autograd of an independently written forward and
central finite differences; except absolute output values for the full-size workloads,
which no page prints ("parity unpinned" for those values; they rest on the pinned pieces).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import math

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
_lock = threading.Lock()
_lib = None

F32, BF16, E4M3, MXFP8 = 0, 1, 2, 3
SOFTMAX_TOPK, SIGMOID_GROUP_TOPK = 0, 1


def build(force: bool = False) -> str:
    """Compile the oracle (gcc, -O2, OpenMP, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-std=c11",
                               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


P = C.c_void_p
I32 = C.c_int
I64 = C.c_int64


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = C.CDLL(_LIB)
            L.orc_e4m3_value.restype = C.c_double
            L.orc_e4m3_value.argtypes = [C.c_uint8]
            L.orc_e4m3_encode.restype = C.c_uint8
            L.orc_e4m3_encode.argtypes = [C.c_float]
            L.orc_quant_rows.argtypes = [P, I32, I64, I32, P, P]
            L.orc_mx_quant.argtypes = [P, I32, I64, I32, P, P]
            L.orc_quant_weight.argtypes = [P, I32, I64, I32, I32, P, P]
            L.orc_router_logits.argtypes = [P, P, I32, I32, I32, I32, P]
            L.orc_route.argtypes = [P, P, P, I32, I32, I32, I32, I32, I32, C.c_double, P, P, P]
            L.orc_permute.argtypes = [P, P, I32, I32, I32, P, P, P, P, P]
            L.orc_expert_rows.argtypes = [I32, I32, I32, P, I32, P, P, P, P, P, I32, P, P,
                                          I32, P, I64, P, P, P]
            L.orc_layer_tokens.argtypes = [I32, I32, I32, I32, I32, I32, P, I32, I32, P, P,
                                           P, P, I32, P, P, P, P, P, P, I32, P, I64, P]
            L.orc_expert_bwd_rows.argtypes = [I32, I32, I32, P, P, I32, P, P, P, P, P, I64,
                                              P, P]
            L.orc_expert_wgrad_entries.argtypes = [I32, I32, P, P, P, P, I32, P, I32, P, P,
                                                   P, P, I64, P, P, P, I64, P]
            L.orc_combine.argtypes = [P, P, I32, P, I32, I32, I32, P]
            L.orc_permute_capacity.argtypes = [P, P, I32, I32, I32, I32, P, P, P, P, P]
            L.orc_set_threads.argtypes = [I32]
            L.orc_set_threads.restype = None
            L.orc_max_threads.argtypes = []
            L.orc_max_threads.restype = I32
            for f in ("orc_quant_rows", "orc_quant_weight", "orc_router_logits", "orc_route",
                      "orc_permute", "orc_expert_rows", "orc_layer_tokens",
                      "orc_expert_bwd_rows", "orc_expert_wgrad_entries", "orc_combine"):
                getattr(L, f).restype = None
            _lib = L
    return _lib


def set_threads(n: int) -> None:
    """Host threads of the oracle's parallel loops (for timing only; results are the same
    for any count)."""
    lib().orc_set_threads(int(n))


def max_threads() -> int:
    return int(lib().orc_max_threads())


# ------------------------------------------------------------------------------------
# array helpers: the oracle takes numpy arrays (bf16 as uint16 bit patterns, e4m3 as uint8)
# ------------------------------------------------------------------------------------

def as_np(t):
    """torch CPU tensor or numpy array -> (contiguous numpy array, dtype code)."""
    try:
        import torch
        if isinstance(t, torch.Tensor):
            t = t.detach().contiguous()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16), BF16
            if t.dtype == torch.float32:
                return t.numpy(), F32
            if t.dtype == torch.uint8:
                return t.numpy(), E4M3
            raise TypeError(f"unsupported dtype {t.dtype}")
    except ImportError:
        pass
    a = np.ascontiguousarray(t)
    if a.dtype == np.uint16:
        return a, BF16
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint8:
        return a, E4M3
    raise TypeError(f"unsupported dtype {a.dtype}")


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _f32(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _sc(a):
    """Block scales: fp32 (1 x 128 / 128 x 128 e4m3 scales) or uint8 E8M0 codes (MXFP8)."""
    if a is None:
        return None
    a = np.asarray(a)
    return np.ascontiguousarray(a if a.dtype == np.uint8 else a.astype(np.float32))


def _i32(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _i64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


# ------------------------------------------------------------------------------------
# number formats
# ------------------------------------------------------------------------------------

def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(int(code))


def e4m3_encode(v: float) -> int:
    return lib().orc_e4m3_encode(float(v))


def e4m3_decode_array(q: np.ndarray) -> np.ndarray:
    table = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
    return table[q]


def quant_rows(v, block: int = 128):
    """1 x 128 block quantisation of [rows, cols] -> (codes uint8 [rows, cols], scales f32)."""
    a, dt = as_np(v)
    rows, cols = a.shape
    assert cols % block == 0 and block == 128
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // 128), np.float32)
    lib().orc_quant_rows(_p(a), dt, rows, cols, _p(q), _p(s))
    return q, s


def mx_quant(v):
    """MXFP8 block quantisation of [rows, cols] (or [n, rows, cols]) along the last axis,
    32 values per block -> (codes uint8, E8M0 scale codes uint8 [..., cols / 32])."""
    a, dt = as_np(v)
    shape = a.shape
    cols = shape[-1]
    rows = int(np.prod(shape[:-1]))
    q = np.empty(shape, np.uint8)
    s = np.empty(shape[:-1] + (cols // 32,), np.uint8)
    lib().orc_mx_quant(_p(a), dt, rows, cols, _p(q), _p(s))
    return q, s


def mx_dequant(q, s):
    """Values of MX codes: e4m3(q) * 2^(s - 127) per 32-value block -> float64."""
    v = e4m3_decode_array(np.asarray(q))
    sc = np.exp2(np.asarray(s, np.float64) - 127.0)
    return v * np.repeat(sc, 32, axis=-1)


def quant_weight(w):
    """128 x 128 block quantisation of [n, rows, cols] (or [rows, cols])."""
    a, dt = as_np(w)
    squeeze = a.ndim == 2
    if squeeze:
        a = a[None]
    n, rows, cols = a.shape
    assert rows % 128 == 0 and cols % 128 == 0
    q = np.empty((n, rows, cols), np.uint8)
    s = np.empty((n, rows // 128, cols // 128), np.float32)
    lib().orc_quant_weight(_p(a), dt, n, rows, cols, _p(q), _p(s))
    if squeeze:
        return q[0], s[0]
    return q, s


# ------------------------------------------------------------------------------------
# routing
# ------------------------------------------------------------------------------------

def router_logits(x, w_router) -> np.ndarray:
    xa, dt = as_np(x)
    wa, dt2 = as_np(w_router)
    assert dt == dt2
    T, H = xa.shape
    E = wa.shape[0]
    out = np.empty((T, E), np.float32)
    lib().orc_router_logits(_p(xa), _p(wa), dt, T, H, E, _p(out))
    return out


def route(logits, k, router=SOFTMAX_TOPK, logit_bias=None, sel_bias=None, n_groups=1,
          topk_groups=1, route_scale=1.0, return_scores=False):
    lg = _f32(logits)
    T, E = lg.shape
    assert E <= 4096 and k <= E
    idx = np.empty((T, k), np.int32)
    gate = np.empty((T, k), np.float32)
    sc = np.empty((T, E), np.float32) if return_scores else None
    lib().orc_route(_p(lg), _p(_f32(logit_bias)), _p(_f32(sel_bias)), T, E, k, router,
                    n_groups, topk_groups, float(route_scale), _p(idx), _p(gate), _p(sc))
    if return_scores:
        return idx, gate, sc
    return idx, gate


def route_cfg(cfg, logits, logit_bias=None, sel_bias=None, return_scores=False):
    return route(logits, cfg.k, cfg.router, logit_bias, sel_bias, cfg.n_groups,
                 cfg.topk_groups, cfg.route_scale, return_scores)


def permute(topk_idx, topk_gate, E, capacity=None):
    """Routing metadata. capacity (assignments per expert, or None = dropless): experts accept
    their assignments in token order while they have slots; dropped ones get pos = -1, and
    src / gate_perm are filled for rows [0, offsets[E]) only."""
    idx = _i32(topk_idx)
    T, k = idx.shape
    g = _f32(topk_gate)
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    pos = np.empty((T, k), np.int32)
    src = np.full(T * k, -1, np.int32)
    gp = np.zeros(T * k, np.float32)
    if capacity is None:
        lib().orc_permute(_p(idx), _p(g), T, k, E, _p(counts), _p(offsets), _p(pos), _p(src),
                          _p(gp))
    else:
        lib().orc_permute_capacity(_p(idx), _p(g), T, k, E, int(capacity), _p(counts),
                                   _p(offsets), _p(pos), _p(src), _p(gp))
    return dict(counts=counts, offsets=offsets, pos=pos, src=src, gate_perm=gp)


def expert_capacity(capacity_factor, T, k, E):
    """Expert capacity ceil(cf * T * k / E) in double, with cf first rounded to fp32 (the
    type of the configuration field); None for cf == 0 (dropless)."""
    cf = float(np.float32(capacity_factor))
    if cf == 0.0:
        return None
    return min(T * k, math.ceil(cf * float(T * k) / float(E)))


def drop_slots(topk_idx, pos):
    """topk_idx with the slots dropped by a capacity (pos < 0) set to -1, the form
    layer_tokens takes for them."""
    idx = np.array(_i32(topk_idx), copy=True)
    idx[np.asarray(pos) < 0] = -1
    return idx


def route_prob_mean(cfg, logits, logit_bias=None):
    """Mean router probability per expert over the T tokens, float64: p = softmax(l) over all
    E experts (softmax router) or p = s / sum s with s = fp32(sigmoid(l)) (sigmoid router),
    l = fp32(logits + logit_bias) as in the routing."""
    l = np.asarray(logits, np.float32)
    if logit_bias is not None:
        l = (l + np.asarray(logit_bias, np.float32)).astype(np.float32)
    l = l.astype(np.float64)
    if cfg.router == SOFTMAX_TOPK:
        z = np.exp(l - l.max(axis=1, keepdims=True))
        p = z / z.sum(axis=1, keepdims=True)
    else:
        s = (1.0 / (1.0 + np.exp(-l))).astype(np.float32).astype(np.float64)
        p = s / s.sum(axis=1, keepdims=True)
    return p.mean(axis=0)


def gather_rows(x, pos):
    """x_perm[pos[t, j]] = x[t]: the permuted copy (pure data movement)."""
    a = np.asarray(x)
    pos = np.asarray(pos)
    T, k = pos.shape
    out = np.empty((T * k,) + a.shape[1:], a.dtype)
    for j in range(k):
        out[pos[:, j]] = a
    return out


def combine(y_perm, pos, shared_y=None):
    """y[t] = sum_j y_perm[pos[t, j]] (+ shared_y[t]) -> float64 [T, H]."""
    ya, dt = as_np(y_perm)
    sa = None
    if shared_y is not None:
        sa, dt2 = as_np(shared_y)
        assert dt2 == dt
    pos = _i32(pos)
    T, k = pos.shape
    H = ya.shape[1]
    y = np.empty((T, H))
    lib().orc_combine(_p(ya), _p(sa), dt, _p(pos), T, k, H, _p(y))
    return y


# ------------------------------------------------------------------------------------
# expert math
# ------------------------------------------------------------------------------------

def expert_rows(x_perm, offsets, gate_perm, w13, w2, rows, x_scales=None, w13_scales=None,
                w2_scales=None, quant_act=False, want_z=False, mx=False):
    """Expert math for selected rows of the expert-grouped buffer.
    mx: the uint8 operands are MXFP8 codes with E8M0 scales per 1 x 32 block (else e4m3 with
    fp32 1 x 128 / 128 x 128 scales), and quant_act quantises the activation the same way.
    Returns (z or None, act, y_perm) as float64 arrays [n, 2F], [n, F], [n, H]."""
    xa, xdt = as_np(x_perm)
    w13a, wdt = as_np(w13)
    w2a, wdt2 = as_np(w2)
    assert wdt == wdt2
    if mx:
        assert wdt == E4M3
        wdt = MXFP8
        xdt = MXFP8 if xdt == E4M3 else xdt
    if w13a.ndim == 2:
        w13a, w2a = w13a[None], w2a[None]
    E, F2, H = w13a.shape
    F = F2 // 2
    rows = _i64(rows)
    n = rows.shape[0]
    z = np.empty((n, 2 * F)) if want_z else None
    act = np.empty((n, F))
    y = np.empty((n, H))
    lib().orc_expert_rows(H, F, E, _p(xa), xdt, _p(_sc(x_scales)), _p(_i32(offsets)),
                          _p(_f32(gate_perm)), _p(w13a), _p(w2a), wdt,
                          _p(_sc(w13_scales)), _p(_sc(w2_scales)),
                          (2 if mx else 1) if quant_act else 0,
                          _p(rows), n, _p(z), _p(act), _p(y))
    return z, act, y


def layer_tokens(x, topk_idx, topk_gate, w13, w2, tokens, ws13=None, ws2=None, fp8=False,
                 w13_scales=None, w2_scales=None, ws13_scales=None, ws2_scales=None,
                 fold=True):
    """The per-token loop for selected tokens -> y [n, H] float64.
    fp8: False; True (e4m3, 1 x 128 activation / 128 x 128 weight scales); or "mx" (MXFP8:
    e4m3 codes with an E8M0 scale per 1 x 32 block for x, the activation and the weights)."""
    xa, xdt = as_np(x)
    T, H = xa.shape
    idx = _i32(topk_idx)
    k = idx.shape[1]
    w13a, wdt = as_np(w13)
    w2a, _ = as_np(w2)
    E, F2, _ = w13a.shape
    F = F2 // 2
    sF = 0
    s13a = s2a = None
    if ws13 is not None:
        s13a, _ = as_np(ws13)
        s2a, _ = as_np(ws2)
        sF = s13a.shape[0] // 2
    tokens = _i64(tokens)
    n = tokens.shape[0]
    y = np.empty((n, H))
    mode = 2 if fp8 == "mx" else int(bool(fp8))
    if mode == 2:
        assert wdt == E4M3
        wdt = MXFP8
    lib().orc_layer_tokens(T, H, E, k, F, sF, _p(xa), xdt, mode, _p(idx),
                           _p(_f32(topk_gate)), _p(w13a), _p(w2a), wdt, _p(_sc(w13_scales)),
                           _p(_sc(w2_scales)), _p(s13a), _p(s2a), _p(_sc(ws13_scales)),
                           _p(_sc(ws2_scales)), int(fold), _p(tokens), n, _p(y))
    return y


def expert_bwd_rows(dy_perm, z, offsets, gate_perm, w13, w2, rows):
    """Data gradients of selected rows -> (dx [n, H], dg [n])."""
    dya, dt = as_np(dy_perm)
    za, dt2 = as_np(z)
    w13a, dt3 = as_np(w13)
    w2a, dt4 = as_np(w2)
    assert dt == dt2 == dt3 == dt4
    if w13a.ndim == 2:
        w13a, w2a = w13a[None], w2a[None]
    E, F2, H = w13a.shape
    F = F2 // 2
    rows = _i64(rows)
    n = rows.shape[0]
    dx = np.empty((n, H))
    dg = np.empty(n)
    lib().orc_expert_bwd_rows(H, F, E, _p(dya), _p(za), dt, _p(_i32(offsets)),
                              _p(_f32(gate_perm)), _p(w13a), _p(w2a), _p(rows), n, _p(dx),
                              _p(dg))
    return dx, dg


def expert_wgrad_entries(dy_perm, z, act, x_perm, offsets, e, gate_perm, w2, w13_rc, w2_rc):
    """Selected entries of dW13_e and dW2_e -> (dw13 [n13], dw2 [n2])."""
    dya, dt = as_np(dy_perm)
    za, _ = as_np(z)
    aa, _ = as_np(act)
    xa, _ = as_np(x_perm)
    w2a, _ = as_np(w2)
    if w2a.ndim == 2:
        w2a = w2a[None]
    _, H, F = w2a.shape
    r13, c13 = (_i32(v) for v in w13_rc)
    r2, c2 = (_i32(v) for v in w2_rc)
    dw13 = np.empty(r13.shape[0])
    dw2 = np.empty(r2.shape[0])
    offs = _i32(offsets)
    lib().orc_expert_wgrad_entries(H, F, _p(dya), _p(za), _p(aa), _p(xa), dt, _p(offs), e,
                                   _p(_f32(gate_perm)), _p(w2a), _p(r13), _p(c13),
                                   r13.shape[0], _p(dw13), _p(r2), _p(c2), r2.shape[0],
                                   _p(dw2))
    return dw13, dw2


# ---------------------------------------------------------------------------------------
# Backward of the whole layer (numpy, float64). It follows the forward of the study notes'
# case 1 (per token: y = sum_j g_j Expert_{e_j}(x), plus the shared expert) with the gate
# folded into the activation (technical summary, section 2.2), differentiated by the chain
# rule; the data and weight gradients are the W/D split of section 2.3. The expert choice
# is a selection and carries no gradient; logit_bias and sel_bias are constants.
# ---------------------------------------------------------------------------------------
def _as_f64(t):
    """torch tensor (fp32 / bf16) or numpy array -> float64 numpy array of its values."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu").double().numpy()


def _silu(u):
    return u / (1.0 + np.exp(-u))


def _dsilu(u):
    s = 1.0 / (1.0 + np.exp(-u))
    return s * (1.0 + u * (1.0 - s))


def _expert_fwd_bwd(xe, w13e, w2e, g, dye):
    """One expert on its n rows: returns (dx [n, H], dW13 [2F, H], dW2 [H, F], dg [n])."""
    F = w13e.shape[0] // 2
    zg = xe @ w13e[:F].T
    zu = xe @ w13e[F:].T
    h = _silu(zg) * zu                       # unweighted hidden
    da = dye @ w2e                           # dL/d(g h)
    dg = np.sum(da * h, axis=1)
    dh = g[:, None] * da
    dz = np.concatenate([dh * zu * _dsilu(zg), dh * _silu(zg)], axis=1)
    return dz @ w13e, dz.T @ xe, dye.T @ (g[:, None] * h), dg


def layer_backward(x, w_router, logits, topk_idx, w13, w2, dy, router=SOFTMAX_TOPK,
                   route_scale=1.0, logit_bias=None, ws13=None, ws2=None):
    """All gradients of the layer for the routing topk_idx (fixed) -> dict of float64
    arrays: dx [T, H], dw_router [E, H], dw13, dw2, dws13, dws2 (None without a shared
    expert), dlogits [T, E] and dgate [T, k]. Gates are recomputed in float64 from the
    logits: softmax over the selected (biased) logits, or route_scale * s / sum s with
    s = sigmoid(logit + bias) of the selected experts."""
    X, Wr, W13, W2, DY = (_as_f64(v) for v in (x, w_router, w13, w2, dy))
    L = _as_f64(logits) + (0.0 if logit_bias is None else _as_f64(logit_bias)[None, :])
    idx = np.asarray(topk_idx, np.int64)
    T, H = X.shape
    E, k = W13.shape[0], idx.shape[1]
    sel = np.take_along_axis(L, idx, axis=1)                  # [T, k]
    if router == SOFTMAX_TOPK:
        p = np.exp(sel - sel.max(axis=1, keepdims=True))
        gate = p / p.sum(axis=1, keepdims=True)
    else:
        s = 1.0 / (1.0 + np.exp(-sel))
        gate = route_scale * s / s.sum(axis=1, keepdims=True)
    dx = np.zeros((T, H))
    dw13, dw2 = np.zeros_like(W13), np.zeros_like(W2)
    dgate = np.zeros((T, k))
    for e in range(E):
        t, j = np.nonzero(idx == e)          # a token selects an expert at most once
        if t.size == 0:
            continue
        dxe, dw13[e], dw2[e], dgate[t, j] = _expert_fwd_bwd(X[t], W13[e], W2[e], gate[t, j],
                                                            DY[t])
        dx[t] += dxe
    dws13 = dws2 = None
    if ws13 is not None:
        dxs, dws13, dws2, _ = _expert_fwd_bwd(X, _as_f64(ws13), _as_f64(ws2), np.ones(T), DY)
        dx += dxs
    # gates -> selected logits
    if router == SOFTMAX_TOPK:
        dsel = gate * (dgate - np.sum(gate * dgate, axis=1, keepdims=True))
    else:
        ssum = s.sum(axis=1, keepdims=True)
        ds = (route_scale / ssum) * (dgate - np.sum(dgate * gate, axis=1, keepdims=True)
                                     / route_scale)
        dsel = ds * s * (1.0 - s)
    dlogits = np.zeros((T, E))
    np.put_along_axis(dlogits, idx, dsel, axis=1)
    dx += dlogits @ Wr
    return dict(dx=dx, dw_router=dlogits.T @ X, dw13=dw13, dw2=dw2, dws13=dws13, dws2=dws2,
                dlogits=dlogits, dgate=dgate)

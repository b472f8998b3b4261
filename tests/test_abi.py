"""The C-ABI library loads on a host without a GPU, exports every entry point include/moe.h
declares, sizes workspaces on the host and rejects invalid arguments before launching
anything (no call here reaches a kernel)."""
import ctypes as C
import os
import re

import pytest

import moe_inputs as mi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_expert_softmax_amd as m
    return m


def test_exports_every_declared_symbol(moe):
    names = header_functions()
    assert "moe_layer_forward" in names and len(names) >= 10
    for n in names:
        assert hasattr(moe.lib(), n), n
    assert sorted(moe.EXPORTED) == names


def test_status_strings(moe):
    for s in range(5):
        assert moe.status_string(s).startswith("MOE_")
    assert "unknown" in moe.status_string(99)


def cfgc(moe, base="dsv3_bf16", **kw):
    return moe.make_config(mi.CONFIGS[base].replace(**kw))


def ws_size(moe, c, op):
    n = C.c_size_t(0)
    st = moe.lib().moe_workspace_size(C.byref(c), op, C.byref(n))
    return st, n.value


def test_workspace_sizes_on_host(moe):
    for name, cfg in mi.CONFIGS.items():
        if cfg.w_dtype == mi.E4M3:
            continue
        c = moe.make_config(cfg)
        st, p = ws_size(moe, c, moe.OP_PERMUTE)
        assert st == 0 and p > 0
        st, g = ws_size(moe, c, moe.OP_GROUPED_GEMM)
        assert st == 0 and g > 0
        st, l = ws_size(moe, c, moe.OP_LAYER_FORWARD)
        assert st == 0
        # the layer workspace holds x_perm and y_perm (A x H each) at least
        eb = 4 if cfg.act_dtype == mi.F32 else 2
        xb = 1 if cfg.w_dtype == mi.MXFP8 else eb
        assert l >= cfg.T * cfg.k * cfg.H * (xb + eb)
    c = cfgc(moe)
    assert ws_size(moe, c, 17)[0] == 1


@pytest.mark.parametrize("kw,status", [
    (dict(T=0), 1), (dict(k=300), 1), (dict(E=2048, k=8, n_groups=8), 2),
    (dict(H=7000), 2), (dict(F=2000), 2), (dict(n_groups=7), 1), (dict(topk_groups=9), 1),
    (dict(router=5), 1), (dict(route_scale=0.0), 1), (dict(act_dtype=mi.F32), 2),
    (dict(act_dtype=7), 1), (dict(k=33, E=256), 2), (dict(n_groups=128, topk_groups=64), 2),
])
def test_invalid_configs_rejected(moe, kw, status):
    c = cfgc(moe, **kw)
    assert ws_size(moe, c, moe.OP_LAYER_FORWARD)[0] == status
    # every entry point runs the same check first and launches nothing
    L = moe.lib()
    dummy = C.c_void_p(16)
    assert L.moe_route(C.byref(c), dummy, None, None, dummy, dummy, None) == status
    assert L.moe_unpermute_combine(C.byref(c), dummy, dummy, None, dummy, None) == status


def test_softmax_router_rejects_groups(moe):
    c = cfgc(moe, "qwen3_bf16", n_groups=2, topk_groups=1)
    assert ws_size(moe, c, moe.OP_PERMUTE)[0] == 1


def test_null_pointers_rejected(moe):
    L = moe.lib()
    c = cfgc(moe)
    d = C.c_void_p(16)
    assert L.moe_router_logits(C.byref(c), None, d, d, None) == 1
    assert L.moe_route(C.byref(c), None, None, None, d, d, None) == 1
    assert L.moe_permute(C.byref(c), d, d, d, d, d, d, d, d, None, None, None, None, d,
                         1 << 40, None) == 1
    assert L.moe_unpermute_combine(C.byref(c), None, d, None, d, None) == 1
    assert L.moe_layer_forward(C.byref(c), d, None, None, None, None, d, None, d, None, d,
                               None, d, None, d, None, None, None, None, d, 1 << 40, None) == 1
    assert L.moe_workspace_size(C.byref(c), 0, None) == 1
    assert L.moe_quantize_e4m3(None, 1, 1, 128, 128, 1, 128, d, d, None) == 1


def test_workspace_too_small_rejected(moe):
    L = moe.lib()
    c = cfgc(moe)
    d = C.c_void_p(16)
    st, need = ws_size(moe, c, moe.OP_PERMUTE)
    assert L.moe_permute(C.byref(c), d, d, d, d, d, d, d, d, d, None, None, None, d,
                         need - 1, None) == 3
    st, need = ws_size(moe, c, moe.OP_LAYER_FORWARD)
    assert L.moe_layer_forward(C.byref(c), d, d, None, None, None, d, None, d, None, d, None,
                               d, None, d, None, None, None, None, d, need - 1, None) == 3


def test_scale_pointer_consistency(moe):
    L = moe.lib()
    d = C.c_void_p(16)
    c = cfgc(moe)                                   # bf16: scales must be NULL
    st, need = ws_size(moe, c, moe.OP_PERMUTE)
    assert L.moe_permute(C.byref(c), d, d, d, d, d, d, d, d, d, d, None, None, d, need,
                         None) == 1
    c8 = cfgc(moe, w_dtype=mi.E4M3)                 # e4m3: x_perm scales required
    st, need8 = ws_size(moe, c8, moe.OP_PERMUTE)
    assert L.moe_permute(C.byref(c8), d, d, d, d, d, d, d, d, d, None, None, None, d, need8,
                         None) == 1


def test_quantize_argument_checks(moe):
    L = moe.lib()
    d = C.c_void_p(16)
    assert L.moe_quantize_e4m3(d, 1, 1, 128, 100, 1, 128, d, d, None) == 1
    assert L.moe_quantize_e4m3(d, 1, 1, 100, 128, 128, 128, d, d, None) == 1
    assert L.moe_quantize_e4m3(d, 1, 1, 128, 128, 64, 128, d, d, None) == 2
    assert L.moe_quantize_e4m3(d, 5, 1, 128, 128, 1, 128, d, d, None) == 1


def test_layout_validation(moe):
    """Layout fields: only 0/1; fp32 supports row-major only; the pack call checks sizes."""
    c = cfgc(moe, a_layout=2)
    assert ws_size(moe, c, moe.OP_PERMUTE)[0] == 1               # MOE_ERR_INVALID_ARG
    c = cfgc(moe, base="tiny_fp32", w_layout=1)
    assert ws_size(moe, c, moe.OP_PERMUTE)[0] == 2               # MOE_ERR_UNSUPPORTED
    c = cfgc(moe, a_layout=1, w_layout=1)
    st, n = ws_size(moe, c, moe.OP_LAYER_FORWARD)
    assert st == 0 and n > 0
    L = moe.lib()
    p = C.c_void_p(0x1000)
    q = C.c_void_p(0x2000)
    assert L.moe_pack_kblock(p, 1, 16, 24, 2, q, None) == 1      # 48 bytes per row: not 64k
    assert L.moe_pack_kblock(p, 1, 16, 32, 3, q, None) == 1      # element size
    assert L.moe_pack_kblock(p, 0, 16, 32, 2, q, None) == 1      # no matrices
    assert L.moe_pack_kblock(p, 1, 16, 32, 2, p, None) == 1      # in place


def test_stage_event_argument_checks(moe):
    """moe_set_stage_events: NULL turns recording off; a wrong count or a NULL handle is an
    invalid argument (host-side checks only, no HIP call is made)."""
    L = moe.lib()
    assert L.moe_set_stage_events(None, 0) == 0
    arr = (C.c_void_p * 7)(*([0x1000] * 7))
    assert L.moe_set_stage_events(arr, 6) == 1
    arr[3] = None
    assert L.moe_set_stage_events(arr, 7) == 1
    assert L.moe_set_stage_events(None, 0) == 0


def test_layer_backward_argument_checks(moe):
    """Workspace query and host-side rejections of moe_layer_backward (no GPU call)."""
    c = cfgc(moe, base="dsv3_bf16")
    st, n = ws_size(moe, c, moe.OP_LAYER_BACKWARD)
    assert st == 0 and n > 0
    assert ws_size(moe, cfgc(moe, base="mixtral_bf16"), moe.OP_LAYER_BACKWARD)[0] == 2  # E = 8
    assert ws_size(moe, cfgc(moe, base="tiny_fp32"), moe.OP_LAYER_BACKWARD)[0] == 2    # fp32
    # weights in either layout; activations row-major only
    assert ws_size(moe, cfgc(moe, base="dsv3_bf16", w_layout=1), moe.OP_LAYER_BACKWARD) == (0, n)
    assert ws_size(moe, cfgc(moe, base="dsv3_bf16", a_layout=1, w_layout=1),
                   moe.OP_LAYER_BACKWARD)[0] == 2
    assert ws_size(moe, cfgc(moe, base="dsv3_bf16", w_layout=1),
                   moe.OP_GROUPED_GEMM_BWD)[0] == 0
    L = moe.lib()
    p = C.c_void_p(0x1000)
    args = [p] * 19
    # missing dy
    a = list(args)
    a[10] = None
    assert L.moe_layer_backward(C.byref(c), *a, C.c_size_t(n), None) == 1
    # workspace too small
    assert L.moe_layer_backward(C.byref(c), *args, C.c_size_t(n - 1), None) == 3


def test_training_pair_argument_checks(moe):
    """moe_layer_forward_train / moe_layer_backward_saved: the saved buffer's size (Z and act
    of the routed rows and of the shared expert, bf16, each region 256-byte aligned) and the
    host-side rejections (no GPU call)."""
    cfg = mi.CONFIGS["dsv3_bf16"]
    c = moe.make_config(cfg)
    st, n = ws_size(moe, c, moe.OP_LAYER_SAVED)
    A, F, sF, T = cfg.T * cfg.k, cfg.F, cfg.shared_F, cfg.T
    al = lambda b: (b + 255) // 256 * 256
    assert st == 0 and n == al(A * 2 * F * 2) + al(A * F * 2) + al(T * 2 * sF * 2) + al(T * sF * 2)
    assert ws_size(moe, cfgc(moe, base="dsv3_fp8_skew"), moe.OP_LAYER_SAVED)[0] == 2   # e4m3
    assert ws_size(moe, cfgc(moe, base="tiny_fp32"), moe.OP_LAYER_SAVED)[0] == 2       # fp32
    assert ws_size(moe, cfgc(moe, capacity_factor=1.25), moe.OP_LAYER_SAVED)[0] == 2
    # K-blocked weights are fine on both sides; K-blocked activations are not
    assert ws_size(moe, cfgc(moe, w_layout=1), moe.OP_LAYER_SAVED) == (0, n)
    assert ws_size(moe, cfgc(moe, a_layout=1, w_layout=1), moe.OP_LAYER_SAVED)[0] == 2
    L = moe.lib()
    p = C.c_void_p(0x1000)
    big = C.c_size_t(1 << 40)
    # forward: x .. counts_out (14 pointers), saved, saved_bytes, ws, ws_bytes, stream
    fwd = [p] * 14
    assert L.moe_layer_forward_train(C.byref(c), *fwd, None, C.c_size_t(n), p, big, None) == 1
    assert L.moe_layer_forward_train(C.byref(c), *fwd, p, C.c_size_t(n - 1), p, big, None) == 3
    cf8 = cfgc(moe, base="dsv3_fp8_skew")
    assert L.moe_layer_forward_train(C.byref(cf8), *fwd, p, big, p, big, None) == 2
    # backward: x .. ws2 (10 pointers), saved, saved_bytes, dy .. dlogits_out (8), ws, ...
    head, tail = [p] * 10, [p] * 8
    assert L.moe_layer_backward_saved(C.byref(c), *head, None, C.c_size_t(n), *tail, p, big,
                                      None) == 1
    assert L.moe_layer_backward_saved(C.byref(c), *head, p, C.c_size_t(n - 1), *tail, p, big,
                                      None) == 3
    ck = cfgc(moe, a_layout=1, w_layout=1)
    assert L.moe_layer_backward_saved(C.byref(ck), *head, p, big, *tail, p, big, None) == 2


def test_capacity_and_stats_argument_checks(moe):
    """capacity_factor must be finite and >= 0; the backward calls need it 0; moe_route_stats
    sizes and checks its workspace (host-side checks only)."""
    assert ws_size(moe, cfgc(moe, capacity_factor=-1.0), moe.OP_PERMUTE)[0] == 1
    assert ws_size(moe, cfgc(moe, capacity_factor=float("inf")), moe.OP_PERMUTE)[0] == 1
    assert ws_size(moe, cfgc(moe, capacity_factor=float("nan")), moe.OP_PERMUTE)[0] == 1
    assert ws_size(moe, cfgc(moe, capacity_factor=1.25), moe.OP_LAYER_FORWARD)[0] == 0
    assert ws_size(moe, cfgc(moe, capacity_factor=1.25), moe.OP_LAYER_BACKWARD)[0] == 2
    assert ws_size(moe, cfgc(moe, capacity_factor=1.25), moe.OP_GROUPED_GEMM_BWD)[0] == 2
    c = cfgc(moe)
    st, n = ws_size(moe, c, moe.OP_ROUTE_STATS)
    # per-block sums of 4 tokens, then of 16 of those, E floats each
    T, E = c.T, c.E
    r1 = (T + 3) // 4
    assert st == 0 and n >= (r1 + (r1 + 15) // 16) * E * 4
    L = moe.lib()
    d = C.c_void_p(16)
    assert L.moe_route_stats(C.byref(c), d, None, None, d, d, d, d, n - 1, None) == 3
    assert L.moe_route_stats(C.byref(c), d, None, None, d, d, None, d, n, None) == 1


def test_mxfp8_argument_checks(moe):
    """MXFP8 takes row-major activations (any weight layout); the quantiser and the scale
    packing check their sizes (host-side checks only)."""
    assert ws_size(moe, cfgc(moe, w_dtype=mi.MXFP8), moe.OP_LAYER_FORWARD)[0] == 0
    assert ws_size(moe, cfgc(moe, w_dtype=mi.MXFP8, w_layout=1), moe.OP_LAYER_FORWARD)[0] == 0
    assert ws_size(moe, cfgc(moe, w_dtype=mi.MXFP8, a_layout=1), moe.OP_PERMUTE)[0] == 2
    L = moe.lib()
    p, q = C.c_void_p(0x1000), C.c_void_p(0x2000)
    assert L.moe_quantize_mx(p, 1, 4, 48, q, q, None) == 1          # cols not a multiple of 32
    assert L.moe_quantize_mx(p, 7, 4, 64, q, q, None) == 1          # input dtype
    assert L.moe_quantize_mx(None, 1, 4, 64, q, q, None) == 1
    assert L.moe_pack_mx_scales(p, 1, 16, 6, q, None) == 1          # cols not a multiple of 4
    assert L.moe_pack_mx_scales(p, 1, 16, 8, p, None) == 1          # in place
    assert L.moe_pack_mx_scales(p, 0, 16, 8, q, None) == 1          # no matrices


def test_fp8_activation_size_limit(moe):
    """The fp8 GEMMs address one-byte activation rows with 32-bit offsets, so every fp8
    activation matrix must stay below 4 GiB: (T*k + T) * max(H, F, shared_F) < 2^32. At the
    limit the configuration is rejected on the host (nothing launched); bf16 with the same
    shape is accepted (its GEMMs keep 64-bit row addresses)."""
    # (70000*8 + 70000) * 7168 = 4.5e9 >= 2^32
    big = dict(T=70000, H=7168)
    for dt in (mi.E4M3, mi.MXFP8):
        assert ws_size(moe, cfgc(moe, w_dtype=dt, **big), moe.OP_LAYER_FORWARD)[0] == 2
        assert ws_size(moe, cfgc(moe, w_dtype=dt, **big), moe.OP_GROUPED_GEMM)[0] == 2
        # below the limit: 60000 * 9 * 7168 = 3.9e9 < 2^32
        assert ws_size(moe, cfgc(moe, w_dtype=dt, T=60000, H=7168), moe.OP_PERMUTE)[0] == 0
    assert ws_size(moe, cfgc(moe, **big), moe.OP_LAYER_FORWARD)[0] == 0
    # the widest of H, F and shared_F counts
    assert ws_size(moe, cfgc(moe, w_dtype=mi.E4M3, T=60000, H=1024, F=8192, shared_F=128),
                   moe.OP_PERMUTE)[0] == 2


"""MXFP8 path (e4m3 elements, one E8M0 scale per 1 x 32 block along K) vs the CPU oracle on
small copies of the DeepSeek-V3 layer: the quantiser and the permute bit-exact, the expert
GEMMs (scales applied by the block-scaled MFMA) and the whole layer within the fp8
tolerance (6e-2 of max|ref|) against the oracle's own MXFP8 simulation. The oracle quantises
with its own code and never sees a GPU value."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from helpers import SMALL_MX, mx_codes_close, rel_err, to_dev

pytestmark = pytest.mark.gpu
TOL8 = 6e-2


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_expert_softmax_amd as m
    return m


_CACHE = {}


def case(name):
    if name in _CACHE:
        return _CACHE[name]
    cfg = SMALL_MX[name]
    inp = mi.make_inputs(cfg)
    logits = oracle.router_logits(inp.x, inp.w_router)
    npy = lambda t: None if t is None else t.numpy()  # noqa: E731
    idx, gate = oracle.route_cfg(cfg, logits, npy(inp.logit_bias), npy(inp.sel_bias))
    perm = oracle.permute(idx, gate, cfg.E)
    q = dict(w13=oracle.mx_quant(inp.w13), w2=oracle.mx_quant(inp.w2),
             ws13=oracle.mx_quant(inp.ws13), ws2=oracle.mx_quant(inp.ws2),
             x=oracle.mx_quant(inp.x))
    c = dict(cfg=cfg, inp=inp, logits=logits, idx=idx, gate=gate, perm=perm, q=q)
    _CACHE[name] = c
    return c


NAMES = list(SMALL_MX)


def edge_values(dtype):
    """Blocks that exercise the MX rule: all zero, a single nonzero, exact powers of two,
    values just below and above the saturating range [448, 512) of a block's scaled
    maximum, bf16 subnormals, both signed zeros, and huge and tiny magnitudes."""
    rows = []
    z = np.zeros(32, np.float32)
    rows.append(z.copy())
    one = z.copy(); one[5] = -3.0; rows.append(one)
    rows.append(np.exp2(np.arange(-12, 20, dtype=np.float32)))
    r = np.linspace(1.0, 1.999, 32, dtype=np.float32) * np.float32(256.0)   # amax < 512
    rows.append(r)
    r = r.copy(); r[0] = 511.0; rows.append(r)
    rows.append(np.full(32, 1e-39, np.float32) * np.arange(32, dtype=np.float32))
    sz = z.copy(); sz[::2] = -0.0; sz[1] = 1e-3; rows.append(sz)
    rows.append(np.linspace(-3e38, 3e38, 32, dtype=np.float32))
    rows.append(np.linspace(-1e-30, 1e-30, 32, dtype=np.float32))
    rng = np.random.default_rng(3)
    rows.append((rng.standard_normal(32) * 1e4).astype(np.float32))
    a = np.stack(rows)
    t = torch.from_numpy(a)
    return t.to(dtype) if dtype == torch.bfloat16 else t


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quantize_mx_edge_blocks_bit_exact(moe, dtype):
    t = edge_values(dtype)
    print(f"[mx quantize edges] {dtype}", flush=True)
    qg, sg = moe.quantize_mx(t.cuda())
    torch.cuda.synchronize()
    qo, so = oracle.mx_quant(t)
    np.testing.assert_array_equal(sg.cpu().numpy(), so)
    np.testing.assert_array_equal(qg.cpu().numpy(), qo)


@pytest.mark.parametrize("name", NAMES)
def test_quantize_mx_bit_exact(moe, name):
    c = case(name)
    inp = c["inp"]
    print(f"[mx quantize] {name}", flush=True)
    for key in ("w13", "w2", "ws13", "ws2", "x"):
        qg, sg = moe.quantize_mx(getattr(inp, key).cuda())
        torch.cuda.synchronize()
        qo, so = c["q"][key]
        np.testing.assert_array_equal(sg.cpu().numpy(), so, err_msg=key)
        np.testing.assert_array_equal(qg.cpu().numpy(), qo, err_msg=key)


@pytest.mark.parametrize("name", NAMES)
def test_permute_mx_bit_exact(moe, name):
    c = case(name)
    cfg, inp, perm = c["cfg"], c["inp"], c["perm"]
    print(f"[mx permute] {name}", flush=True)
    out = moe.permute(cfg, inp.x.cuda(), torch.from_numpy(c["idx"]).cuda(),
                      torch.from_numpy(c["gate"]).cuda(), want_x_q=True)
    torch.cuda.synchronize()
    for key in ("counts", "offsets", "pos", "src"):
        np.testing.assert_array_equal(out[key].cpu().numpy(), perm[key], err_msg=key)
    xq, xs = c["q"]["x"]
    np.testing.assert_array_equal(out["x_perm"].cpu().numpy(), oracle.gather_rows(xq, perm["pos"]))
    np.testing.assert_array_equal(out["x_perm_scales"].cpu().numpy(),
                                  oracle.gather_rows(xs, perm["pos"]))
    np.testing.assert_array_equal(out["x_q"].cpu().numpy(), xq)
    np.testing.assert_array_equal(out["x_q_scales"].cpu().numpy(), xs)


@pytest.mark.parametrize("name", NAMES)
def test_grouped_gemm_mx(moe, name):
    c = case(name)
    cfg, perm, q = c["cfg"], c["perm"], c["q"]
    print(f"[mx grouped gemm] {name}", flush=True)
    xq, xs = q["x"]
    xp_q = oracle.gather_rows(xq, perm["pos"])
    xp_s = oracle.gather_rows(xs, perm["pos"])
    T8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    W = {k: T8(q[k][0]) for k in ("w13", "w2", "ws13", "ws2")}
    S = {k: T8(q[k][1]) for k in ("w13", "w2", "ws13", "ws2")}
    if cfg.w_layout:           # K-blocked codes take blocked scales
        W = {k: moe.pack_kblock(v) for k, v in W.items()}
        S = {k: moe.pack_mx_scales(v) for k, v in S.items()}
    out = moe.grouped_gemm_swiglu(
        cfg, T8(xp_q), T8(perm["offsets"]), T8(perm["gate_perm"]), W["w13"], W["w2"],
        x_perm_scales=T8(xp_s), w13_scales=S["w13"], w2_scales=S["w2"],
        x_shared=T8(xq), x_shared_scales=T8(xs), ws13=W["ws13"],
        ws13_scales=S["ws13"], ws2=W["ws2"], ws2_scales=S["ws2"])
    torch.cuda.synchronize()
    rows = np.arange(cfg.A)
    kw = dict(x_scales=xp_s, w13_scales=q["w13"][1], w2_scales=q["w2"][1], mx=True)
    _, act_pre, _ = oracle.expert_rows(xp_q, perm["offsets"], perm["gate_perm"], q["w13"][0],
                                       q["w2"][0], rows, quant_act=False, **kw)
    _, _, y_ref = oracle.expert_rows(xp_q, perm["offsets"], perm["gate_perm"], q["w13"][0],
                                     q["w2"][0], rows, quant_act=True, **kw)
    ratio, dfrac, sdiff, sfrac = mx_codes_close(out["act"].cpu().numpy(),
                                                out["act_scales"].cpu().numpy(), act_pre)
    print(f"   act codes: max err / (1 step + saturation + 1e-3 range) {ratio:.2f}, differing "
          f"{dfrac:.2e}; scale codes: max diff {sdiff}, differing {sfrac:.2e}", flush=True)
    assert ratio <= 1.0 and dfrac <= 0.02 and sdiff <= 1 and sfrac <= 1e-3
    e_y = rel_err(out["y_perm"], y_ref)
    _, _, ys_ref = oracle.expert_rows(xq, None, None, q["ws13"][0], q["ws2"][0],
                                      np.arange(cfg.T), x_scales=xs, w13_scales=q["ws13"][1],
                                      w2_scales=q["ws2"][1], quant_act=True, mx=True)
    e_s = rel_err(out["shared_y"], ys_ref)
    print(f"   y_perm {e_y:.3e}  shared_y {e_s:.3e}", flush=True)
    assert e_y <= TOL8 and e_s <= TOL8


@pytest.mark.parametrize("name", NAMES)
def test_layer_forward_mx(moe, name):
    c = case(name)
    cfg, inp, q = c["cfg"], c["inp"], c["q"]
    print(f"[mx layer forward] {name}", flush=True)
    w = {k: moe.quantize_mx(getattr(inp, k).cuda()) for k in ("w13", "w2", "ws13", "ws2")}
    if cfg.w_layout:
        w = {k: (moe.pack_kblock(v[0]), moe.pack_mx_scales(v[1])) for k, v in w.items()}
    y, ex = moe.layer_forward(cfg, inp.x.cuda(), inp.w_router.cuda(), w["w13"][0], w["w2"][0],
                              to_dev(inp.logit_bias), to_dev(inp.sel_bias),
                              torch.from_numpy(c["logits"]).cuda(), w13_scales=w["w13"][1],
                              w2_scales=w["w2"][1], ws13=w["ws13"][0],
                              ws13_scales=w["ws13"][1], ws2=w["ws2"][0],
                              ws2_scales=w["ws2"][1], want=("topk_idx", "counts"))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ex["topk_idx"].cpu().numpy(), c["idx"])
    np.testing.assert_array_equal(ex["counts"].cpu().numpy(), c["perm"]["counts"])
    ref = oracle.layer_tokens(inp.x, c["idx"], c["gate"], q["w13"][0], q["w2"][0],
                              np.arange(cfg.T), q["ws13"][0], q["ws2"][0], fp8="mx",
                              w13_scales=q["w13"][1], w2_scales=q["w2"][1],
                              ws13_scales=q["ws13"][1], ws2_scales=q["ws2"][1])
    e = rel_err(y, ref)
    print(f"   y {e:.3e}", flush=True)
    assert e <= TOL8


def test_pack_mx_scales_bit_exact(moe):
    """[n, rows, cols] scale bytes -> [n][cols/4][rows][4]: a numpy transpose of 4-byte words."""
    rng = np.random.default_rng(12)
    a = rng.integers(0, 256, size=(3, 40, 28), dtype=np.uint8)
    out = moe.pack_mx_scales(torch.from_numpy(a).cuda())
    torch.cuda.synchronize()
    ref = a.reshape(3, 40, 7, 4).transpose(0, 2, 1, 3).reshape(3, 40, 28)
    np.testing.assert_array_equal(out.cpu().numpy(), ref)

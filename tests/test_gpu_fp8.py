"""e4m3 path vs the CPU oracle on small copies of the skewed DeepSeek-V3-shaped workload:
the quantisers and the e4m3 permute bit-exact, the block-scaled expert GEMMs and the whole
layer within the fp8 tolerance (6e-2 of max|ref|) against the oracle's own simulated e4m3
quantisation. The oracle always quantises with its own code; it never sees a GPU value."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from helpers import SMALL_FP8, block, e4m3_codes_close, rel_err, to_dev, unblock

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
    cfg = SMALL_FP8[name]
    inp = mi.make_inputs(cfg)
    logits = oracle.router_logits(inp.x, inp.w_router)
    lb = inp.logit_bias.numpy()
    sb = inp.sel_bias.numpy()
    idx, gate = oracle.route_cfg(cfg, logits, lb, sb)
    perm = oracle.permute(idx, gate, cfg.E)
    q = dict(w13=oracle.quant_weight(inp.w13), w2=oracle.quant_weight(inp.w2),
             ws13=oracle.quant_weight(inp.ws13), ws2=oracle.quant_weight(inp.ws2),
             x=oracle.quant_rows(inp.x))
    c = dict(cfg=cfg, inp=inp, logits=logits, idx=idx, gate=gate, perm=perm, q=q)
    _CACHE[name] = c
    return c


NAMES = list(SMALL_FP8)


def gpu_quant(moe, w):
    qq, ss = moe.quantize_e4m3(w.cuda(), 128)
    return qq, ss


def maybe_block(cfg, t, which):
    on = cfg.a_layout if which == "a" else cfg.w_layout
    return block(t) if on else t


@pytest.mark.parametrize("name", NAMES)
def test_quantizers_bit_exact(moe, name):
    c = case(name)
    inp = c["inp"]
    print(f"[fp8 quantizers] {name}", flush=True)
    for key in ("w13", "w2", "ws13", "ws2"):
        qg, sg = moe.quantize_e4m3(getattr(inp, key).cuda(), 128)
        torch.cuda.synchronize()
        qo, so = c["q"][key]
        np.testing.assert_array_equal(qg.cpu().numpy(), qo, err_msg=key)
        np.testing.assert_array_equal(sg.cpu().numpy(), so, err_msg=key)
    qg, sg = moe.quantize_e4m3(inp.x.cuda(), 1)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(qg.cpu().numpy(), c["q"]["x"][0])
    np.testing.assert_array_equal(sg.cpu().numpy(), c["q"]["x"][1])


@pytest.mark.parametrize("name", NAMES)
def test_permute_e4m3_bit_exact(moe, name):
    c = case(name)
    cfg, inp, perm = c["cfg"], c["inp"], c["perm"]
    print(f"[fp8 permute] {name}", flush=True)
    out = moe.permute(cfg, inp.x.cuda(), torch.from_numpy(c["idx"]).cuda(),
                      torch.from_numpy(c["gate"]).cuda(), want_x_q=True)
    torch.cuda.synchronize()
    for key in ("counts", "offsets", "pos", "src"):
        np.testing.assert_array_equal(out[key].cpu().numpy(), perm[key], err_msg=key)
    xq, xs = c["q"]["x"]
    xp = out["x_perm"].cpu()
    if cfg.a_layout:
        xp = unblock(xp, cfg.A, cfg.H)
    np.testing.assert_array_equal(xp.numpy(), oracle.gather_rows(xq, perm["pos"]))
    np.testing.assert_array_equal(out["x_perm_scales"].cpu().numpy(),
                                  oracle.gather_rows(xs, perm["pos"]))
    np.testing.assert_array_equal(out["x_q"].cpu().numpy(), xq)
    np.testing.assert_array_equal(out["x_q_scales"].cpu().numpy(), xs)


def dequant_rows(q, s):
    """codes [R, C] uint8 + scales [R, C/128] -> float64 values (oracle's e4m3 table)."""
    v = oracle.e4m3_decode_array(np.asarray(q))
    return v * np.repeat(np.asarray(s, np.float64), 128, axis=1)


@pytest.mark.parametrize("name", NAMES)
def test_grouped_gemm_e4m3(moe, name):
    c = case(name)
    cfg, inp, perm, q = c["cfg"], c["inp"], c["perm"], c["q"]
    print(f"[fp8 grouped gemm] {name}", flush=True)
    xq, xs = q["x"]
    xp_q = oracle.gather_rows(xq, perm["pos"])
    xp_s = oracle.gather_rows(xs, perm["pos"])
    T8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    w13q, w13s = gpu_quant(moe, inp.w13)
    w2q, w2s = gpu_quant(moe, inp.w2)
    s13q, s13s = gpu_quant(moe, inp.ws13)
    s2q, s2s = gpu_quant(moe, inp.ws2)
    if cfg.w_layout:
        w13q, w2q, s13q, s2q = (moe.pack_kblock(t) for t in (w13q, w2q, s13q, s2q))
    xpq = T8(xp_q)
    if cfg.a_layout:
        xpq = moe.pack_kblock(xpq)
    out = moe.grouped_gemm_swiglu(cfg, xpq, T8(perm["offsets"]), T8(perm["gate_perm"]),
                                  w13q, w2q, x_perm_scales=T8(xp_s), w13_scales=w13s,
                                  w2_scales=w2s, x_shared=T8(xq), x_shared_scales=T8(xs),
                                  ws13=s13q, ws13_scales=s13s, ws2=s2q, ws2_scales=s2s)
    torch.cuda.synchronize()
    rows = np.arange(cfg.A)
    _, act_ref, y_ref = oracle.expert_rows(
        xp_q, perm["offsets"], perm["gate_perm"], q["w13"][0], q["w2"][0], rows,
        x_scales=xp_s, w13_scales=q["w13"][1], w2_scales=q["w2"][1], quant_act=True)
    act = out["act"].cpu()
    if cfg.a_layout:
        act = unblock(act, cfg.A, cfg.F)
    _, act_pre, _ = oracle.expert_rows(
        xp_q, perm["offsets"], perm["gate_perm"], q["w13"][0], q["w2"][0], rows,
        x_scales=xp_s, w13_scales=q["w13"][1], w2_scales=q["w2"][1], quant_act=False)
    ratio, dfrac, srel = e4m3_codes_close(act.numpy(), out["act_scales"].cpu().numpy(), act_pre)
    print(f"   act codes: max err / (1 step + 1e-3 range) {ratio:.2f}, differing {dfrac:.2e}, scale rel {srel:.1e}",
          flush=True)
    assert ratio <= 1.0 and dfrac <= 0.02 and srel <= 1e-4
    act_gpu = dequant_rows(act.numpy(), out["act_scales"].cpu().numpy())
    e_act = rel_err(act_gpu, act_ref)
    e_y = rel_err(out["y_perm"], y_ref)
    _, _, ys_ref = oracle.expert_rows(xq, None, None, q["ws13"][0], q["ws2"][0], np.arange(cfg.T),
                                      x_scales=xs, w13_scales=q["ws13"][1],
                                      w2_scales=q["ws2"][1], quant_act=True)
    e_s = rel_err(out["shared_y"], ys_ref)
    print(f"   act {e_act:.3e}  y_perm {e_y:.3e}  shared_y {e_s:.3e}", flush=True)
    assert e_y <= TOL8 and e_s <= TOL8


@pytest.mark.parametrize("name", NAMES)
def test_layer_forward_e4m3(moe, name):
    c = case(name)
    cfg, inp, q = c["cfg"], c["inp"], c["q"]
    print(f"[fp8 layer forward] {name}", flush=True)
    w13q, w13s = gpu_quant(moe, inp.w13)
    w2q, w2s = gpu_quant(moe, inp.w2)
    s13q, s13s = gpu_quant(moe, inp.ws13)
    s2q, s2s = gpu_quant(moe, inp.ws2)
    if cfg.w_layout:
        w13q, w2q, s13q, s2q = (moe.pack_kblock(t) for t in (w13q, w2q, s13q, s2q))
    y, ex = moe.layer_forward(cfg, inp.x.cuda(), inp.w_router.cuda(), w13q, w2q,
                              to_dev(inp.logit_bias), to_dev(inp.sel_bias),
                              torch.from_numpy(c["logits"]).cuda(), w13_scales=w13s,
                              w2_scales=w2s, ws13=s13q, ws13_scales=s13s, ws2=s2q,
                              ws2_scales=s2s, want=("topk_idx", "counts"))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ex["topk_idx"].cpu().numpy(), c["idx"])
    np.testing.assert_array_equal(ex["counts"].cpu().numpy(), c["perm"]["counts"])
    ref = oracle.layer_tokens(inp.x, c["idx"], c["gate"], q["w13"][0], q["w2"][0],
                              np.arange(cfg.T), q["ws13"][0], q["ws2"][0], fp8=True,
                              w13_scales=q["w13"][1], w2_scales=q["w2"][1],
                              ws13_scales=q["ws13"][1], ws2_scales=q["ws2"][1])
    e = rel_err(y, ref)
    print(f"   y {e:.3e}", flush=True)
    assert e <= TOL8

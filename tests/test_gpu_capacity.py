"""Token-dropping routing (expert capacity) and the fused load-balancing statistics vs the
CPU oracle: the capacity permutation bit-exact (counts, offsets, pos with -1 for dropped
slots, src and gate_perm of the kept rows), the combine skipping dropped slots, the whole
layer with drops within each dtype's tolerance, and the routing statistics (top-k
bit-exact, mean router probabilities within 1e-5) on ragged token counts."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from helpers import SMALL, SMALL_FP8, SMALL_MX, rel_err, to_dev, tol

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_expert_softmax_amd as m
    return m


# workloads with drops: the skewed fp8 router overflows its hot experts at any factor near 1
CASES = {
    "tiny_fp32_cf1": SMALL["tiny_fp32"].replace(capacity_factor=1.0),
    "qwen3_small_cf1": SMALL["qwen3_small"].replace(capacity_factor=1.0),
    "dsv3_small_cf1.25": SMALL["dsv3_small"].replace(capacity_factor=1.25),
    "dsv3_fp8_small_cf1": SMALL_FP8["dsv3_fp8_small"].replace(capacity_factor=1.0),
    "dsv3_fp8_kblock_cf2": SMALL_FP8["dsv3_fp8_small_kblock"].replace(capacity_factor=2.0),
    "dsv3_mx_small_cf1": SMALL_MX["dsv3_mx_small"].replace(capacity_factor=1.0),
}
_CACHE = {}


def case(name):
    if name in _CACHE:
        return _CACHE[name]
    cfg = CASES[name]
    inp = mi.make_inputs(cfg)
    logits = oracle.router_logits(inp.x, inp.w_router)
    npy = lambda t: None if t is None else t.numpy()  # noqa: E731
    idx, gate = oracle.route_cfg(cfg, logits, npy(inp.logit_bias), npy(inp.sel_bias))
    cap = oracle.expert_capacity(cfg.capacity_factor, cfg.T, cfg.k, cfg.E)
    perm = oracle.permute(idx, gate, cfg.E, capacity=cap)
    c = dict(cfg=cfg, inp=inp, logits=logits, idx=idx, gate=gate, perm=perm, cap=cap)
    _CACHE[name] = c
    return c


NAMES = list(CASES)


@pytest.mark.parametrize("name", NAMES)
def test_capacity_permute_bit_exact(moe, name):
    c = case(name)
    cfg, perm = c["cfg"], c["perm"]
    dropped = int((perm["pos"] < 0).sum())
    print(f"[capacity permute] {name}: capacity {c['cap']}, dropped {dropped} of {cfg.A}",
          flush=True)
    assert dropped > 0
    out = moe.permute(cfg, c["inp"].x.cuda(), torch.from_numpy(c["idx"]).cuda(),
                      torch.from_numpy(c["gate"]).cuda())
    torch.cuda.synchronize()
    for key in ("counts", "offsets", "pos"):
        np.testing.assert_array_equal(out[key].cpu().numpy(), perm[key], err_msg=key)
    n = int(perm["offsets"][cfg.E])
    np.testing.assert_array_equal(out["src"].cpu().numpy()[:n], perm["src"][:n])
    np.testing.assert_array_equal(out["gate_perm"].cpu().numpy()[:n], perm["gate_perm"][:n])


@pytest.mark.parametrize("name", ["qwen3_small_cf1", "dsv3_small_cf1.25"])
def test_combine_skips_dropped_slots(moe, name):
    c = case(name)
    cfg, perm = c["cfg"], c["perm"]
    print(f"[capacity combine] {name}", flush=True)
    g = torch.Generator().manual_seed(11)
    y_perm = torch.randn(cfg.A, cfg.H, generator=g).to(torch.bfloat16)
    y = moe.unpermute_combine(cfg, y_perm.cuda(), torch.from_numpy(perm["pos"]).cuda())
    torch.cuda.synchronize()
    ref = oracle.combine(y_perm, perm["pos"])
    e = rel_err(y, ref)
    print(f"   y {e:.3e}", flush=True)
    # the fp32 sum of the kept slots, rounded once to bf16: |error| <= 2^-9 |y| <= 2^-9 max|y|
    assert e <= 2.0 ** -8


def _weights(moe, cfg, inp):
    keys = ("w13", "w2", "ws13", "ws2")
    W = {k: getattr(inp, k) for k in keys}
    sc = {k + "_scales": None for k in keys}
    q = {}
    if cfg.w_dtype == mi.E4M3:
        for k in keys:
            if W[k] is not None:
                q[k] = oracle.quant_weight(W[k])
                W[k], sc[k + "_scales"] = moe.quantize_e4m3(W[k].cuda(), 128)
    elif cfg.w_dtype == mi.MXFP8:
        for k in keys:
            if W[k] is not None:
                q[k] = oracle.mx_quant(W[k])
                W[k], sc[k + "_scales"] = moe.quantize_mx(W[k].cuda())
    W = {k: (None if v is None else v.cuda()) for k, v in W.items()}
    if cfg.w_layout:
        W = {k: (None if v is None else moe.pack_kblock(v)) for k, v in W.items()}
        if cfg.w_dtype == mi.MXFP8:
            sc = {k: (None if v is None else moe.pack_mx_scales(v)) for k, v in sc.items()}
    return W, sc, q


@pytest.mark.parametrize("name", NAMES)
def test_layer_forward_with_capacity(moe, name):
    c = case(name)
    cfg, inp, perm = c["cfg"], c["inp"], c["perm"]
    print(f"[capacity layer] {name}", flush=True)
    W, sc, q = _weights(moe, cfg, inp)
    y, ex = moe.layer_forward(cfg, inp.x.cuda(), inp.w_router.cuda(), W["w13"], W["w2"],
                              to_dev(inp.logit_bias), to_dev(inp.sel_bias),
                              torch.from_numpy(c["logits"]).cuda(), ws13=W["ws13"],
                              ws2=W["ws2"], want=("topk_idx", "counts"), **sc)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ex["topk_idx"].cpu().numpy(), c["idx"])
    np.testing.assert_array_equal(ex["counts"].cpu().numpy(), perm["counts"])
    idx_kept = oracle.drop_slots(c["idx"], perm["pos"])
    T = np.arange(cfg.T)
    if cfg.w_dtype == mi.E4M3 or cfg.w_dtype == mi.MXFP8:
        mode = True if cfg.w_dtype == mi.E4M3 else "mx"
        ref = oracle.layer_tokens(inp.x, idx_kept, c["gate"], q["w13"][0], q["w2"][0], T,
                                  q["ws13"][0] if "ws13" in q else None,
                                  q["ws2"][0] if "ws2" in q else None, fp8=mode,
                                  w13_scales=q["w13"][1], w2_scales=q["w2"][1],
                                  ws13_scales=q["ws13"][1] if "ws13" in q else None,
                                  ws2_scales=q["ws2"][1] if "ws2" in q else None)
    else:
        ref = oracle.layer_tokens(inp.x, idx_kept, c["gate"], inp.w13, inp.w2, T, inp.ws13,
                                  inp.ws2)
    e = rel_err(y, ref)
    print(f"   y {e:.3e} (tol {tol(cfg):.0e})", flush=True)
    assert e <= tol(cfg)


STATS = {
    "softmax_E8_T1001": (mi.CONFIGS["tiny_fp32"].replace(T=1001), None),
    "softmax_E128_T513": (mi.scaled(mi.CONFIGS["qwen3_bf16"], T=513, H=256, F=128), None),
    "sigmoid_E256_T770": (mi.scaled(mi.CONFIGS["dsv3_bf16"], T=770, H=256, F=128), None),
    "sigmoid_skew_T1": (mi.scaled(mi.CONFIGS["dsv3_fp8_skew"], T=1, H=256, F=128), None),
    "sigmoid_E48_T99": (mi.scaled(mi.CONFIGS["dsv3_bf16"], T=99, H=256, F=128, E=48, k=4,
                                  n_groups=4, topk_groups=2), None),
    # the largest E the ABI takes: 16 keys per lane, a 16 KB LDS block sum
    "softmax_E1024_T37": (mi.scaled(mi.CONFIGS["qwen3_bf16"], T=37, H=256, F=128, E=1024,
                                    k=8), None),
}


@pytest.mark.parametrize("name", list(STATS))
def test_route_stats(moe, name):
    cfg = STATS[name][0]
    print(f"[route stats] {name}", flush=True)
    inp = mi.make_inputs(cfg)
    logits = oracle.router_logits(inp.x, inp.w_router)
    npy = lambda t: None if t is None else t.numpy()  # noqa: E731
    lb, sb = npy(inp.logit_bias), npy(inp.sel_bias)
    idx, gate = oracle.route_cfg(cfg, logits, lb, sb)
    ti, tg, pm = moe.route_stats(cfg, torch.from_numpy(logits).cuda(), to_dev(inp.logit_bias),
                                 to_dev(inp.sel_bias))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ti.cpu().numpy(), idx)
    assert rel_err(tg, gate) <= 1e-5
    ref = oracle.route_prob_mean(cfg, logits, lb)
    e = float(np.max(np.abs(pm.cpu().double().numpy() - ref) / np.max(ref)))
    print(f"   prob_mean {e:.2e}, sum {float(pm.sum()):.6f}", flush=True)
    assert e <= 1e-5

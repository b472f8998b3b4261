"""Grouped-GEMM backward (data and weight gradients, bf16) vs the CPU oracle on small copies
of the skewed DeepSeek-V3-shaped workload, through moe_grouped_gemm_swiglu_bwd. The oracle
and the GPU get the same inputs (the oracle's routing and Z, seeded dy); the oracle never sees
a GPU value."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from helpers import rel_err

pytestmark = pytest.mark.gpu
TOL = 2e-2

BWD = {
    "dsv3_bwd_small": mi.scaled(mi.CONFIGS["dsv3_fp8_skew"], T=520, H=512, F=256, shared_F=256),
    "dsv3_bwd_small2": mi.scaled(mi.CONFIGS["dsv3_fp8_skew"], T=300, H=768, F=384, shared_F=384),
    # one token: 248 of 256 experts get no rows (zero weight gradients), K = 1 row for the rest
    "dsv3_bwd_one_token": mi.scaled(mi.CONFIGS["dsv3_fp8_skew"], T=1, H=256, F=128, shared_F=128),
    # 64 experts (the smallest count the weight gradients' XCD plan takes), 128 x 128 tiles
    "dsv3_bwd_e64": mi.scaled(mi.CONFIGS["dsv3_fp8_skew"], T=300, H=256, F=128, shared_F=128,
                              E=64),
}


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_expert_softmax_amd as m
    return m


def bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16)


_CACHE = {}


def case(name):
    if name in _CACHE:
        return _CACHE[name]
    cfg = BWD[name]
    inp = mi.make_inputs(cfg)
    logits = oracle.router_logits(inp.x, inp.w_router)
    idx, gate = oracle.route_cfg(cfg, logits, inp.logit_bias.numpy(), inp.sel_bias.numpy())
    perm = oracle.permute(idx, gate, cfg.E)
    xp = torch.from_numpy(oracle.gather_rows(oracle.as_np(inp.x)[0], perm["pos"]).view(np.int16)).view(torch.bfloat16)
    dyp = torch.from_numpy(oracle.gather_rows(oracle.as_np(inp.dy)[0], perm["pos"]).view(np.int16)).view(torch.bfloat16)
    z, act, _ = oracle.expert_rows(xp, perm["offsets"], perm["gate_perm"], inp.w13, inp.w2,
                                   np.arange(cfg.A), want_z=True)
    c = dict(cfg=cfg, inp=inp, perm=perm, xp=xp, dyp=dyp, z=bf16(z), act=bf16(act))
    _CACHE[name] = c
    return c


@pytest.mark.parametrize("name", list(BWD))
def test_bwd_data_and_weight_gradients(moe, name):
    c = case(name)
    cfg, inp, perm = c["cfg"], c["inp"], c["perm"]
    print(f"[bwd] {name}", flush=True)
    T8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    out = moe.grouped_gemm_swiglu_bwd(cfg, c["dyp"].cuda(), c["xp"].cuda(), c["z"].cuda(),
                                      c["act"].cuda(), T8(perm["gate_perm"]),
                                      T8(perm["offsets"]), inp.w13.cuda(), inp.w2.cuda())
    torch.cuda.synchronize()
    rows = np.arange(cfg.A)
    dx_ref, dg_ref = oracle.expert_bwd_rows(c["dyp"], c["z"], perm["offsets"], perm["gate_perm"],
                                            inp.w13, inp.w2, rows)
    e_dx = rel_err(out["dx_perm"], dx_ref)
    e_dg = rel_err(out["dgate_perm"], dg_ref)
    counts = perm["counts"]
    order = np.argsort(counts)
    experts = sorted({int(order[-1]), int(order[0]), int(order[len(order) // 2]),
                      int(np.argmax(counts > 0))})
    rng = np.random.default_rng(11)
    dw13 = out["dw13"].cpu()
    dw2 = out["dw2"].cpu()
    worst = 0.0
    for e in experts:
        r13 = rng.integers(0, 2 * cfg.F, 64)
        c13 = rng.integers(0, cfg.H, 64)
        r2 = rng.integers(0, cfg.H, 64)
        c2 = rng.integers(0, cfg.F, 64)
        ref13, ref2 = oracle.expert_wgrad_entries(c["dyp"], c["z"], c["act"], c["xp"],
                                                  perm["offsets"], e, perm["gate_perm"],
                                                  inp.w2, (r13, c13), (r2, c2))
        got13 = dw13[e][r13, c13].double().numpy()
        got2 = dw2[e][r2, c2].double().numpy()
        if counts[e] == 0:
            assert not got13.any() and not got2.any()
            continue
        worst = max(worst, rel_err(got13, ref13), rel_err(got2, ref2))
    empty = np.nonzero(counts == 0)[0]
    if len(empty):
        assert not dw13[int(empty[0])].any() and not dw2[int(empty[0])].any()
    print(f"   dx {e_dx:.3e}  dg {e_dg:.3e}  dW (sampled, experts {experts}) {worst:.3e}",
          flush=True)
    assert e_dx <= TOL and e_dg <= TOL and worst <= TOL


@pytest.mark.parametrize("name", ["dsv3_bwd_small"])
def test_bwd_shared_expert_as_one_group(moe, name):
    """A shared expert's backward: one group of all T rows, gate 1 (gate_perm NULL)."""
    c = case(name)
    cfg, inp = c["cfg"], c["inp"]
    print(f"[bwd shared] {name}", flush=True)
    sc = cfg.replace(E=1, k=1, F=cfg.shared_F, router=mi.SOFTMAX_TOPK, n_groups=1,
                     topk_groups=1, route_scale=1.0)
    x = inp.x
    dy = inp.dy
    z, act, _ = oracle.expert_rows(x, None, None, inp.ws13, inp.ws2, np.arange(cfg.T), want_z=True)
    zb, ab = bf16(z), bf16(act)
    offs = torch.tensor([0, cfg.T], dtype=torch.int32)
    out = moe.grouped_gemm_swiglu_bwd(sc, dy.cuda(), x.cuda(), zb.cuda(), ab.cuda(), None,
                                      offs.cuda(), inp.ws13[None].contiguous().cuda(),
                                      inp.ws2[None].contiguous().cuda(), want_dgate=False)
    torch.cuda.synchronize()
    dx_ref, _ = oracle.expert_bwd_rows(dy, zb, offs.numpy(), None, inp.ws13, inp.ws2,
                                       np.arange(cfg.T))
    rng = np.random.default_rng(3)
    r13, c13 = rng.integers(0, 2 * sc.F, 64), rng.integers(0, cfg.H, 64)
    r2, c2 = rng.integers(0, cfg.H, 64), rng.integers(0, sc.F, 64)
    ref13, ref2 = oracle.expert_wgrad_entries(dy, zb, ab, x, offs.numpy(), 0, None, inp.ws2,
                                              (r13, c13), (r2, c2))
    e_dx = rel_err(out["dx_perm"], dx_ref)
    e13 = rel_err(out["dw13"][0].cpu()[r13, c13], ref13)
    e2 = rel_err(out["dw2"][0].cpu()[r2, c2], ref2)
    print(f"   dx {e_dx:.3e}  dW13 {e13:.3e}  dW2 {e2:.3e}", flush=True)
    assert e_dx <= TOL and e13 <= TOL and e2 <= TOL


@pytest.mark.parametrize("name", ["dsv3_bwd_small", "dsv3_bwd_small2"])
def test_bwd_kblocked_weights_bit_identical(moe, name):
    """The backward reads the weights in either layout: with w_layout = 1 and the weights
    K-blocked (the forward's layout, so one copy serves both passes) every output equals the
    row-major run bit for bit. small covers the 256 x 256 tiles, small2 the 128 x 128 ones."""
    c = case(name)
    cfg, inp, perm = c["cfg"], c["inp"], c["perm"]
    print(f"[bwd kblock] {name}", flush=True)
    T8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    w13, w2 = inp.w13.cuda(), inp.w2.cuda()
    common = (c["dyp"].cuda(), c["xp"].cuda(), c["z"].cuda(), c["act"].cuda(),
              T8(perm["gate_perm"]), T8(perm["offsets"]))
    ref = moe.grouped_gemm_swiglu_bwd(cfg, *common, w13, w2)
    got = moe.grouped_gemm_swiglu_bwd(cfg.replace(w_layout=1), *common, moe.pack_kblock(w13),
                                      moe.pack_kblock(w2))
    torch.cuda.synchronize()
    for n in ("dx_perm", "dw13", "dw2", "dgate_perm"):
        assert torch.equal(ref[n], got[n]), n


@pytest.mark.parametrize("name", ["dsv3_bwd_small", "dsv3_bwd_e64"])
def test_bwd_every_expert_weight_gradient(moe, name):
    """The weight gradients' tiles are dealt over the XCDs by a group plan computed on the
    device (largest groups first, each XCD an equal number of groups): every expert must get
    its own gradient. Eight sampled entries of dW13 and of dW2 of every expert against the
    oracle, on the skewed routing (256 experts on 256 x 256 tiles, 64 on 128 x 128 ones)."""
    c = case(name)
    cfg, inp, perm = c["cfg"], c["inp"], c["perm"]
    print(f"[bwd every expert] {name}", flush=True)
    T8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    out = moe.grouped_gemm_swiglu_bwd(cfg, c["dyp"].cuda(), c["xp"].cuda(), c["z"].cuda(),
                                      c["act"].cuda(), T8(perm["gate_perm"]),
                                      T8(perm["offsets"]), inp.w13.cuda(), inp.w2.cuda())
    torch.cuda.synchronize()
    dw13, dw2 = out["dw13"].cpu(), out["dw2"].cpu()
    rng = np.random.default_rng(5)
    worst = 0.0
    for e in range(cfg.E):
        r13, c13 = rng.integers(0, 2 * cfg.F, 8), rng.integers(0, cfg.H, 8)
        r2, c2 = rng.integers(0, cfg.H, 8), rng.integers(0, cfg.F, 8)
        ref13, ref2 = oracle.expert_wgrad_entries(c["dyp"], c["z"], c["act"], c["xp"],
                                                  perm["offsets"], e, perm["gate_perm"],
                                                  inp.w2, (r13, c13), (r2, c2))
        got13 = dw13[e][r13, c13].double().numpy()
        got2 = dw2[e][r2, c2].double().numpy()
        assert np.isfinite(got13).all() and np.isfinite(got2).all(), e
        if perm["counts"][e] == 0:              # no rows: the gradient is exactly zero
            assert not dw13[e].any() and not dw2[e].any(), e
            continue
        err = max(rel_err(got13, ref13), rel_err(got2, ref2))
        assert err <= TOL, (e, err)
        worst = max(worst, err)
    print(f"   worst per-expert rel err {worst:.3e}", flush=True)

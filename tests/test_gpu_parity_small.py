"""GPU path vs the CPU oracle, element by element, on small copies of every workload
(several tiles per GEMM, ragged per-expert tails). All calls go through the C ABI."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from helpers import SMALL, rel_err, routing_margin, tol, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_expert_softmax_amd as m
    return m


_CACHE = {}


def case(name):
    """Inputs and the oracle's routing / permutation of one small workload."""
    if name in _CACHE:
        return _CACHE[name]
    cfg = SMALL[name]
    inp = mi.make_inputs(cfg)
    logits = oracle.router_logits(inp.x, inp.w_router)
    lb = None if inp.logit_bias is None else inp.logit_bias.numpy()
    sb = None if inp.sel_bias is None else inp.sel_bias.numpy()
    idx, gate = oracle.route_cfg(cfg, logits, lb, sb)
    perm = oracle.permute(idx, gate, cfg.E)
    c = dict(cfg=cfg, inp=inp, logits=logits, idx=idx, gate=gate, perm=perm)
    _CACHE[name] = c
    return c


NAMES = list(SMALL)


@pytest.mark.parametrize("name", NAMES)
def test_router_logits(moe, name):
    c = case(name)
    cfg, inp = c["cfg"], c["inp"]
    print(f"[router_logits] {name}", flush=True)
    got = moe.router_logits(cfg, inp.x.cuda(), inp.w_router.cuda())
    torch.cuda.synchronize()
    assert rel_err(got, c["logits"]) <= 1e-5


@pytest.mark.parametrize("name", NAMES)
def test_route_bit_exact_on_oracle_logits(moe, name):
    c = case(name)
    cfg, inp = c["cfg"], c["inp"]
    print(f"[route] {name}", flush=True)
    idx, gate = moe.route(cfg, torch.from_numpy(c["logits"]).cuda(), to_dev(inp.logit_bias),
                          to_dev(inp.sel_bias))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), c["idx"])
    np.testing.assert_allclose(gate.cpu().numpy(), c["gate"], rtol=1e-6, atol=0)


@pytest.mark.parametrize("name", NAMES)
def test_permute_bit_exact(moe, name):
    c = case(name)
    cfg, inp, perm = c["cfg"], c["inp"], c["perm"]
    print(f"[permute] {name}", flush=True)
    out = moe.permute(cfg, inp.x.cuda(), torch.from_numpy(c["idx"]).cuda(),
                      torch.from_numpy(c["gate"]).cuda())
    torch.cuda.synchronize()
    for key in ("counts", "offsets", "pos", "src"):
        np.testing.assert_array_equal(out[key].cpu().numpy(), perm[key], err_msg=key)
    np.testing.assert_array_equal(out["gate_perm"].cpu().numpy(), perm["gate_perm"])
    x_ref = oracle.gather_rows(oracle.as_np(inp.x)[0], perm["pos"])
    np.testing.assert_array_equal(oracle.as_np(out["x_perm"].cpu())[0], x_ref)


def oracle_x_perm(c):
    x_np = oracle.as_np(c["inp"].x)[0]
    xp = oracle.gather_rows(x_np, c["perm"]["pos"])
    return torch.from_numpy(xp.view(np.int16)).view(torch.bfloat16) if xp.dtype == np.uint16 \
        else torch.from_numpy(xp)


@pytest.mark.parametrize("name", NAMES)
def test_grouped_gemm(moe, name):
    c = case(name)
    cfg, inp, perm = c["cfg"], c["inp"], c["perm"]
    print(f"[grouped_gemm] {name}", flush=True)
    xp = oracle_x_perm(c)
    sh = dict(x_shared=inp.x.cuda(), ws13=inp.ws13.cuda(), ws2=inp.ws2.cuda()) if cfg.shared_F else {}
    out = moe.grouped_gemm_swiglu(cfg, xp.cuda(), torch.from_numpy(perm["offsets"]).cuda(),
                                  torch.from_numpy(perm["gate_perm"]).cuda(), inp.w13.cuda(),
                                  inp.w2.cuda(), save_z=True, **sh)
    torch.cuda.synchronize()
    rows = np.arange(cfg.A)
    z_ref, act_ref, y_ref = oracle.expert_rows(xp, perm["offsets"], perm["gate_perm"], inp.w13,
                                               inp.w2, rows, want_z=True)
    t = tol(cfg)
    assert rel_err(out["act"], act_ref) <= t
    assert rel_err(out["y_perm"], y_ref) <= t
    assert rel_err(out["z"], z_ref) <= t
    if cfg.shared_F:
        _, _, ys = oracle.expert_rows(inp.x, None, None, inp.ws13, inp.ws2, np.arange(cfg.T))
        assert rel_err(out["shared_y"], ys) <= t


@pytest.mark.parametrize("name", NAMES)
def test_combine(moe, name):
    c = case(name)
    cfg, perm = c["cfg"], c["perm"]
    print(f"[combine] {name}", flush=True)
    g = torch.Generator().manual_seed(5)
    dt = moe.act_torch_dtype(cfg)
    yp = torch.randn(cfg.A, cfg.H, generator=g).to(dt)
    sh = torch.randn(cfg.T, cfg.H, generator=g).to(dt) if cfg.shared_F else None
    y = moe.unpermute_combine(cfg, yp.cuda(), torch.from_numpy(perm["pos"]).cuda(), to_dev(sh))
    torch.cuda.synchronize()
    ref = oracle.combine(yp, perm["pos"], sh)
    # one rounding of an fp32 sum to the output dtype
    bound = 1e-6 if cfg.act_dtype == mi.F32 else 2.0 ** -8
    assert rel_err(y, ref) <= bound


@pytest.mark.parametrize("name", NAMES)
def test_layer_forward_on_oracle_logits(moe, name):
    c = case(name)
    cfg, inp = c["cfg"], c["inp"]
    print(f"[layer_forward logits_in] {name}", flush=True)
    y, ex = moe.layer_forward(cfg, inp.x.cuda(), inp.w_router.cuda(), inp.w13.cuda(),
                              inp.w2.cuda(), to_dev(inp.logit_bias), to_dev(inp.sel_bias),
                              torch.from_numpy(c["logits"]).cuda(), ws13=to_dev(inp.ws13),
                              ws2=to_dev(inp.ws2), want=("topk_idx", "counts"))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ex["topk_idx"].cpu().numpy(), c["idx"])
    np.testing.assert_array_equal(ex["counts"].cpu().numpy(), c["perm"]["counts"])
    ref = oracle.layer_tokens(inp.x, c["idx"], c["gate"], inp.w13, inp.w2, np.arange(cfg.T),
                              inp.ws13, inp.ws2)
    assert rel_err(y, ref) <= tol(cfg)


@pytest.mark.parametrize("name", NAMES)
def test_layer_forward_full_gpu_path(moe, name):
    """Router GEMM on the GPU too. Tokens whose expert set differs from the oracle's must
    sit on a near-tie of the routing key; the rest must match the oracle."""
    c = case(name)
    cfg, inp = c["cfg"], c["inp"]
    print(f"[layer_forward full] {name}", flush=True)
    y, ex = moe.layer_forward(cfg, inp.x.cuda(), inp.w_router.cuda(), inp.w13.cuda(),
                              inp.w2.cuda(), to_dev(inp.logit_bias), to_dev(inp.sel_bias),
                              ws13=to_dev(inp.ws13), ws2=to_dev(inp.ws2),
                              want=("topk_idx", "logits"))
    torch.cuda.synchronize()
    gi = ex["topk_idx"].cpu().numpy()
    same = np.all(np.sort(gi, 1) == np.sort(c["idx"], 1), axis=1)
    assert same.mean() > 0.99
    # every token whose expert set changed sits on a near-tie of the oracle's keys (the
    # router logits differ from the oracle's only by fp32 summation order)
    lb = None if inp.logit_bias is None else inp.logit_bias.numpy()
    sb = None if inp.sel_bias is None else inp.sel_bias.numpy()
    margin = routing_margin(cfg, c["logits"], lb, sb)
    flipped = np.nonzero(~same)[0]
    print(f"   flipped tokens {len(flipped)}, their largest margin "
          f"{margin[flipped].max() if len(flipped) else 0.0:.2e}", flush=True)
    assert np.all(margin[flipped] <= 1e-4), margin[flipped]
    toks = np.nonzero(same)[0]
    ref = oracle.layer_tokens(inp.x, c["idx"], c["gate"], inp.w13, inp.w2, toks, inp.ws13,
                              inp.ws2)
    assert rel_err(y.cpu()[toks], ref) <= tol(cfg)


@pytest.mark.parametrize("name", ["dsv3_small", "tiny_fp32"])
def test_deterministic(moe, name):
    c = case(name)
    cfg, inp = c["cfg"], c["inp"]
    args = (cfg, inp.x.cuda(), inp.w_router.cuda(), inp.w13.cuda(), inp.w2.cuda(),
            to_dev(inp.logit_bias), to_dev(inp.sel_bias))
    kw = dict(ws13=to_dev(inp.ws13), ws2=to_dev(inp.ws2))
    y1, _ = moe.layer_forward(*args, **kw)
    y2, _ = moe.layer_forward(*args, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("name", ["dsv3_small", "mixtral_small"])
def test_stage_events_leave_results_unchanged(moe, name):
    """With stage events set, the layer gives the same bits, every event completes, and the
    stage durations add up to the span of the call."""
    c = case(name)
    cfg, inp = c["cfg"], c["inp"]
    args = (cfg, inp.x.cuda(), inp.w_router.cuda(), inp.w13.cuda(), inp.w2.cuda(),
            to_dev(inp.logit_bias), to_dev(inp.sel_bias))
    kw = dict(ws13=to_dev(inp.ws13), ws2=to_dev(inp.ws2))
    y1, _ = moe.layer_forward(*args, **kw)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(moe.N_STAGE_EVENTS)]
    moe.set_stage_events(evs)
    try:
        y2, _ = moe.layer_forward(*args, **kw)
    finally:
        moe.set_stage_events(None)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert all(e.query() for e in evs)
    parts = [evs[i].elapsed_time(evs[i + 1]) for i in range(moe.N_STAGE_EVENTS - 1)]
    assert min(parts) >= 0.0
    assert abs(sum(parts) - evs[0].elapsed_time(evs[-1])) <= 1e-2


# ---------------------------------------------------------------------------------------
# K-blocked layouts (expert-grouped activations and packed expert weights)
# ---------------------------------------------------------------------------------------
from helpers import block, unblock  # noqa: E402

BF_NAMES = [n for n in NAMES if SMALL[n].act_dtype != mi.F32]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.uint8, torch.float32])
def test_pack_kblock_matches_reshape(moe, dtype):
    print(f"[pack_kblock] {dtype}", flush=True)
    g = torch.Generator().manual_seed(3)
    t = (torch.randn(3, 40, 256, generator=g) * 7).to(dtype)
    got = moe.pack_kblock(t.cuda())
    torch.cuda.synchronize()
    assert torch.equal(got.cpu(), block(t))
    assert torch.equal(unblock(got.cpu(), 40, 256), t)


@pytest.mark.parametrize("name", BF_NAMES)
def test_permute_kblock(moe, name):
    c = case(name)
    cfg, inp, perm = c["cfg"].replace(a_layout=1), c["inp"], c["perm"]
    print(f"[permute kblock] {name}", flush=True)
    out = moe.permute(cfg, inp.x.cuda(), torch.from_numpy(c["idx"]).cuda(),
                      torch.from_numpy(c["gate"]).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out["pos"].cpu().numpy(), perm["pos"])
    got = unblock(out["x_perm"].cpu(), cfg.A, cfg.H)
    x_ref = oracle.gather_rows(oracle.as_np(inp.x)[0], perm["pos"])
    np.testing.assert_array_equal(oracle.as_np(got)[0], x_ref)


@pytest.mark.parametrize("name", BF_NAMES)
def test_grouped_gemm_kblock(moe, name):
    """K-blocked x_perm / act and packed weights give the oracle's results, and exactly the
    row-major path's results (same MFMA order)."""
    c = case(name)
    base = c["cfg"]
    cfg = base.replace(a_layout=1, w_layout=1)
    inp, perm = c["inp"], c["perm"]
    print(f"[grouped_gemm kblock] {name}", flush=True)
    xp = oracle_x_perm(c)
    offs = torch.from_numpy(perm["offsets"]).cuda()
    gp = torch.from_numpy(perm["gate_perm"]).cuda()
    w13, w2 = inp.w13.cuda(), inp.w2.cuda()
    sh = dict(x_shared=inp.x.cuda(), ws13=inp.ws13.cuda(), ws2=inp.ws2.cuda()) if cfg.shared_F else {}
    ref_rows = moe.grouped_gemm_swiglu(base, xp.cuda(), offs, gp, w13, w2, **sh)
    shb = dict(x_shared=inp.x.cuda(), ws13=moe.pack_kblock(inp.ws13.cuda()),
               ws2=moe.pack_kblock(inp.ws2.cuda())) if cfg.shared_F else {}
    out = moe.grouped_gemm_swiglu(cfg, moe.pack_kblock(xp.cuda()), offs, gp,
                                  moe.pack_kblock(w13), moe.pack_kblock(w2), **shb)
    torch.cuda.synchronize()
    act = unblock(out["act"].cpu(), cfg.A, cfg.F)
    assert torch.equal(act, ref_rows["act"].cpu())
    assert torch.equal(out["y_perm"].cpu(), ref_rows["y_perm"].cpu())
    if cfg.shared_F:
        assert torch.equal(out["shared_y"].cpu(), ref_rows["shared_y"].cpu())
    rows = np.arange(cfg.A)
    _, act_ref, y_ref = oracle.expert_rows(xp, perm["offsets"], perm["gate_perm"], inp.w13,
                                           inp.w2, rows)
    assert rel_err(act, act_ref) <= tol(cfg)
    assert rel_err(out["y_perm"], y_ref) <= tol(cfg)


@pytest.mark.parametrize("name", BF_NAMES)
def test_layer_forward_packed_weights(moe, name):
    c = case(name)
    cfg, inp = c["cfg"].replace(w_layout=1), c["inp"]
    print(f"[layer_forward packed] {name}", flush=True)
    pk = lambda t: None if t is None else moe.pack_kblock(t.cuda())  # noqa: E731
    y, ex = moe.layer_forward(cfg, inp.x.cuda(), inp.w_router.cuda(), pk(inp.w13), pk(inp.w2),
                              to_dev(inp.logit_bias), to_dev(inp.sel_bias),
                              torch.from_numpy(c["logits"]).cuda(), ws13=pk(inp.ws13),
                              ws2=pk(inp.ws2), want=("topk_idx",))
    y0, _ = moe.layer_forward(c["cfg"], inp.x.cuda(), inp.w_router.cuda(), inp.w13.cuda(),
                              inp.w2.cuda(), to_dev(inp.logit_bias), to_dev(inp.sel_bias),
                              torch.from_numpy(c["logits"]).cuda(), ws13=to_dev(inp.ws13),
                              ws2=to_dev(inp.ws2))
    torch.cuda.synchronize()
    assert torch.equal(y, y0)
    np.testing.assert_array_equal(ex["topk_idx"].cpu().numpy(), c["idx"])
    ref = oracle.layer_tokens(inp.x, c["idx"], c["gate"], inp.w13, inp.w2, np.arange(cfg.T),
                              inp.ws13, inp.ws2)
    assert rel_err(y, ref) <= tol(cfg)

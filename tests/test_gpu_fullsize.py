"""Full-size parity: every bf16/e4m3/MXFP8 workload at its full size, in the launch configuration
bench.py times (expert weights packed K-blocked; inside the layer GEMM1 gathers its rows),
checked against the CPU oracle on outputs it can compute one by one (sampled tokens and
rows) and on properties that hold at any size. All GPU work goes through the C ABI; the
oracle only ever sees seeded inputs and its own results."""
import gc

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from helpers import TOL, e4m3_codes_close, rel_err, routing_margin, tol, to_dev

pytestmark = pytest.mark.gpu

FULL = ["mixtral_bf16", "qwen3_bf16", "dsv3_bf16", "dsv3_fp8_skew"]
# the whole-layer tests also run the MXFP8 widening of the DeepSeek-V3 layer
FULL_LAYER = FULL + ["dsv3_mxfp8"]
_STATE = {}


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_expert_softmax_amd as m
    return m


def log(msg):
    print(f"[fullsize] {msg}", flush=True)


def full_case(moe, name):
    """Inputs, oracle routing and device weights of one workload (one held at a time)."""
    if name in _STATE:
        return _STATE[name]
    _STATE.clear()
    gc.collect()
    torch.cuda.empty_cache()
    mx = mi.CONFIGS[name].w_dtype == mi.MXFP8
    cfg = mi.CONFIGS[name].replace(a_layout=0 if mx else 1, w_layout=1)
    log(f"{name}: generating inputs")
    inp = mi.make_inputs(cfg)
    log(f"{name}: oracle router logits and routing")
    logits = oracle.router_logits(inp.x, inp.w_router)
    lb = None if inp.logit_bias is None else inp.logit_bias.numpy()
    sb = None if inp.sel_bias is None else inp.sel_bias.numpy()
    idx, gate = oracle.route_cfg(cfg, logits, lb, sb)
    perm = oracle.permute(idx, gate, cfg.E)
    log(f"{name}: device weights")
    dev = {}
    sc = dict(w13_scales=None, w2_scales=None, ws13_scales=None, ws2_scales=None)
    keys = ["w13", "w2"] + (["ws13", "ws2"] if cfg.shared_F else [])
    for kname in keys:
        t = getattr(inp, kname).cuda()
        if cfg.w_dtype == mi.E4M3:
            t, sc[kname + "_scales"] = moe.quantize_e4m3(t, 128)
        elif cfg.w_dtype == mi.MXFP8:      # K-blocked codes, blocked scales
            t, s8 = moe.quantize_mx(t)
            sc[kname + "_scales"] = moe.pack_mx_scales(s8)
            del s8
        dev[kname] = moe.pack_kblock(t)
        del t
    torch.cuda.synchronize()
    c = dict(cfg=cfg, inp=inp, logits=logits, idx=idx, gate=gate, perm=perm, dev=dev, sc=sc,
             lb=lb, sb=sb)
    _STATE[name] = c
    return c


def sample_tokens(c, n=24, seed=0):
    """Tokens routed to the hottest and to the coldest non-empty expert, plus random ones."""
    counts, idx = c["perm"]["counts"], c["idx"]
    hot = int(np.argmax(counts))
    nz = np.nonzero(counts)[0]
    cold = int(nz[np.argmin(counts[nz])])
    pick = [int(np.nonzero((idx == hot).any(1))[0][0]), int(np.nonzero((idx == cold).any(1))[0][0])]
    rng = np.random.default_rng(seed)
    pick += list(rng.choice(c["cfg"].T, n - 2, replace=False))
    return np.unique(np.array(pick, np.int64))


def oracle_tokens(c, toks):
    """The oracle's y for selected tokens; e4m3 workloads quantise (with the oracle's own
    quantiser) only the experts those tokens use."""
    cfg, inp = c["cfg"], c["inp"]
    idx = c["idx"]
    if cfg.w_dtype not in (mi.E4M3, mi.MXFP8):
        return oracle.layer_tokens(inp.x, idx, c["gate"], inp.w13, inp.w2, toks, inp.ws13,
                                   inp.ws2)
    mx = cfg.w_dtype == mi.MXFP8
    used = np.unique(idx[toks])
    remap = np.full(cfg.E, -1, np.int32)
    remap[used] = np.arange(len(used), dtype=np.int32)
    sub_idx = np.zeros_like(idx)
    sub_idx[toks] = remap[idx[toks]]
    qw = oracle.mx_quant if mx else oracle.quant_weight
    q13 = qw(inp.w13[torch.from_numpy(used)])
    q2 = qw(inp.w2[torch.from_numpy(used)])
    s13, s2 = qw(inp.ws13), qw(inp.ws2)
    return oracle.layer_tokens(inp.x, sub_idx, c["gate"], q13[0], q2[0], toks, s13[0], s2[0],
                               fp8="mx" if mx else True, w13_scales=q13[1], w2_scales=q2[1],
                               ws13_scales=s13[1], ws2_scales=s2[1])


def kblock_rows(t, rows, n_rows, cols_bytes):
    """Rows of a K-blocked [n_rows, cols] device tensor -> uint8 [len(rows), cols_bytes]."""
    b = t.view(torch.uint8).reshape(cols_bytes // 64, n_rows, 64)
    r = torch.as_tensor(rows, device=t.device)
    return b[:, r, :].permute(1, 0, 2).reshape(len(rows), cols_bytes).cpu()


@pytest.mark.parametrize("name", FULL_LAYER)
def test_full_layer_on_oracle_logits(moe, name):
    c = full_case(moe, name)
    cfg, inp, dev = c["cfg"], c["inp"], c["dev"]
    log(f"{name}: layer forward on the oracle's logits")
    y, ex = moe.layer_forward(cfg, inp.x.cuda(), inp.w_router.cuda(), dev["w13"], dev["w2"],
                              to_dev(inp.logit_bias), to_dev(inp.sel_bias),
                              torch.from_numpy(c["logits"]).cuda(), ws13=dev.get("ws13"),
                              ws2=dev.get("ws2"), want=("topk_idx", "topk_gate", "counts"),
                              **c["sc"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ex["topk_idx"].cpu().numpy(), c["idx"])
    np.testing.assert_array_equal(ex["counts"].cpu().numpy(), c["perm"]["counts"])
    np.testing.assert_allclose(ex["topk_gate"].cpu().numpy(), c["gate"], rtol=1e-6, atol=0)
    assert int(c["perm"]["counts"].sum()) == cfg.T * cfg.k
    toks = sample_tokens(c)
    ref = oracle_tokens(c, toks)
    e = rel_err(y[torch.from_numpy(toks).cuda()], ref)
    log(f"{name}: y on {len(toks)} sampled tokens: rel err {e:.3e}")
    assert e <= tol(cfg)


@pytest.mark.parametrize("name", FULL_LAYER)
def test_full_router_gemm_and_routing_on_gpu(moe, name):
    """Router GEMM on the GPU too: logits within 1e-5 of the oracle's; tokens whose expert set
    changes (fp32 rounding on a near-tie) are counted, must be rare, and are excluded."""
    c = full_case(moe, name)
    cfg, inp, dev = c["cfg"], c["inp"], c["dev"]
    y, ex = moe.layer_forward(cfg, inp.x.cuda(), inp.w_router.cuda(), dev["w13"], dev["w2"],
                              to_dev(inp.logit_bias), to_dev(inp.sel_bias), None,
                              ws13=dev.get("ws13"), ws2=dev.get("ws2"),
                              want=("logits", "topk_idx"), **c["sc"])
    torch.cuda.synchronize()
    e_l = rel_err(ex["logits"], c["logits"])
    gi = ex["topk_idx"].cpu().numpy()
    same = np.all(np.sort(gi, 1) == np.sort(c["idx"], 1), axis=1)
    log(f"{name}: router logits rel err {e_l:.3e}; tokens with another expert set: "
        f"{int((~same).sum())} of {cfg.T}")
    assert e_l <= 1e-5
    assert same.mean() >= 0.995
    # every token whose expert set changed sits on a near-tie of the oracle's keys
    margin = routing_margin(cfg, c["logits"], c["lb"], c["sb"])
    flipped = np.nonzero(~same)[0]
    log(f"{name}: flipped tokens' largest tie margin "
        f"{margin[flipped].max() if len(flipped) else 0.0:.2e} (bound 1e-4)")
    assert np.all(margin[flipped] <= 1e-4), margin[flipped]
    toks = [t for t in sample_tokens(c, 16, seed=1) if same[t]]
    ref = oracle_tokens(c, np.array(toks, np.int64))
    assert rel_err(y[torch.tensor(toks).cuda()], ref) <= tol(cfg)


@pytest.mark.parametrize("name", FULL)
def test_full_permute(moe, name):
    c = full_case(moe, name)
    cfg, inp, perm = c["cfg"], c["inp"], c["perm"]
    log(f"{name}: permute")
    out = moe.permute(cfg, inp.x.cuda(), torch.from_numpy(c["idx"]).cuda(),
                      torch.from_numpy(c["gate"]).cuda(), want_x_q=cfg.w_dtype == mi.E4M3)
    torch.cuda.synchronize()
    for key in ("counts", "offsets", "pos", "src", "gate_perm"):
        np.testing.assert_array_equal(out[key].cpu().numpy(), perm[key], err_msg=key)
    # bijection onto the T*k rows, src inverts pos
    pos = perm["pos"].ravel()
    assert np.array_equal(np.sort(pos), np.arange(cfg.A))
    assert np.array_equal(perm["src"][pos], np.repeat(np.arange(cfg.T), cfg.k))
    rows = np.unique(np.concatenate([perm["offsets"][:-1][perm["counts"] > 0],
                                     perm["offsets"][1:][perm["counts"] > 0] - 1]))[:600]
    eb = 1 if cfg.w_dtype == mi.E4M3 else 2
    got = kblock_rows(out["x_perm"], rows, cfg.A, cfg.H * eb).numpy()
    src_rows = perm["src"][rows]
    if cfg.w_dtype == mi.E4M3:
        xq, xs = oracle.quant_rows(inp.x[torch.from_numpy(src_rows)])
        np.testing.assert_array_equal(got, xq)
        np.testing.assert_array_equal(out["x_perm_scales"].cpu().numpy()[rows], xs)
    else:
        ref = oracle.as_np(inp.x[torch.from_numpy(src_rows)])[0].view(np.uint8)
        np.testing.assert_array_equal(got, ref.reshape(len(rows), -1))


@pytest.mark.parametrize("name", FULL)
def test_full_grouped_gemm_sampled_rows(moe, name):
    """The grouped GEMM halves at full size, on the first and last row of every expert."""
    c = full_case(moe, name)
    cfg, inp, perm, dev, sc = c["cfg"], c["inp"], c["perm"], c["dev"], c["sc"]
    fp8 = cfg.w_dtype == mi.E4M3
    log(f"{name}: grouped GEMM (sampled rows)")
    p = moe.permute(cfg, inp.x.cuda(), torch.from_numpy(c["idx"]).cuda(),
                    torch.from_numpy(c["gate"]).cuda(), want_x_q=fp8)
    A, F, H, T = cfg.A, cfg.F, cfg.H, cfg.T
    gd, ad = moe.gemm_torch_dtype(cfg), moe.act_torch_dtype(cfg)
    act = torch.empty(A, F, dtype=gd, device="cuda")
    act_sc = torch.empty(A, F // 128, dtype=torch.float32, device="cuda") if fp8 else None
    y_perm = torch.empty(A, H, dtype=ad, device="cuda")
    sh = cfg.shared_F
    sh_act = torch.empty(T, sh, dtype=gd, device="cuda") if sh else None
    sh_sc = torch.empty(T, sh // 128, dtype=torch.float32, device="cuda") if (sh and fp8) else None
    sh_y = torch.empty(T, H, dtype=ad, device="cuda") if sh else None
    xs = (p["x_q"] if fp8 else inp.x.cuda()) if sh else None
    xss = p["x_q_scales"] if (sh and fp8) else None
    moe.grouped_gemm_up(cfg, p["x_perm"], p["offsets"], p["gate_perm"], dev["w13"], act,
                        x_perm_scales=p["x_perm_scales"], w13_scales=sc["w13_scales"],
                        x_shared=xs, x_shared_scales=xss, ws13=dev.get("ws13"),
                        ws13_scales=sc["ws13_scales"], act_scales=act_sc, shared_act=sh_act,
                        shared_act_scales=sh_sc)
    moe.grouped_gemm_down(cfg, act, p["offsets"], dev["w2"], y_perm, act_scales=act_sc,
                          w2_scales=sc["w2_scales"], shared_act=sh_act,
                          shared_act_scales=sh_sc, ws2=dev.get("ws2"),
                          ws2_scales=sc["ws2_scales"], shared_y=sh_y)
    torch.cuda.synchronize()
    nz = np.nonzero(perm["counts"] > 0)[0]
    offs = perm["offsets"]
    if fp8:
        # 16 experts (hottest, coldest, random); the oracle quantises just those
        rng = np.random.default_rng(2)
        hot, cold = int(np.argmax(perm["counts"])), int(nz[np.argmin(perm["counts"][nz])])
        ex = np.unique(np.concatenate([[hot, cold], rng.choice(nz, 14, replace=False)]))
        rows = np.unique(np.concatenate([offs[ex], offs[ex + 1] - 1]))
        experts = np.searchsorted(offs, rows, side="right") - 1
        remap = np.zeros(cfg.E, np.int32)
        remap[ex] = np.arange(len(ex))
        sub_off = np.zeros(len(ex) + 1, np.int32)
        sub_off[1:] = np.cumsum(np.bincount(remap[experts], minlength=len(ex)))
        q13 = oracle.quant_weight(inp.w13[torch.from_numpy(ex)])
        q2 = oracle.quant_weight(inp.w2[torch.from_numpy(ex)])
        xq, xsr = oracle.quant_rows(inp.x[torch.from_numpy(perm["src"][rows])])
        _, act_ref, y_ref = oracle.expert_rows(
            xq, sub_off, perm["gate_perm"][rows], q13[0], q2[0], np.arange(len(rows)),
            x_scales=xsr, w13_scales=q13[1], w2_scales=q2[1], quant_act=True)
        _, act_pre, _ = oracle.expert_rows(
            xq, sub_off, perm["gate_perm"][rows], q13[0], q2[0], np.arange(len(rows)),
            x_scales=xsr, w13_scales=q13[1], w2_scales=q2[1], quant_act=False)
        ga = kblock_rows(act, rows, A, F).numpy()
        gs = act_sc.cpu().numpy()[rows]
        ratio, dfrac, srel = e4m3_codes_close(ga, gs, act_pre)
        log(f"{name}: act codes: max err / (1 step + 1e-3 range) {ratio:.2f}, differing {dfrac:.2e}, scale rel {srel:.1e}")
        assert ratio <= 1.0 and dfrac <= 0.02 and srel <= 1e-4
        v = oracle.e4m3_decode_array(ga) * np.repeat(gs.astype(np.float64), 128, axis=1)
        e_act = rel_err(v, act_ref)
    else:
        # first and last row of every expert, on the oracle's own x_perm and full weights
        rows = np.unique(np.concatenate([offs[:-1][nz], offs[1:][nz] - 1]))
        x_perm_o = oracle.gather_rows(oracle.as_np(inp.x)[0], perm["pos"])
        _, act_ref, y_ref = oracle.expert_rows(x_perm_o, offs, perm["gate_perm"], inp.w13,
                                               inp.w2, rows)
        del x_perm_o
        ga = kblock_rows(act, rows, A, F * 2).view(torch.bfloat16)
        e_act = rel_err(ga, act_ref)
    e_y = rel_err(y_perm[torch.from_numpy(rows).cuda()], y_ref)
    log(f"{name}: {len(rows)} rows (first/last of the sampled experts): act {e_act:.3e}, "
        f"y_perm {e_y:.3e}")
    # quantised act: checked code by code above (fp8); bf16 act and y_perm to the tolerance
    assert e_y <= tol(cfg) and (fp8 or e_act <= tol(cfg))


def test_full_backward_dsv3_fp8_skew(moe):
    """Grouped-GEMM backward at full size on the skewed layer (hottest expert 2578 rows):
    seeded synthetic saved Z / act / dy (any values are valid saved tensors); dx and dg on
    the first and last row of every expert, dW entries of the three smallest experts and
    one mid-sized expert."""
    c = full_case(moe, "dsv3_fp8_skew")
    cfg, inp, perm = c["cfg"], c["inp"], c["perm"]
    bcfg = cfg.replace(w_dtype=mi.BF16, a_layout=0, w_layout=0, shared_F=0)
    A, F, H = cfg.A, cfg.F, cfg.H
    g = torch.Generator().manual_seed(20261202)
    z = torch.randn(A, 2 * F, generator=g).to(torch.bfloat16)
    act = (torch.randn(A, F, generator=g) * 0.1).to(torch.bfloat16)
    dy = torch.randn(A, H, generator=g).to(torch.bfloat16)
    xp = inp.x[torch.from_numpy(perm["src"].astype(np.int64))].contiguous()
    T8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    log("dsv3_fp8_skew: backward")
    out = moe.grouped_gemm_swiglu_bwd(bcfg, dy.cuda(), xp.cuda(), z.cuda(), act.cuda(),
                                      T8(perm["gate_perm"]), T8(perm["offsets"]),
                                      inp.w13.cuda(), inp.w2.cuda())
    torch.cuda.synchronize()
    nz = perm["counts"] > 0
    rows = np.unique(np.concatenate([perm["offsets"][:-1][nz], perm["offsets"][1:][nz] - 1]))
    dx_ref, dg_ref = oracle.expert_bwd_rows(dy, z, perm["offsets"], perm["gate_perm"], inp.w13,
                                            inp.w2, rows)
    e_dx = rel_err(out["dx_perm"][torch.from_numpy(rows).cuda()], dx_ref)
    e_dg = rel_err(out["dgate_perm"][torch.from_numpy(rows).cuda()], dg_ref)
    order = np.argsort(perm["counts"])
    small = [int(e) for e in order if perm["counts"][e] > 0][:3]
    experts = small + [int(order[len(order) // 2])]
    rng = np.random.default_rng(5)
    worst = 0.0
    for e in experts:
        r13, c13 = rng.integers(0, 2 * F, 48), rng.integers(0, H, 48)
        r2, c2 = rng.integers(0, H, 48), rng.integers(0, F, 48)
        ref13, ref2 = oracle.expert_wgrad_entries(dy, z, act, xp, perm["offsets"], e,
                                                  perm["gate_perm"], inp.w2, (r13, c13), (r2, c2))
        got13 = out["dw13"][e][torch.from_numpy(r13).cuda(), torch.from_numpy(c13).cuda()]
        got2 = out["dw2"][e][torch.from_numpy(r2).cuda(), torch.from_numpy(c2).cuda()]
        worst = max(worst, rel_err(got13, ref13), rel_err(got2, ref2))
    log(f"dsv3_fp8_skew backward: dx {e_dx:.3e}, dg {e_dg:.3e}, dW (experts {experts}) "
        f"{worst:.3e}")
    assert e_dx <= TOL[mi.BF16] and e_dg <= TOL[mi.BF16] and worst <= TOL[mi.BF16]


def test_full_layer_backward_dsv3(moe):
    """Whole-layer backward at the DeepSeek-V3 bf16 size on the oracle's routing:
    - the full batch: dx and dlogits of sampled tokens (the oracle on that sub-batch), the
      full dW13 / dW2 of the hottest and the coldest expert (the oracle's per-expert
      gradient), and the shared expert's full dWs13 / dWs2 (the oracle's expert gradient
      over all T tokens);
    - a sub-batch of the same tokens run through the GPU backward on its own: every output,
      dW_r included, against oracle.layer_backward of that sub-batch."""
    c = full_case(moe, "dsv3_bf16")
    cfg, inp = c["cfg"].replace(a_layout=0, w_layout=0), c["inp"]
    T, H, F, sF = cfg.T, cfg.H, cfg.F, cfg.shared_F
    log("dsv3_bf16: layer backward")
    rng = np.random.default_rng(5)
    dy = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16)
    dev = {n: getattr(inp, n).cuda() for n in ("w13", "w2", "ws13", "ws2")}
    T8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    g = moe.layer_backward(cfg, inp.x.cuda(), inp.w_router.cuda(), T8(c["logits"]),
                           T8(c["idx"]), T8(c["gate"]), dev["w13"], dev["w2"], dy.cuda(),
                           ws13=dev["ws13"], ws2=dev["ws2"], want_dlogits=True)
    torch.cuda.synchronize()
    # the sub-batch: the same tokens through the GPU backward alone (T = 16)
    toks = sample_tokens(c, n=16, seed=3)
    scfg = cfg.replace(T=len(toks))
    gs = moe.layer_backward(scfg, inp.x[toks].cuda(), inp.w_router.cuda(),
                            T8(c["logits"][toks]), T8(c["idx"][toks]), T8(c["gate"][toks]),
                            dev["w13"], dev["w2"], dy[toks].cuda(), ws13=dev["ws13"],
                            ws2=dev["ws2"], want_dlogits=True)
    torch.cuda.synchronize()
    del dev
    sub = oracle.layer_backward(inp.x[toks], inp.w_router, c["logits"][toks], c["idx"][toks],
                                inp.w13, inp.w2, dy[toks], cfg.router, cfg.route_scale,
                                None, inp.ws13, inp.ws2)
    e_dx = rel_err(g["dx"][torch.from_numpy(toks).cuda()].float().cpu(), sub["dx"])
    e_dl = rel_err(g["dlogits"][torch.from_numpy(toks).cuda()].cpu(), sub["dlogits"])
    log(f"dsv3_bf16 backward: dx {e_dx:.3e}, dlogits {e_dl:.3e} on {len(toks)} tokens")
    assert e_dx <= 2e-2 and e_dl <= 2e-2
    # the sub-batch run: dW_r = dl^T x, dx, dlogits, the shared expert's and the touched
    # experts' weight gradients, all from the oracle
    used = np.unique(c["idx"][toks])
    errs = {n: rel_err(gs[n].float().cpu(), sub[n])
            for n in ("dw_router", "dx", "dlogits", "dws13", "dws2")}

    def stacked_err(name):
        # max |got - ref| / max |ref| over the used experts, one expert at a time (host memory)
        num = den = 0.0
        for e in used:
            gv = gs[name][int(e)].float().cpu().double().numpy()
            num = max(num, float(np.max(np.abs(gv - sub[name][e]))))
            den = max(den, float(np.max(np.abs(sub[name][e]))))
        return num / den
    errs["dw13 (used experts)"] = stacked_err("dw13")
    errs["dw2 (used experts)"] = stacked_err("dw2")
    log("dsv3_bf16 backward, 16-token batch: " + ", ".join(f"{kk} {v:.3e}" for kk, v in errs.items()))
    unused = torch.from_numpy(np.setdiff1d(np.arange(cfg.E), used)).cuda()
    assert float(gs["dw13"][unused].abs().max()) == 0.0
    assert float(gs["dw2"][unused].abs().max()) == 0.0
    assert all(v <= 2e-2 for v in errs.values()), errs
    del gs, sub
    # the hottest and the coldest expert's weight gradients in full
    X = inp.x.double().numpy()
    counts = c["perm"]["counts"]
    nz = np.nonzero(counts)[0]
    lsel = np.take_along_axis(c["logits"].astype(np.float64), c["idx"].astype(np.int64), 1)
    for e in (int(np.argmax(counts)), int(nz[np.argmin(counts[nz])])):
        t, j = np.nonzero(c["idx"] == e)
        s = 1.0 / (1.0 + np.exp(-lsel[t]))
        gate = cfg.route_scale * s[np.arange(len(t)), j] / s.sum(1)
        _, dw13, dw2, _ = oracle._expert_fwd_bwd(X[t], inp.w13[e].double().numpy(),
                                                  inp.w2[e].double().numpy(), gate,
                                                  dy[torch.from_numpy(t)].double().numpy())
        e13 = rel_err(g["dw13"][e].float().cpu(), dw13)
        e2 = rel_err(g["dw2"][e].float().cpu(), dw2)
        log(f"dsv3_bf16 backward: expert {e} ({len(t)} rows) dW13 {e13:.3e} dW2 {e2:.3e}")
        assert e13 <= 2e-2 and e2 <= 2e-2
    # the shared expert over all T tokens (gate 1), the oracle's expert gradient
    _, dws13, dws2, _ = oracle._expert_fwd_bwd(X, inp.ws13.double().numpy(),
                                                inp.ws2.double().numpy(), np.ones(T),
                                                dy.double().numpy())
    e13 = rel_err(g["dws13"].float().cpu(), dws13)
    e2 = rel_err(g["dws2"].float().cpu(), dws2)
    log(f"dsv3_bf16 backward: shared expert dWs13 {e13:.3e} dWs2 {e2:.3e} (all {T} tokens)")
    assert e13 <= 2e-2 and e2 <= 2e-2


def test_full_training_pair_dsv3(moe):
    """The training pair at the DeepSeek-V3 bf16 size in the benchmarked launch configuration
    (K-blocked weights for the forward, row-major ones for the backward):
    moe_layer_forward_train's y and routing equal moe_layer_forward's, and
    moe_layer_backward_saved's gradients equal moe_layer_backward's, bit for bit; so do the
    saved backward's gradients on the forward's K-blocked weight copy."""
    c = full_case(moe, "dsv3_bf16")
    cfg, inp, dev = c["cfg"].replace(a_layout=0), c["inp"], c["dev"]
    log("dsv3_bf16: training pair")
    x, wr = inp.x.cuda(), inp.w_router.cuda()
    lb = None if c["lb"] is None else torch.from_numpy(c["lb"]).cuda()
    sb = None if c["sb"] is None else torch.from_numpy(c["sb"]).cuda()
    want = ("logits", "topk_idx", "topk_gate", "counts")
    y, ex = moe.layer_forward(cfg, x, wr, dev["w13"], dev["w2"], lb, sb, ws13=dev["ws13"],
                              ws2=dev["ws2"], want=want)
    yt, ext, saved = moe.layer_forward_train(cfg, x, wr, dev["w13"], dev["w2"], lb, sb,
                                             ws13=dev["ws13"], ws2=dev["ws2"], want=want)
    torch.cuda.synchronize()
    assert torch.equal(y, yt)
    for n in want:
        assert torch.equal(ex[n], ext[n]), n
    del y, yt, ext
    bcfg = cfg.replace(w_layout=0)
    rm = {n: getattr(inp, n).cuda() for n in ("w13", "w2", "ws13", "ws2")}
    rng = np.random.default_rng(8)
    dy = torch.from_numpy(rng.standard_normal((cfg.T, cfg.H)).astype(np.float32)).to(
        torch.bfloat16).cuda()
    args = (bcfg, x, wr, ex["logits"], ex["topk_idx"], ex["topk_gate"], rm["w13"], rm["w2"], dy)
    kw = dict(logit_bias=lb, ws13=rm["ws13"], ws2=rm["ws2"], want_dlogits=True)
    g = moe.layer_backward(*args, **kw)
    gs = moe.layer_backward_saved(*args, saved, **kw)
    torch.cuda.synchronize()
    for n, t in g.items():
        assert torch.equal(t, gs[n]), n
    log("dsv3_bf16: training pair bit-identical")
    del g
    # the saved backward on the forward's own K-blocked weight copy: the same gradients
    kargs = (cfg, x, wr, ex["logits"], ex["topk_idx"], ex["topk_gate"], dev["w13"], dev["w2"],
             dy)
    gk = moe.layer_backward_saved(*kargs, saved, logit_bias=lb, ws13=dev["ws13"],
                                  ws2=dev["ws2"], want_dlogits=True)
    torch.cuda.synchronize()
    for n, t in gs.items():
        assert torch.equal(t, gk[n]), n
    log("dsv3_bf16: backward on the K-blocked weights bit-identical")

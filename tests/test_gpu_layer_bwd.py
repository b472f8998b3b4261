"""Whole-layer backward (moe_layer_backward) through the C ABI against the oracle's float64
layer backward, on the routing the GPU forward chose. Tolerance: bf16 (2e-2 of the largest
reference value per tensor)."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from helpers import rel_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_expert_softmax_amd as m
    return m


BF = mi.BF16
CASES = {
    # DeepSeek-style router (sigmoid, groups, x2.5) with a shared expert
    "dsv3": mi.scaled(mi.CONFIGS["dsv3_bf16"], T=300, H=512, F=256, shared_F=256),
    # the skewed config's router: a Zipf logit bias on top (bf16 expert weights)
    "dsv3_skew": mi.scaled(mi.CONFIGS["dsv3_fp8_skew"], T=260, H=256, F=128, shared_F=128,
                           w_dtype=BF, backward=True),
    # softmax router, no shared expert, F not a multiple of 256 (128 x 128 tiles)
    "qwen3": mi.scaled(mi.CONFIGS["qwen3_bf16"], T=200, H=256, F=384),
    # a shared expert narrower than the routed ones (its GEMMs run as launches of their own)
    "dsv3_narrow_shared": mi.scaled(mi.CONFIGS["dsv3_bf16"], T=160, H=256, F=256, shared_F=128),
}


@pytest.mark.parametrize("name", list(CASES))
def test_layer_backward(moe, name):
    cfg = CASES[name]
    print(f"[layer bwd] {name}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} F={cfg.F} "
          f"shared={cfg.shared_F}", flush=True)
    inp = mi.make_inputs(cfg)
    rng = np.random.default_rng(97)
    dy = torch.from_numpy(rng.standard_normal((cfg.T, cfg.H)).astype(np.float32)).to(
        torch.bfloat16)
    d = dict(x=inp.x.cuda(), wr=inp.w_router.cuda(), w13=inp.w13.cuda(), w2=inp.w2.cuda(),
             lb=to_dev(inp.logit_bias), sb=to_dev(inp.sel_bias), ws13=to_dev(inp.ws13),
             ws2=to_dev(inp.ws2))
    _, ex = moe.layer_forward(cfg, d["x"], d["wr"], d["w13"], d["w2"], d["lb"], d["sb"],
                              ws13=d["ws13"], ws2=d["ws2"],
                              want=("logits", "topk_idx", "topk_gate"))
    g = moe.layer_backward(cfg, d["x"], d["wr"], ex["logits"], ex["topk_idx"],
                           ex["topk_gate"], d["w13"], d["w2"], dy.cuda(),
                           logit_bias=d["lb"], ws13=d["ws13"], ws2=d["ws2"],
                           want_dlogits=True)
    torch.cuda.synchronize()
    ref = oracle.layer_backward(inp.x, inp.w_router, ex["logits"].cpu().numpy(),
                                ex["topk_idx"].cpu().numpy(), inp.w13, inp.w2, dy,
                                cfg.router, cfg.route_scale,
                                None if inp.logit_bias is None else inp.logit_bias.numpy(),
                                inp.ws13, inp.ws2)
    names = ["dx", "dw_router", "dw13", "dw2", "dlogits"] + (
        ["dws13", "dws2"] if cfg.shared_F else [])
    for n in names:
        err = rel_err(g[n].float().cpu(), ref[n])
        print(f"[layer bwd] {name}: {n} rel err {err:.3e}", flush=True)
        assert err <= 2e-2, n
    # experts that received no rows get zero weight gradients
    counts = np.bincount(ex["topk_idx"].cpu().numpy().ravel(), minlength=cfg.E)
    empty = np.nonzero(counts == 0)[0]
    if empty.size:
        assert torch.count_nonzero(g["dw13"][torch.from_numpy(empty).cuda()]) == 0


def test_layer_backward_deterministic(moe):
    cfg = CASES["dsv3"]
    inp = mi.make_inputs(cfg)
    dy = torch.ones(cfg.T, cfg.H, dtype=torch.bfloat16).cuda()
    x, wr, w13, w2 = inp.x.cuda(), inp.w_router.cuda(), inp.w13.cuda(), inp.w2.cuda()
    ws13, ws2, sb = to_dev(inp.ws13), to_dev(inp.ws2), to_dev(inp.sel_bias)
    _, ex = moe.layer_forward(cfg, x, wr, w13, w2, None, sb, ws13=ws13, ws2=ws2,
                              want=("logits", "topk_idx", "topk_gate"))
    outs = [moe.layer_backward(cfg, x, wr, ex["logits"], ex["topk_idx"], ex["topk_gate"], w13,
                               w2, dy, ws13=ws13, ws2=ws2) for _ in range(2)]
    torch.cuda.synchronize()
    for n in ("dx", "dw_router", "dw13", "dw2", "dws13", "dws2"):
        assert torch.equal(outs[0][n], outs[1][n]), n


@pytest.mark.parametrize("name", list(CASES))
def test_training_pair_bit_identical(moe, name):
    """moe_layer_forward_train keeps GEMM1's Z and act; moe_layer_backward_saved uses them
    instead of recomputing GEMM1. Both must give exactly what moe_layer_forward and
    moe_layer_backward give (the same kernels compute the same values). The dsv3 case runs the
    training forward on K-blocked weights, as the benchmark does; every case then runs both
    backwards on K-blocked weights too."""
    cfg = CASES[name]
    print(f"[train pair] {name}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} F={cfg.F} "
          f"shared={cfg.shared_F}", flush=True)
    inp = mi.make_inputs(cfg)
    rng = np.random.default_rng(41)
    dy = torch.from_numpy(rng.standard_normal((cfg.T, cfg.H)).astype(np.float32)).to(
        torch.bfloat16).cuda()
    x, wr, w13, w2 = inp.x.cuda(), inp.w_router.cuda(), inp.w13.cuda(), inp.w2.cuda()
    ws13, ws2 = to_dev(inp.ws13), to_dev(inp.ws2)
    lb, sb = to_dev(inp.logit_bias), to_dev(inp.sel_bias)
    want = ("logits", "topk_idx", "topk_gate", "counts")
    y, ex = moe.layer_forward(cfg, x, wr, w13, w2, lb, sb, ws13=ws13, ws2=ws2, want=want)
    fcfg, fw = cfg, dict(w13=w13, w2=w2, ws13=ws13, ws2=ws2)
    if name == "dsv3":
        fcfg = cfg.replace(w_layout=1)
        fw = {n: (moe.pack_kblock(t) if t is not None else None) for n, t in fw.items()}
    yt, ext, saved = moe.layer_forward_train(fcfg, x, wr, fw["w13"], fw["w2"], lb, sb,
                                             ws13=fw["ws13"], ws2=fw["ws2"], want=want)
    torch.cuda.synchronize()
    assert torch.equal(y, yt)
    for n in want:
        assert torch.equal(ex[n], ext[n]), n
    args = (cfg, x, wr, ex["logits"], ex["topk_idx"], ex["topk_gate"], w13, w2, dy)
    kw = dict(logit_bias=lb, ws13=ws13, ws2=ws2, want_dlogits=True)
    g = moe.layer_backward(*args, **kw)
    gs = moe.layer_backward_saved(*args, saved, **kw)
    # a second saved backward after the buffer was used once: it is only read
    gs2 = moe.layer_backward_saved(*args, saved, **kw)
    torch.cuda.synchronize()
    for n, t in g.items():
        if t is None:
            assert gs[n] is None, n
            continue
        assert torch.equal(t, gs[n]), n
        assert torch.equal(t, gs2[n]), n
    # both backwards on K-blocked weights (the forward's copy): the same gradients, bit for bit
    kcfg = cfg.replace(w_layout=1)
    kw_ = {n: (moe.pack_kblock(t) if t is not None else None)
           for n, t in dict(w13=w13, w2=w2, ws13=ws13, ws2=ws2).items()}
    kargs = (kcfg, x, wr, ex["logits"], ex["topk_idx"], ex["topk_gate"], kw_["w13"], kw_["w2"],
             dy)
    kkw = dict(logit_bias=lb, ws13=kw_["ws13"], ws2=kw_["ws2"], want_dlogits=True)
    gk = moe.layer_backward(*kargs, **kkw)
    gks = moe.layer_backward_saved(*kargs, saved, **kkw)
    torch.cuda.synchronize()
    for n, t in g.items():
        if t is not None:
            assert torch.equal(t, gk[n]), n
            assert torch.equal(t, gks[n]), n



def test_concurrent_backwards_on_two_streams(moe):
    """The backward's weight gradients run on side streams shared by every caller on a
    device. Two host threads, each queuing layer backwards (one recomputing, one from saved
    activations) on a stream of its own, must get exactly what the same calls give when run
    one after the other."""
    import threading
    cfg = CASES["dsv3"]
    inp = mi.make_inputs(cfg)
    x, wr, w13, w2 = inp.x.cuda(), inp.w_router.cuda(), inp.w13.cuda(), inp.w2.cuda()
    ws13, ws2, sb = to_dev(inp.ws13), to_dev(inp.ws2), to_dev(inp.sel_bias)
    want = ("logits", "topk_idx", "topk_gate")
    _, ex, saved = moe.layer_forward_train(cfg, x, wr, w13, w2, None, sb, ws13=ws13, ws2=ws2,
                                           want=want)
    rng = np.random.default_rng(13)
    dys = [torch.from_numpy(rng.standard_normal((cfg.T, cfg.H)).astype(np.float32)).to(
        torch.bfloat16).cuda() for _ in range(2)]
    args = lambda dy: (cfg, x, wr, ex["logits"], ex["topk_idx"], ex["topk_gate"], w13, w2, dy)
    kw = dict(ws13=ws13, ws2=ws2)
    runs = [lambda ws=None, stream=None: moe.layer_backward(*args(dys[0]), ws=ws, stream=stream,
                                                            **kw),
            lambda ws=None, stream=None: moe.layer_backward_saved(*args(dys[1]), saved, ws=ws,
                                                                  stream=stream, **kw)]
    ref = [r() for r in runs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in runs]
    wss = [moe.workspace(cfg, moe.OP_LAYER_BACKWARD) for _ in runs]
    torch.cuda.synchronize()
    out = [[None] * 3 for _ in runs]

    def worker(i):
        with torch.cuda.stream(streams[i]):
            for rep in range(3):
                out[i][rep] = runs[i](ws=wss[i], stream=streams[i])
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(runs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    for i in range(len(runs)):
        for rep in range(3):
            for n, t in ref[i].items():
                if t is not None:
                    assert torch.equal(t, out[i][rep][n]), (i, rep, n)

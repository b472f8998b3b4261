"""moe_layer_forward and moe_layer_backward captured into a HIP graph (torch.cuda.CUDAGraph)
and replayed.

Neither path synchronises the host, allocates device memory or issues a memset; expert
counts and offsets stay on the device. The forward enqueues on the caller's stream only; the
backward also forks its weight gradients onto the library's side streams and joins them
back, which a capture records as a fork and a join. So both can be captured once and
replayed with new input values. Each replay is checked bit for bit against an eager call on
the same input (the paths are deterministic), with eager work and stream synchronisations
between the replays; in the forward the routing changes from one input to the next, so the
replays also exercise the device-side tile schedule."""
import pytest
import torch

import moe_inputs as mi

pytestmark = pytest.mark.gpu

CASES = {
    # sigmoid + bias, group-limited top-8 of 256, shared expert
    "dsv3_small": mi.scaled(mi.CONFIGS["dsv3_bf16"], T=300, H=256, F=128, shared_F=128),
    # softmax top-8 of 16
    "qwen3_small": mi.scaled(mi.CONFIGS["qwen3_bf16"], T=257, H=256, F=128, E=16),
    # N a multiple of 512 in both GEMMs: the bf16 kernels' mixed 256 / 128-row tile schedule
    "qwen3_mixed_tiles": mi.scaled(mi.CONFIGS["qwen3_bf16"], T=700, H=512, F=256, E=16),
}


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_expert_softmax_amd as m
    return m


def _dev(t):
    return None if t is None else t.cuda()


def _forward(moe, cfg, d, x, y=None, ws=None):
    return moe.layer_forward(cfg, x, d["w_router"], d["w13"], d["w2"],
                             logit_bias=d["logit_bias"], sel_bias=d["sel_bias"],
                             ws13=d["ws13"], ws2=d["ws2"], y=y, ws=ws,
                             want=("topk_idx", "counts"))


def _bits(t):
    return t.contiguous().view(torch.int16)


@pytest.mark.parametrize("name", list(CASES))
def test_layer_forward_graph_replays(moe, name):
    cfg = CASES[name]
    print(f"[graph] {name}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k}", flush=True)
    inp = mi.make_inputs(cfg)
    d = dict(w_router=inp.w_router.cuda(), w13=inp.w13.cuda(), w2=inp.w2.cuda(),
             logit_bias=_dev(inp.logit_bias), sel_bias=_dev(inp.sel_bias),
             ws13=_dev(inp.ws13), ws2=_dev(inp.ws2))
    x_buf = inp.x.cuda()                           # the captured input buffer
    y_buf = torch.empty(cfg.T, cfg.H, dtype=x_buf.dtype, device="cuda")
    ws = moe.workspace(cfg, moe.OP_LAYER_FORWARD, "cuda")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                  # warm-up outside the capture
        for _ in range(2):
            _forward(moe, cfg, d, x_buf, y_buf, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _, ex_g = _forward(moe, cfg, d, x_buf, y_buf, ws)
    torch.cuda.synchronize()

    gen = torch.Generator().manual_seed(20261203)
    for rep in range(3):
        x_new = torch.randn(cfg.T, cfg.H, generator=gen).to(x_buf.dtype).cuda()
        x_buf.copy_(x_new)
        y_ref, ex_ref = _forward(moe, cfg, d, x_new.clone())   # eager, own buffers
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ex_g["topk_idx"], ex_ref["topk_idx"]), rep
        assert torch.equal(ex_g["counts"], ex_ref["counts"]), rep
        assert torch.equal(_bits(y_buf), _bits(y_ref)), rep
        print(f"   replay {rep}: identical to eager (max count {int(ex_ref['counts'].max())})",
              flush=True)


def test_layer_backward_graph_replays(moe):
    """moe_layer_backward captured into a graph: its weight gradients fork onto the library's
    side streams and join back, which a capture records as a fork and a join of the graph.
    Each replay with a new dY equals an eager backward on it, bit for bit."""
    cfg = CASES["dsv3_small"]
    inp = mi.make_inputs(cfg)
    d = dict(w_router=inp.w_router.cuda(), w13=inp.w13.cuda(), w2=inp.w2.cuda(),
             logit_bias=_dev(inp.logit_bias), sel_bias=_dev(inp.sel_bias),
             ws13=_dev(inp.ws13), ws2=_dev(inp.ws2))
    x = inp.x.cuda()
    _, ex = moe.layer_forward(cfg, x, d["w_router"], d["w13"], d["w2"],
                              logit_bias=d["logit_bias"], sel_bias=d["sel_bias"],
                              ws13=d["ws13"], ws2=d["ws2"],
                              want=("logits", "topk_idx", "topk_gate"))
    dy_buf = torch.zeros(cfg.T, cfg.H, dtype=torch.bfloat16, device="cuda")
    ws = moe.workspace(cfg, moe.OP_LAYER_BACKWARD, "cuda")

    def backward(dy, ws=None):
        return moe.layer_backward(cfg, x, d["w_router"], ex["logits"], ex["topk_idx"],
                                  ex["topk_gate"], d["w13"], d["w2"], dy,
                                  logit_bias=d["logit_bias"], ws13=d["ws13"], ws2=d["ws2"],
                                  ws=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                  # warm-up outside the capture
        for _ in range(2):
            backward(dy_buf, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g_out = backward(dy_buf, ws)
    torch.cuda.synchronize()

    gen = torch.Generator().manual_seed(20261204)
    for rep in range(3):
        dy_new = torch.randn(cfg.T, cfg.H, generator=gen).to(torch.bfloat16).cuda()
        dy_buf.copy_(dy_new)
        ref = backward(dy_new.clone())             # eager, own buffers and workspace
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n, t in ref.items():
            if t is not None:
                assert torch.equal(_bits(g_out[n]), _bits(t)), (rep, n)
        print(f"   backward replay {rep}: identical to eager", flush=True)

"""Degenerate and boundary shapes of the whole layer through the C ABI, against the oracle:
one token, a single expert (a dense SwiGLU MLP), every expert selected (k = E), odd sizes
that fill no tile, and a routing that leaves most experts empty. Routing runs on the
oracle's logits, so the expert sets must match exactly; outputs meet the dtype tolerance."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from helpers import rel_err, tol, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_expert_softmax_amd as m
    return m


MIX, QWEN, DS = mi.CONFIGS["mixtral_bf16"], mi.CONFIGS["qwen3_bf16"], mi.CONFIGS["dsv3_bf16"]
CASES = {
    # one token: E - k experts empty, every GEMM tile holds one live row
    "ds_one_token": (mi.scaled(DS, T=1, H=256, F=128, shared_F=128), None),
    "fp32_one_token": (mi.scaled(mi.CONFIGS["tiny_fp32"], T=1), None),
    # E = k = 1: the gate is 1 and the layer is a plain SwiGLU MLP
    "single_expert": (mi.scaled(MIX, T=70, H=256, F=128, E=1, k=1), None),
    # k = E: every token visits every expert; gates are the full softmax
    "all_experts": (mi.scaled(MIX, T=65, H=256, F=128, E=8, k=8), None),
    # sizes that fill no tile: T * k = 231 rows over 16 experts
    "odd_sizes": (mi.scaled(QWEN, T=77, H=256, F=128, E=16, k=3), None),
    # a bias that sends every token to experts 0 and 1: six experts stay empty, two hold T
    # rows each (several M tiles of one expert)
    "two_hot_experts": (mi.scaled(MIX, T=600, H=256, F=128, E=8, k=2),
                        np.array([50, 49, 0, 0, 0, 0, 0, 0], np.float32)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_layer_edge_case(moe, name):
    cfg, lb_np = CASES[name]
    print(f"[edge] {name}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} F={cfg.F}", flush=True)
    inp = mi.make_inputs(cfg)
    lb = lb_np if lb_np is not None else (None if inp.logit_bias is None
                                           else inp.logit_bias.numpy())
    sb = None if inp.sel_bias is None else inp.sel_bias.numpy()
    logits = oracle.router_logits(inp.x, inp.w_router)
    idx, gate = oracle.route_cfg(cfg, logits, lb, sb)
    y, ex = moe.layer_forward(
        cfg, inp.x.cuda(), inp.w_router.cuda(), inp.w13.cuda(), inp.w2.cuda(),
        None if lb is None else torch.from_numpy(lb).cuda(), to_dev(inp.sel_bias),
        torch.from_numpy(np.ascontiguousarray(logits, np.float32)).cuda(),
        ws13=to_dev(inp.ws13), ws2=to_dev(inp.ws2), want=("topk_idx", "counts"))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ex["topk_idx"].cpu().numpy(), idx)
    np.testing.assert_array_equal(ex["counts"].cpu().numpy(),
                                  np.bincount(np.asarray(idx).ravel(), minlength=cfg.E))
    ref = oracle.layer_tokens(inp.x, idx, gate, inp.w13, inp.w2, np.arange(cfg.T), inp.ws13,
                              inp.ws2)
    err = rel_err(y.cpu(), ref)
    print(f"[edge] {name}: rel err {err:.3e}", flush=True)
    assert err <= tol(cfg)


def test_binding_rejects_misaligned_tensor(moe):
    """A contiguous tensor whose data starts 2 bytes into an allocation is refused by the
    binding before anything is launched (the kernels move 16-byte vectors)."""
    cfg = mi.scaled(mi.CONFIGS["qwen3_bf16"], T=4, H=256, F=128, E=16)
    raw = torch.empty(cfg.T * cfg.H * 2 + 16, dtype=torch.uint8, device="cuda")
    x_bad = raw[2:2 + cfg.T * cfg.H * 2].view(torch.bfloat16).view(cfg.T, cfg.H)
    assert x_bad.is_contiguous() and x_bad.data_ptr() % 16 == 2
    w_r = torch.zeros(cfg.E, cfg.H, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="16-byte aligned"):
        moe.router_logits(cfg, x_bad, w_r)

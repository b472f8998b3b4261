"""Ragged M tiles of the grouped GEMMs at the row counts where the tile boundaries move: one
row past a tile (257, 513, 2049 rows), counts between tile multiples (300, 767), exact
multiples (256, 512 - 1, 32), tiny and empty experts, and remainders around 128 rows past a
multiple of 256 (128, 129, 384, 385, 640, 100), where the bf16 kernels switch between a last
256-row tile and a last 128-row tile on the 128 x 512 shape (the shape is used when N is a
multiple of 512: the H512F256 case takes it in both GEMMs, F256 in the up GEMM only).
The expert-grouped offsets are set directly (one slot per token, k = 1), every output row is
compared with the oracle's expert math, and the backward's data gradients and gate gradients
use the same offsets."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from helpers import rel_err, tol

pytestmark = pytest.mark.gpu

COUNTS = np.array([257, 300, 0, 513, 33, 1, 2049, 32, 511, 767, 256, 255, 128, 129, 384, 385,
                   640, 100], np.int64)
SHAPES = {"F128": dict(H=256, F=128), "F256": dict(H=256, F=256),
          "H512F256": dict(H=512, F=256)}


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_expert_softmax_amd as m
    return m


def bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16)


def case(shape):
    A = int(COUNTS.sum())
    cfg = mi.scaled(mi.CONFIGS["mixtral_bf16"], T=A, k=1, E=len(COUNTS), **SHAPES[shape])
    inp = mi.make_inputs(cfg)
    offsets = np.concatenate([[0], np.cumsum(COUNTS)]).astype(np.int32)
    gate = np.random.default_rng(5).uniform(0.1, 1.0, A).astype(np.float32)
    return cfg, inp, offsets, gate


@pytest.mark.parametrize("shape", list(SHAPES))
def test_forward_rows_around_tile_boundaries(moe, shape):
    cfg, inp, offsets, gate = case(shape)
    print(f"[split] forward {shape}: rows {COUNTS.tolist()}", flush=True)
    T32 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    out = moe.grouped_gemm_swiglu(cfg, inp.x.cuda(), T32(offsets), T32(gate), inp.w13.cuda(),
                                  inp.w2.cuda())
    torch.cuda.synchronize()
    _, act_ref, y_ref = oracle.expert_rows(inp.x, offsets, gate, inp.w13, inp.w2,
                                           np.arange(cfg.A))
    e_act = rel_err(out["act"].cpu(), act_ref)
    e_y = rel_err(out["y_perm"].cpu(), y_ref)
    # every expert's first and last row on its own, so a wrong tile boundary cannot hide in
    # the global max
    worst = 0.0
    act, y = out["act"].cpu().double().numpy(), out["y_perm"].cpu().double().numpy()
    scale_a, scale_y = np.abs(act_ref).max(), np.abs(y_ref).max()
    for e in np.nonzero(COUNTS)[0]:
        for r in (offsets[e], offsets[e + 1] - 1):
            worst = max(worst, np.abs(act[r] - act_ref[r]).max() / scale_a,
                        np.abs(y[r] - y_ref[r]).max() / scale_y)
    print(f"   act {e_act:.3e}  y_perm {e_y:.3e}  segment edges {worst:.3e}", flush=True)
    assert e_act <= tol(cfg) and e_y <= tol(cfg) and worst <= tol(cfg)


@pytest.mark.parametrize("shape", list(SHAPES))
def test_backward_rows_around_tile_boundaries(moe, shape):
    cfg, inp, offsets, gate = case(shape)
    print(f"[split] backward {shape}: rows {COUNTS.tolist()}", flush=True)
    z, act, _ = oracle.expert_rows(inp.x, offsets, gate, inp.w13, inp.w2, np.arange(cfg.A),
                                   want_z=True)
    zb, ab = bf16(z), bf16(act)
    dy = torch.from_numpy(np.random.default_rng(6).standard_normal((cfg.A, cfg.H), np.float32)
                          ).to(torch.bfloat16)
    T32 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    out = moe.grouped_gemm_swiglu_bwd(cfg, dy.cuda(), inp.x.cuda(), zb.cuda(), ab.cuda(),
                                      T32(gate), T32(offsets), inp.w13.cuda(), inp.w2.cuda())
    torch.cuda.synchronize()
    dx_ref, dg_ref = oracle.expert_bwd_rows(dy, zb, offsets, gate, inp.w13, inp.w2,
                                            np.arange(cfg.A))
    e_dx = rel_err(out["dx_perm"].cpu(), dx_ref)
    e_dg = rel_err(out["dgate_perm"].cpu(), dg_ref)
    rng = np.random.default_rng(7)
    worst = 0.0
    for e in (0, 6):                       # 257 and 2049 rows: K of the weight gradients
        r13, c13 = rng.integers(0, 2 * cfg.F, 64), rng.integers(0, cfg.H, 64)
        r2, c2 = rng.integers(0, cfg.H, 64), rng.integers(0, cfg.F, 64)
        ref13, ref2 = oracle.expert_wgrad_entries(dy, zb, ab, inp.x, offsets, e, gate, inp.w2,
                                                  (r13, c13), (r2, c2))
        worst = max(worst, rel_err(out["dw13"][e].cpu()[r13, c13].double().numpy(), ref13),
                    rel_err(out["dw2"][e].cpu()[r2, c2].double().numpy(), ref2))
    assert not out["dw13"][2].cpu().any() and not out["dw2"][2].cpu().any()   # empty expert
    print(f"   dx {e_dx:.3e}  dg {e_dg:.3e}  dW (sampled) {worst:.3e}", flush=True)
    assert e_dx <= 2e-2 and e_dg <= 2e-2 and worst <= 2e-2

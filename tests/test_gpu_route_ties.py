"""moe_route on crafted logits full of exact ties, bit-exact against the oracle.

The selection step of the per-token loop (study notes "Megatron-Core MoE -- 大规模稀疏专家并行
实践", 实践案例 案例 1) takes the k best experts; equal keys go to the lower expert index and
-0.0 ties +0.0. These cases feed moe_route logits where that rule decides most of the
selection: all-equal rows, -0.0/+0.0 mixes, half-integer logits with many exact ties, and for
the group-limited sigmoid router groups whose scores tie exactly -- on the 32-lane group path
(groups of 32 experts, E a multiple of 64) and on the general group path. Indices must be
bit-exact and gates within 1e-6 of the oracle's."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_expert_softmax_amd as m
    return m


def softmax_cfg(E, k, T):
    return mi.CONFIGS["qwen3_bf16"].replace(T=T, E=E, k=k, H=256, F=128)


def sigmoid_cfg(E, G, TG, k, T):
    return mi.CONFIGS["dsv3_bf16"].replace(T=T, E=E, k=k, n_groups=G, topk_groups=TG,
                                           H=256, F=128, shared_F=0)


def run(moe, cfg, logits, logit_bias=None, sel_bias=None):
    dev = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    idx, gate = moe.route(cfg, dev(logits), dev(logit_bias), dev(sel_bias))
    torch.cuda.synchronize()
    ref_idx, ref_gate = oracle.route_cfg(cfg, logits, logit_bias, sel_bias)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_allclose(gate.cpu().numpy(), ref_gate, rtol=1e-6, atol=0)
    return ref_idx


def tie_rows(T, E, seed):
    """Rows that make the tie rule decide: all +0.0, all -0.0, a -0.0/+0.0 mix, a constant,
    then half-integer logits in [-2, 2] (9 values over E experts: many exact ties) with a
    random sign of zero."""
    rng = np.random.default_rng(seed)
    lg = np.round(rng.uniform(-2, 2, (T, E)) * 2).astype(np.float32) / np.float32(2)
    zeros = lg == 0
    lg[zeros] = np.where(rng.random(int(zeros.sum())) < 0.5, np.float32(-0.0), np.float32(0.0))
    lg[0] = 0.0
    lg[1] = -0.0
    lg[2] = np.where(np.arange(E) % 3 == 0, np.float32(-0.0), np.float32(0.0))
    lg[3] = 1.5
    return lg


@pytest.mark.parametrize("E,k", [(8, 2), (128, 8), (256, 8), (64, 32), (1000, 17)])
def test_softmax_ties(moe, E, k):
    T = 517
    print(f"[route ties] softmax E={E} k={k}", flush=True)
    lg = tie_rows(T, E, seed=E + k)
    idx = run(moe, softmax_cfg(E, k, T), lg)
    # all-equal rows (any sign of zero, or a constant) select experts 0..k-1 in order
    for t in range(4):
        np.testing.assert_array_equal(idx[t], np.arange(k))


@pytest.mark.parametrize("E,k", [(8, 2), (256, 8)])
def test_softmax_ties_with_logit_bias(moe, E, k):
    """A half-integer logit bias keeps the keys on the half-integer grid: still many ties."""
    T = 300
    print(f"[route ties] softmax + logit bias E={E} k={k}", flush=True)
    lg = tie_rows(T, E, seed=7 * E)
    lb = (np.arange(E) % 3 - 1).astype(np.float32) * np.float32(0.5)
    run(moe, softmax_cfg(E, k, T), lg, logit_bias=lb)


# (E, n_groups, topk_groups, k): the first three take the 32-lane group path (groups of 32
# experts, E a multiple of 64), the others the general group path
SIG = [(256, 8, 4, 8), (64, 2, 1, 4), (512, 16, 3, 8), (96, 3, 2, 6), (64, 4, 2, 8),
       (120, 5, 3, 7)]


@pytest.mark.parametrize("E,G,TG,k", SIG)
def test_sigmoid_tied_group_scores(moe, E, G, TG, k):
    """Every group holds the same half-integer pattern, so all group scores tie exactly and
    the lowest groups must be kept; inside them equal keys go to the lower index."""
    T = 400
    per = E // G
    print(f"[route ties] sigmoid tied groups E={E} G={G} TG={TG} k={k}", flush=True)
    rng = np.random.default_rng(E * G + k)
    pat = np.round(rng.uniform(-2, 2, (T, per)) * 2).astype(np.float32) / np.float32(2)
    lg = np.tile(pat, (1, G))
    lg[0] = 0.0                                     # every key equal
    cfg = sigmoid_cfg(E, G, TG, k, T)
    idx = run(moe, cfg, lg, sel_bias=np.zeros(E, np.float32))
    assert np.all(idx < TG * per)                   # only the lowest TG groups are kept
    np.testing.assert_array_equal(idx[0], np.arange(k))
    run(moe, cfg, lg, sel_bias=None)


@pytest.mark.parametrize("E,G,TG,k", SIG)
def test_sigmoid_half_integer_ties(moe, E, G, TG, k):
    """Random half-integer logits (ties inside and across groups) with a selection bias on a
    coarse grid (more ties between keys), and a Zipf-like logit bias on the same grid."""
    T = 400
    print(f"[route ties] sigmoid half-integer E={E} G={G} TG={TG} k={k}", flush=True)
    lg = tie_rows(T, E, seed=3 * E + G)
    rng = np.random.default_rng(E + TG)
    sb = (rng.integers(-2, 3, E) * 0.0625).astype(np.float32)
    lb = (rng.integers(-1, 2, E) * 0.5).astype(np.float32)
    cfg = sigmoid_cfg(E, G, TG, k, T)
    run(moe, cfg, lg, sel_bias=sb)
    run(moe, cfg, lg, logit_bias=lb, sel_bias=sb)

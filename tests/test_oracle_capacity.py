"""Pins of the oracle's token-dropping permutation (expert capacity), of the dropped-slot
handling in combine / layer_tokens, and of the mean router probabilities: a numpy
restatement of first-come-first-served slots, the dropless limit, the fold identity (a
dropped slot is the same as a zero gate), closed forms and torch's softmax / sigmoid."""
import numpy as np
import pytest
import torch

import oracle


def routed(T, E, k, seed, skew=0.0):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg += (skew * -np.log(np.arange(1, E + 1))).astype(np.float32)   # a few hot experts
    return oracle.route(lg, k)


def numpy_capacity(idx, E, cap):
    """kept[a] for the flattened assignments a = t * k + j: fewer than cap earlier
    assignments (in a order) to the same expert."""
    flat = idx.reshape(-1)
    kept = np.zeros(flat.size, bool)
    for e in range(E):
        where = np.flatnonzero(flat == e)
        kept[where[:cap]] = True
    return kept


@pytest.mark.parametrize("T,E,k,cap,skew", [(64, 8, 2, 5, 2.0), (300, 16, 4, 40, 1.0),
                                            (33, 4, 1, 1, 0.0), (50, 8, 3, 1000, 3.0)])
def test_capacity_permutation_first_come_first_served(T, E, k, cap, skew):
    idx, gate = routed(T, E, k, seed=T + E, skew=skew)
    out = oracle.permute(idx, gate, E, capacity=cap)
    kept = numpy_capacity(idx, E, cap)
    flat = idx.reshape(-1)
    np.testing.assert_array_equal(out["counts"], np.bincount(flat, minlength=E))
    kept_counts = np.minimum(np.bincount(flat, minlength=E), cap)
    np.testing.assert_array_equal(out["offsets"], np.concatenate([[0], np.cumsum(kept_counts)]))
    np.testing.assert_array_equal(out["pos"].reshape(-1) >= 0, kept)
    # kept rows: grouped by expert, token order inside (a stable sort of the kept ones)
    a_kept = np.flatnonzero(kept)
    order = a_kept[np.argsort(flat[a_kept], kind="stable")]
    n = out["offsets"][E]
    np.testing.assert_array_equal(out["src"][:n], order // k)
    np.testing.assert_array_equal(out["gate_perm"][:n], gate.reshape(-1)[order])
    np.testing.assert_array_equal(out["pos"].reshape(-1)[order], np.arange(n))


def test_large_capacity_is_dropless():
    idx, gate = routed(200, 8, 2, seed=1, skew=2.0)
    a = oracle.permute(idx, gate, 8)
    b = oracle.permute(idx, gate, 8, capacity=400)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)


def test_expert_capacity_formula():
    assert oracle.expert_capacity(0.0, 10, 2, 4) is None
    assert oracle.expert_capacity(1.0, 10, 2, 4) == 5
    assert oracle.expert_capacity(1.25, 10, 2, 4) == 7          # ceil(6.25)
    assert oracle.expert_capacity(0.5, 4, 2, 4) == 1            # exactly 1.0
    # 1.1 is rounded to fp32 (1.10000002...) before the product: ceil(5.5000001) = 6
    assert oracle.expert_capacity(1.1, 10, 2, 4) == 6
    assert oracle.expert_capacity(100.0, 10, 2, 4) == 20        # at most T * k


def test_dropped_slot_equals_zero_gate():
    """With the gate folded in, a dropped slot contributes exactly what a zero gate does."""
    T, H, E, k, F = 24, 32, 4, 2, 16
    g = torch.Generator().manual_seed(3)
    x = torch.randn(T, H, generator=g)
    w13 = torch.randn(E, 2 * F, H, generator=g) * 0.1
    w2 = torch.randn(E, H, F, generator=g) * 0.1
    idx, gate = routed(T, E, k, seed=5, skew=2.0)
    perm = oracle.permute(idx, gate, E, capacity=8)
    assert (perm["pos"] < 0).any()
    y_drop = oracle.layer_tokens(x, oracle.drop_slots(idx, perm["pos"]), gate, w13, w2,
                                 np.arange(T))
    gz = np.where(perm["pos"] < 0, 0.0, gate).astype(np.float32)
    y_zero = oracle.layer_tokens(x, idx, gz, w13, w2, np.arange(T))
    np.testing.assert_allclose(y_drop, y_zero, rtol=0, atol=1e-12)
    # and the combine of the expert rows skips the dropped slots the same way
    n = int(perm["offsets"][E])
    x_perm = x.numpy()[perm["src"][:n]]                  # row r holds token src[r]
    _, _, yp = oracle.expert_rows(x_perm, perm["offsets"], perm["gate_perm"], w13, w2,
                                  np.arange(n))
    y_comb = oracle.combine(yp.astype(np.float32), perm["pos"])
    np.testing.assert_allclose(y_comb, y_drop, rtol=0, atol=1e-5)


class _Cfg:
    def __init__(self, router):
        self.router = router


def test_prob_mean_softmax_matches_torch():
    rng = np.random.default_rng(9)
    lg = rng.standard_normal((37, 24)).astype(np.float32) * 3
    lb = rng.standard_normal(24).astype(np.float32)
    pm = oracle.route_prob_mean(_Cfg(oracle.SOFTMAX_TOPK), lg, lb)
    l = torch.from_numpy(lg) + torch.from_numpy(lb)
    ref = torch.softmax(l.double(), dim=1).mean(0).numpy()
    np.testing.assert_allclose(pm, ref, rtol=1e-12)
    assert abs(pm.sum() - 1.0) < 1e-12
    # equal logits: every expert gets 1/E
    np.testing.assert_allclose(oracle.route_prob_mean(_Cfg(oracle.SOFTMAX_TOPK),
                                                      np.zeros((5, 24), np.float32)),
                               np.full(24, 1 / 24), rtol=1e-14)


def test_prob_mean_sigmoid_matches_torch():
    rng = np.random.default_rng(10)
    lg = rng.standard_normal((41, 32)).astype(np.float32) * 2
    pm = oracle.route_prob_mean(_Cfg(oracle.SIGMOID_GROUP_TOPK), lg)
    s = torch.sigmoid(torch.from_numpy(lg).double()).float().double()
    ref = (s / s.sum(1, keepdim=True)).mean(0).numpy()
    np.testing.assert_allclose(pm, ref, rtol=1e-7)
    assert abs(pm.sum() - 1.0) < 1e-12

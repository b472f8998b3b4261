"""Pins of the oracle's router, top-k, gates and permutation metadata against library
routines (numpy lexsort / argsort / bincount, torch softmax / sigmoid), closed forms,
brute force on tiny inputs and the routing-event count the pages print."""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def lexsort_topk(key, k):
    """Top-k by (key desc, index asc) via numpy's stable lexsort."""
    T, E = key.shape
    out = np.empty((T, k), np.int64)
    idx = np.arange(E)
    for t in range(T):
        order = np.lexsort((idx, -key[t].astype(np.float64)))
        out[t] = order[:k]
    return out


def random_logits(T, E, seed, ties=False):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if ties:
        lg = np.round(lg * 2) / 2                 # many exact ties
        lg[np.abs(lg) == 0] = np.where(rng.random(np.sum(np.abs(lg) == 0)) < 0.5, -0.0, 0.0)
    return lg


@pytest.mark.parametrize("E,k,ties", [(8, 2, False), (8, 2, True), (128, 8, False),
                                      (128, 8, True), (16, 16, False), (5, 1, True)])
def test_softmax_topk_matches_lexsort(E, k, ties):
    lg = random_logits(300, E, seed=E * 10 + k, ties=ties)
    idx, gate = oracle.route(lg, k)
    np.testing.assert_array_equal(idx, lexsort_topk(lg, k))


def test_all_equal_logits_pick_lowest_indices():
    lg = np.zeros((4, 16), np.float32)
    lg[1] = -0.0                                  # -0.0 ties with +0.0
    lg[2, ::2] = -0.0
    lg[3] = 1.5
    idx, gate = oracle.route(lg, 4)
    for t in range(4):
        np.testing.assert_array_equal(idx[t], [0, 1, 2, 3])
        np.testing.assert_allclose(gate[t], 0.25, rtol=0, atol=0)


def test_bruteforce_topk_subset():
    """For tiny E, enumerate every k-subset: exactly one has each member ranking before
    every non-member, and it is the oracle's selection."""
    rng = np.random.default_rng(7)
    for trial in range(200):
        E, k = rng.integers(2, 7), 0
        k = int(rng.integers(1, E + 1))
        key = (rng.integers(-3, 4, E) / 2).astype(np.float32)
        idx, _ = oracle.route(key[None], k)

        def before(a, b):
            return key[a] > key[b] or (key[a] == key[b] and a < b)
        good = [S for S in itertools.combinations(range(E), k)
                if all(before(a, b) for a in S for b in range(E) if b not in S)]
        assert len(good) == 1
        assert sorted(idx[0].tolist()) == list(good[0])
        # slot order is rank order
        for j in range(k - 1):
            assert before(idx[0, j], idx[0, j + 1])


def test_softmax_gates_closed_forms():
    lg = random_logits(500, 64, seed=11) * 3
    idx, gate = oracle.route(lg, 6)
    # renormalised gates sum to one (each gate is rounded to fp32 once)
    np.testing.assert_allclose(gate.astype(np.float64).sum(1), 1.0, rtol=0, atol=6 * 2.0 ** -24)
    # equal to the full softmax renormalised over the kept experts (torch, fp64)
    full = torch.softmax(torch.from_numpy(lg).double(), dim=1).numpy()
    sel = np.take_along_axis(full, idx.astype(np.int64), 1)
    ref = sel / sel.sum(1, keepdims=True)
    np.testing.assert_allclose(gate, ref, rtol=2 ** -23, atol=0)
    # k = E: the gates are exactly the full softmax
    idx2, gate2 = oracle.route(lg[:, :8], 8)
    full8 = torch.softmax(torch.from_numpy(lg[:, :8]).double(), dim=1).numpy()
    np.testing.assert_allclose(gate2, np.take_along_axis(full8, idx2.astype(np.int64), 1),
                               rtol=2 ** -23, atol=0)


def test_logit_bias_is_added_in_fp32():
    lg = random_logits(64, 8, seed=5)
    b = np.random.default_rng(6).standard_normal(8).astype(np.float32)
    idx, gate = oracle.route(lg, 2, logit_bias=b)
    idx_ref, gate_ref = oracle.route((lg + b).astype(np.float32), 2)
    np.testing.assert_array_equal(idx, idx_ref)
    np.testing.assert_array_equal(gate, gate_ref)


def ds_numpy(lg, b, G, TG, k, scale):
    """DeepSeek-style sigmoid router via library primitives (torch sigmoid, numpy sorts)."""
    s = torch.sigmoid(torch.from_numpy(lg).double()).float().numpy()
    key = (s + b).astype(np.float32)
    T, E = lg.shape
    per = E // G
    idx = np.empty((T, k), np.int64)
    for t in range(T):
        grp = key[t].reshape(G, per)
        top2 = -np.sort(-grp, axis=1)[:, :2]
        gscore = (top2[:, 0] + top2[:, 1]).astype(np.float32)
        gorder = np.lexsort((np.arange(G), -gscore.astype(np.float64)))[:TG]
        mask = np.zeros(E, bool)
        for g in gorder:
            mask[g * per:(g + 1) * per] = True
        cand = np.nonzero(mask)[0]
        order = np.lexsort((cand, -key[t, cand].astype(np.float64)))
        idx[t] = cand[order[:k]]
    sel = np.take_along_axis(s.astype(np.float64), idx, 1)
    gate = scale * sel / sel.sum(1, keepdims=True)
    return s, idx, gate


@pytest.mark.parametrize("E,G,TG,k", [(256, 8, 4, 8), (64, 4, 2, 6), (32, 8, 8, 4)])
def test_sigmoid_group_router_matches_library_version(E, G, TG, k):
    rng = np.random.default_rng(E + G)
    lg = (rng.standard_normal((200, E)) * 2).astype(np.float32)
    b = (rng.standard_normal(E) * 0.01).astype(np.float32)
    idx, gate, s = oracle.route(lg, k, oracle.SIGMOID_GROUP_TOPK, None, b, G, TG, 2.5,
                                return_scores=True)
    s_ref, idx_ref, gate_ref = ds_numpy(lg, b, G, TG, k, 2.5)
    # fp64 sigmoid rounded once to fp32: libm exp vs torch exp agree to the last fp32 bit
    np.testing.assert_array_equal(s, s_ref)
    np.testing.assert_array_equal(idx, idx_ref)
    np.testing.assert_allclose(gate, gate_ref, rtol=2 ** -23, atol=0)
    np.testing.assert_allclose(gate.astype(np.float64).sum(1), 2.5, rtol=k * 2.0 ** -23)


def test_sigmoid_router_reduces_to_plain_topk():
    """All groups kept and zero bias: plain top-k of the sigmoid scores."""
    rng = np.random.default_rng(9)
    lg = rng.standard_normal((100, 32)).astype(np.float32)
    idx, gate, s = oracle.route(lg, 4, oracle.SIGMOID_GROUP_TOPK, None, np.zeros(32, np.float32),
                                4, 4, 1.0, return_scores=True)
    np.testing.assert_array_equal(idx, lexsort_topk(s, 4))
    # sigmoid is monotone: the same experts as the plain top-k of the logits, unless two
    # logits round to the same fp32 score
    sel = np.take_along_axis(s.astype(np.float64), idx.astype(np.int64), 1)
    np.testing.assert_allclose(gate, sel / sel.sum(1, keepdims=True), rtol=2 ** -23)


def test_group_limit_excludes_experts():
    """An expert with the largest key in a losing group is not selected."""
    E, G = 16, 4
    lg = np.full((1, E), -4.0, np.float32)
    lg[0, 0] = 6.0            # group 0: one large key, the rest small
    lg[0, 4:8] = 2.0          # group 1: uniformly large -> larger top-2 sum
    lg[0, 8:12] = 1.9         # group 2
    idx, _ = oracle.route(lg, 2, oracle.SIGMOID_GROUP_TOPK, None, np.zeros(E, np.float32),
                          G, 2, 1.0)
    # top-2 sums: g0 = s(6)+s(-4) ~ 1.015, g1 = 2 s(2) ~ 1.76, g2 = 2 s(1.9) ~ 1.74
    assert 0 not in idx[0]
    np.testing.assert_array_equal(idx[0], [4, 5])


def check_permutation(idx, gate, E, perm):
    T, k = idx.shape
    flat = idx.reshape(-1)
    np.testing.assert_array_equal(perm["counts"], np.bincount(flat, minlength=E))
    assert perm["counts"].sum() == T * k
    np.testing.assert_array_equal(perm["offsets"], np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    order = np.argsort(flat, kind="stable")              # row -> flat assignment
    inv = np.empty_like(order)
    inv[order] = np.arange(order.size)
    np.testing.assert_array_equal(perm["pos"].reshape(-1), inv)
    assert np.array_equal(np.sort(perm["pos"].reshape(-1)), np.arange(T * k))   # bijection
    np.testing.assert_array_equal(perm["src"][perm["pos"].reshape(-1)], np.repeat(np.arange(T), k))
    np.testing.assert_array_equal(perm["gate_perm"][perm["pos"].reshape(-1)], gate.reshape(-1))


@pytest.mark.parametrize("T,E,k", [(256, 8, 2), (1000, 128, 8), (7, 256, 8), (1, 4, 4)])
def test_permutation_matches_stable_argsort(T, E, k):
    lg = random_logits(T, E, seed=T + E, ties=True)
    idx, gate = oracle.route(lg, k)
    check_permutation(idx, gate, E, oracle.permute(idx, gate, E))


def test_permutation_with_empty_experts():
    idx = np.array([[3, 1], [1, 3], [3, 0]], np.int32)
    gate = np.ones((3, 2), np.float32)
    perm = oracle.permute(idx, gate, 6)
    np.testing.assert_array_equal(perm["counts"], [1, 2, 0, 3, 0, 0])
    np.testing.assert_array_equal(perm["offsets"], [0, 1, 3, 3, 6, 6, 6])
    np.testing.assert_array_equal(perm["pos"], [[3, 1], [2, 4], [5, 0]])
    np.testing.assert_array_equal(perm["src"], [2, 0, 1, 0, 1, 2])


def test_routing_event_count_from_the_pages():
    """The pages' worked count: 1M tokens with 2 experts per token give 2M routing events.
    Dropless routing must turn every one of them into a row of the grouped buffer."""
    with open(os.path.join(GOLDEN, "routing_events.json")) as f:
        g = json.load(f)
    T, k, events = g["tokens"], g["experts_per_token"], g["routing_events"]
    lg = np.random.default_rng(0).standard_normal((T, 8)).astype(np.float32)
    idx, gate = oracle.route(lg, k)
    perm = oracle.permute(idx, gate, 8)
    assert int(perm["counts"].sum()) == events
    assert int(perm["offsets"][-1]) == events


def test_combine_inverts_the_permutation():
    """Combining the permuted copy of x (every row an identical expert output) gives k x."""
    rng = np.random.default_rng(12)
    T, E, k, H = 50, 16, 3, 24
    lg = rng.standard_normal((T, E)).astype(np.float32)
    idx, gate = oracle.route(lg, k)
    perm = oracle.permute(idx, gate, E)
    x = rng.standard_normal((T, H)).astype(np.float32)
    xp = oracle.gather_rows(x, perm["pos"])
    np.testing.assert_array_equal(oracle.combine(xp, perm["pos"]), k * x.astype(np.float64))
    sh = rng.standard_normal((T, H)).astype(np.float32)
    np.testing.assert_allclose(oracle.combine(xp, perm["pos"], sh), k * x.astype(np.float64) + sh,
                               rtol=1e-15)
    # rows of expert e are the tokens routed to e, in ascending token order
    for e in range(E):
        rows = np.arange(perm["offsets"][e], perm["offsets"][e + 1])
        toks = perm["src"][rows]
        assert np.all(np.diff(toks) > 0)
        assert set(toks) == set(np.nonzero((idx == e).any(1))[0])


def _exact_logits(x64, w64):
    """Router scores from their definition with no rounding before the end: every product of
    two fp32 (or bf16) values is exact in fp64, and math.fsum returns the correctly rounded
    sum of the exact products; one rounding to fp32 follows."""
    import math
    T, E = x64.shape[0], w64.shape[0]
    out = np.empty((T, E), np.float64)
    for t in range(T):
        prod = x64[t][None, :] * w64            # [E, H], exact
        for e in range(E):
            out[t, e] = math.fsum(prod[e])
    return out


@pytest.mark.parametrize("dtype,T,H,E", [("f32", 37, 129, 13), ("bf16", 29, 257, 7),
                                          ("f32", 5, 1, 3), ("bf16", 16, 64, 24)])
def test_router_logits_match_exact_matmul(dtype, T, H, E):
    """Pin of the scoring step (study notes, 实践案例 案例 1; linear router without bias):
    logits = fp32(x W_r^T) with W_r stored [E, H]. Checked against (a) the exactly rounded
    definition (fsum of exact products) and (b) numpy's fp64 matmul, bit-equal after the
    fp32 rounding. An odd H and an E that is not a multiple of 8 are included; a reading of
    W_r as [H, E] or an fp32 accumulation would break the bit-equality."""
    rng = np.random.default_rng(1000 + T * H + E)
    x = rng.standard_normal((T, H)).astype(np.float32)
    w = (rng.standard_normal((E, H)) * 0.5).astype(np.float32)
    if dtype == "bf16":
        xt = torch.from_numpy(x).to(torch.bfloat16)
        wt = torch.from_numpy(w).to(torch.bfloat16)
        x64, w64 = xt.double().numpy(), wt.double().numpy()
        got = oracle.router_logits(xt, wt)
    else:
        x64, w64 = x.astype(np.float64), w.astype(np.float64)
        got = oracle.router_logits(x, w)
    assert got.shape == (T, E) and got.dtype == np.float32
    exact = _exact_logits(x64, w64).astype(np.float32)
    np.testing.assert_array_equal(got.view(np.uint32), exact.view(np.uint32))
    mm = (x64 @ w64.T).astype(np.float32)
    np.testing.assert_array_equal(got.view(np.uint32), mm.view(np.uint32))
    # the transposed reading or an fp32 accumulation would give other bits
    if H > 1:
        acc32 = np.zeros((T, E), np.float32)
        for h in range(H):
            acc32 = (acc32 + (x[:, h:h + 1] * w[:, h][None, :]).astype(np.float32)).astype(np.float32)
        if dtype == "f32":
            assert not np.array_equal(acc32.view(np.uint32), got.view(np.uint32))


def test_router_logits_one_hot_weights_expose_x():
    """W_r with one 1 per row selects a column of x: logits[t, e] = x[t, c_e] exactly."""
    rng = np.random.default_rng(3)
    T, H, E = 11, 40, 6
    x = rng.standard_normal((T, H)).astype(np.float32)
    cols = np.array([39, 0, 7, 7, 21, 2])
    w = np.zeros((E, H), np.float32)
    w[np.arange(E), cols] = 1.0
    np.testing.assert_array_equal(oracle.router_logits(x, w), x[:, cols])


@pytest.mark.parametrize("name", ["qwen3_bf16", "dsv3_bf16"])
def test_routing_margin_bounds_flips_under_perturbation(name):
    """The tie margin the GPU-router tests use (helpers.routing_margin): perturbing the
    oracle's logits by ~2e-5 relative changes the expert set of some tokens, and only of
    tokens whose margin is tiny; every margin is >= 0 (the oracle's selection is a true
    top-k)."""
    import moe_inputs as mi
    from helpers import routing_margin
    cfg = mi.scaled(mi.CONFIGS[name], T=3000, H=256)
    rng = np.random.default_rng(17)
    lg = (rng.standard_normal((cfg.T, cfg.E)) * 1.3).astype(np.float32)
    sb = (rng.standard_normal(cfg.E) * 0.01).astype(np.float32) if cfg.router else None
    idx, _ = oracle.route_cfg(cfg, lg, None, sb)
    m = routing_margin(cfg, lg, None, sb)
    assert np.all(m >= 0)
    pert = (lg * (1 + 2e-5 * rng.standard_normal(lg.shape))).astype(np.float32)
    idx2, _ = oracle.route_cfg(cfg, pert, None, sb)
    flipped = ~np.all(np.sort(idx, 1) == np.sort(idx2, 1), axis=1)
    assert flipped.any()
    assert np.all(m[flipped] <= 1e-4)
    # margins spread far above the bound for most tokens
    assert np.median(m) > 1e-3

"""Pins of the oracle's whole-layer backward (oracle.layer_backward): against torch.autograd
of an independently written float64 forward (per token, per selected expert, shared expert,
gates from the selected logits), and against central finite differences. The expert
selection is held fixed (it carries no gradient)."""
import numpy as np
import pytest
import torch

import oracle


def torch_forward(x, wr, w13, w2, ws13, ws2, idx, router, scale, lb):
    """y [T, H] by the per-token loop: gates from the selected logits, y = sum_j g_j W2 h."""
    l = x @ wr.T + lb[None, :]
    sel = l.gather(1, idx)
    if router == oracle.SOFTMAX_TOPK:
        g = torch.softmax(sel, dim=1)
    else:
        s = torch.sigmoid(sel)
        g = scale * s / s.sum(dim=1, keepdim=True)
    F = w13.shape[1] // 2
    rows = []
    for t in range(x.shape[0]):
        yt = torch.zeros(x.shape[1], dtype=x.dtype)
        for j in range(idx.shape[1]):
            e = int(idx[t, j])
            h = torch.nn.functional.silu(w13[e, :F] @ x[t]) * (w13[e, F:] @ x[t])
            yt = yt + g[t, j] * (w2[e] @ h)
        if ws13 is not None:
            Fs = ws13.shape[0] // 2
            yt = yt + ws2 @ (torch.nn.functional.silu(ws13[:Fs] @ x[t]) * (ws13[Fs:] @ x[t]))
        rows.append(yt)
    return torch.stack(rows), l, g


def case(seed, router, shared, T=7, H=8, E=5, k=2, F=3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    wr = rng.standard_normal((E, H)) * 0.5
    w13 = rng.standard_normal((E, 2 * F, H)) * 0.5
    w2 = rng.standard_normal((E, H, F)) * 0.5
    ws13 = rng.standard_normal((2 * F, H)) * 0.5 if shared else None
    ws2 = rng.standard_normal((H, F)) * 0.5 if shared else None
    lb = rng.standard_normal(E) * 0.3
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int64)
    dy = rng.standard_normal((T, H))
    return dict(x=x, wr=wr, w13=w13, w2=w2, ws13=ws13, ws2=ws2, lb=lb, idx=idx, dy=dy,
                router=router, scale=2.5 if router else 1.0)


@pytest.mark.parametrize("router", [oracle.SOFTMAX_TOPK, oracle.SIGMOID_GROUP_TOPK])
@pytest.mark.parametrize("shared", [False, True])
def test_layer_backward_matches_autograd(router, shared):
    c = case(1 + router + 2 * shared, router, shared)
    tt = {n: (None if c[n] is None else torch.tensor(c[n], requires_grad=True))
          for n in ("x", "wr", "w13", "w2", "ws13", "ws2")}
    y, l, g = torch_forward(tt["x"], tt["wr"], tt["w13"], tt["w2"], tt["ws13"], tt["ws2"],
                            torch.tensor(c["idx"]), router, c["scale"], torch.tensor(c["lb"]))
    l.retain_grad()
    g.retain_grad()
    (y * torch.tensor(c["dy"])).sum().backward()
    logits = c["x"] @ c["wr"].T
    got = oracle.layer_backward(c["x"], c["wr"], logits, c["idx"], c["w13"], c["w2"], c["dy"],
                                router, c["scale"], c["lb"], c["ws13"], c["ws2"])
    pairs = [("dx", tt["x"].grad), ("dw_router", tt["wr"].grad), ("dw13", tt["w13"].grad),
             ("dw2", tt["w2"].grad), ("dlogits", l.grad), ("dgate", g.grad)]
    if shared:
        pairs += [("dws13", tt["ws13"].grad), ("dws2", tt["ws2"].grad)]
    for name, ref in pairs:
        np.testing.assert_allclose(got[name], ref.numpy(), rtol=1e-10, atol=1e-12,
                                   err_msg=name)


@pytest.mark.parametrize("router", [oracle.SOFTMAX_TOPK, oracle.SIGMOID_GROUP_TOPK])
def test_layer_backward_finite_differences(router):
    """dL/dW_r[e, h] and dL/dx[t, h] by central differences of L = sum(y * dy)."""
    c = case(11 + router, router, True)

    def loss(x, wr):
        with torch.no_grad():
            y, _, _ = torch_forward(*(torch.tensor(v) if v is not None else None for v in
                                      (x, wr, c["w13"], c["w2"], c["ws13"], c["ws2"])),
                                    torch.tensor(c["idx"]), router, c["scale"],
                                    torch.tensor(c["lb"]))
        return float((y.numpy() * c["dy"]).sum())

    got = oracle.layer_backward(c["x"], c["wr"], c["x"] @ c["wr"].T, c["idx"], c["w13"],
                                c["w2"], c["dy"], router, c["scale"], c["lb"], c["ws13"],
                                c["ws2"])
    eps = 1e-6
    for (e, h) in [(0, 0), (2, 5), (4, 7)]:
        wp, wm = c["wr"].copy(), c["wr"].copy()
        wp[e, h] += eps
        wm[e, h] -= eps
        fd = (loss(c["x"], wp) - loss(c["x"], wm)) / (2 * eps)
        assert abs(fd - got["dw_router"][e, h]) <= 1e-6 * max(1.0, abs(fd))
    for (t, h) in [(0, 1), (3, 4), (6, 7)]:
        xp, xm = c["x"].copy(), c["x"].copy()
        xp[t, h] += eps
        xm[t, h] -= eps
        fd = (loss(xp, c["wr"]) - loss(xm, c["wr"])) / (2 * eps)
        assert abs(fd - got["dx"][t, h]) <= 1e-6 * max(1.0, abs(fd))

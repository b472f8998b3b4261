"""Pins of the oracle's expert MLP, fold, shared expert, fp8 simulation and backward:
a dense every-expert computation masked by the routing matrix (numpy / torch fp64
matmuls), special cases that reduce to a plain SwiGLU MLP, the fold identity, and
torch.autograd for the gradients."""
import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import oracle


def make(T, H, E, k, F, seed, dtype=torch.float32, shared_F=0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, H, generator=g).to(dtype)
    w13 = (torch.randn(E, 2 * F, H, generator=g) * 0.1).to(dtype)
    w2 = (torch.randn(E, H, F, generator=g) * 0.1).to(dtype)
    lg = torch.randn(T, E, generator=g).numpy()
    idx, gate = oracle.route(lg, k)
    ws13 = ws2 = None
    if shared_F:
        ws13 = (torch.randn(2 * shared_F, H, generator=g) * 0.1).to(dtype)
        ws2 = (torch.randn(H, shared_F, generator=g) * 0.1).to(dtype)
    return x, w13, w2, idx, gate, ws13, ws2


def swiglu_torch(x, w13, w2):
    """Plain SwiGLU MLP in fp64 with torch's silu."""
    F = w13.shape[0] // 2
    z = x @ w13.T
    return (Fn.silu(z[:, :F]) * z[:, F:]) @ w2.T


def dense_masked(x, w13, w2, idx, gate, ws13=None, ws2=None):
    """Every expert on every token, then weighted by the one-hot routing matrix."""
    x = x.double()
    T, E = x.shape[0], w13.shape[0]
    M = torch.zeros(T, E, dtype=torch.float64)
    M.scatter_(1, torch.from_numpy(idx).long(), torch.from_numpy(gate).double())
    all_e = torch.stack([swiglu_torch(x, w13[e].double(), w2[e].double()) for e in range(E)], 1)
    y = (M[:, :, None] * all_e).sum(1)
    if ws13 is not None:
        y = y + swiglu_torch(x, ws13.double(), ws2.double())
    return y.numpy()


def rel(a, b):
    return np.max(np.abs(a - b)) / np.max(np.abs(b))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("T,H,E,k,F,sF", [(40, 64, 8, 2, 32, 0), (33, 32, 16, 4, 48, 24),
                                          (12, 16, 4, 4, 8, 0)])
def test_layer_equals_dense_masked(T, H, E, k, F, sF, dtype):
    x, w13, w2, idx, gate, ws13, ws2 = make(T, H, E, k, F, seed=T + H, dtype=dtype, shared_F=sF)
    y = oracle.layer_tokens(x, idx, gate, w13, w2, np.arange(T), ws13, ws2)
    ref = dense_masked(x, w13, w2, idx, gate, ws13, ws2)
    assert rel(y, ref) < 1e-12


def test_fold_equals_unfolded():
    x, w13, w2, idx, gate, ws13, ws2 = make(50, 64, 8, 3, 40, seed=2, shared_F=16)
    a = oracle.layer_tokens(x, idx, gate, w13, w2, np.arange(50), ws13, ws2, fold=True)
    b = oracle.layer_tokens(x, idx, gate, w13, w2, np.arange(50), ws13, ws2, fold=False)
    assert rel(a, b) < 1e-12


def test_single_expert_is_plain_swiglu():
    x, w13, w2, _, _, _, _ = make(20, 32, 1, 1, 24, seed=3)
    idx = np.zeros((20, 1), np.int32)
    idx_, gate = oracle.route(np.zeros((20, 1), np.float32), 1)
    np.testing.assert_array_equal(idx_, idx)
    np.testing.assert_array_equal(gate, 1.0)
    y = oracle.layer_tokens(x, idx, gate, w13, w2, np.arange(20))
    ref = swiglu_torch(x.double(), w13[0].double(), w2[0].double()).numpy()
    assert rel(y, ref) < 1e-12


def test_identical_experts_scale_by_gate_sum():
    x, w13, w2, idx, gate, _, _ = make(30, 32, 6, 3, 16, seed=4)
    w13[:] = w13[0]
    w2[:] = w2[0]
    y = oracle.layer_tokens(x, idx, gate, w13, w2, np.arange(30))
    ref = swiglu_torch(x.double(), w13[0].double(), w2[0].double()).numpy()
    ref = ref * gate.astype(np.float64).sum(1, keepdims=True)
    assert rel(y, ref) < 1e-12


def test_expert_rows_expose_activation_and_match_layer():
    """W2 = identity makes y_perm equal the folded activation; the per-row outputs summed
    back per token give the layer output."""
    T, H, E, k, F = 24, 32, 4, 2, 32
    x, w13, w2, idx, gate, _, _ = make(T, H, E, k, F, seed=5)
    perm = oracle.permute(idx, gate, E)
    xp = oracle.gather_rows(x.numpy(), perm["pos"])
    rows = np.arange(T * k)
    eye = torch.eye(H).expand(E, H, F).contiguous()
    _, act, y = oracle.expert_rows(xp, perm["offsets"], perm["gate_perm"], w13, eye, rows)
    np.testing.assert_array_equal(act, y)
    # folded activation = gate * silu(z_g) * z_u (torch silu, fp64)
    e_of_row = np.searchsorted(perm["offsets"], rows, side="right") - 1
    xd = torch.from_numpy(xp).double()
    for r in range(T * k):
        z = w13[e_of_row[r]].double() @ xd[r]
        ref = perm["gate_perm"][r] * (Fn.silu(z[:F]) * z[F:])
        assert rel(act[r], ref.numpy()) < 1e-13
    _, _, yp = oracle.expert_rows(xp, perm["offsets"], perm["gate_perm"], w13, w2, rows)
    y_tok = oracle.layer_tokens(x, idx, gate, w13, w2, np.arange(T))
    summed = np.stack([sum(yp[perm["pos"][t, j]] for j in range(k)) for t in range(T)])
    assert rel(summed, y_tok) < 1e-12


# ------------------------------------------------------------------------------------
# fp8 simulation
# ------------------------------------------------------------------------------------

def torch_fake_quant_rows(v):
    """1 x 128 e4m3 round trip with torch's float8_e4m3fn cast (fp32 scale amax/448)."""
    v = v.float()
    R, Cc = v.shape
    b = v.reshape(R, Cc // 128, 128)
    amax = b.abs().amax(2, keepdim=True)
    s = torch.where(amax == 0, torch.ones_like(amax), amax / 448.0)
    q = (b / s).clamp(-448, 448).to(torch.float8_e4m3fn)
    return (q.double() * s.double()).reshape(R, Cc)


def torch_fake_quant_weight(w):
    w = w.float()
    R, Cc = w.shape
    b = w.reshape(R // 128, 128, Cc // 128, 128)
    amax = b.abs().amax((1, 3), keepdim=True)
    s = torch.where(amax == 0, torch.ones_like(amax), amax / 448.0)
    q = (b / s).clamp(-448, 448).to(torch.float8_e4m3fn)
    return (q.double() * s.double()).reshape(R, Cc)


def test_fp8_layer_equals_dense_torch_simulation():
    T, H, E, k, F, sF = 16, 256, 4, 2, 128, 128
    x, w13, w2, idx, gate, ws13, ws2 = make(T, H, E, k, F, seed=6, dtype=torch.bfloat16,
                                             shared_F=sF)
    q13, s13 = oracle.quant_weight(w13)
    q2, s2 = oracle.quant_weight(w2)
    qs13, ss13 = oracle.quant_weight(ws13)
    qs2, ss2 = oracle.quant_weight(ws2)
    y = oracle.layer_tokens(x, idx, gate, q13, q2, np.arange(T), qs13, qs2, fp8=True,
                            w13_scales=s13, w2_scales=s2, ws13_scales=ss13, ws2_scales=ss2)
    xq = torch_fake_quant_rows(x)
    ref = np.zeros((T, H))

    def expert(xrow, W13, W2, g):
        z = W13 @ xrow
        a = g * (Fn.silu(z[:W13.shape[0] // 2]) * z[W13.shape[0] // 2:])
        a = torch_fake_quant_rows(a.float()[None])[0]
        return W2 @ a
    Wq13 = [torch_fake_quant_weight(w13[e]) for e in range(E)]
    Wq2 = [torch_fake_quant_weight(w2[e]) for e in range(E)]
    Sq13, Sq2 = torch_fake_quant_weight(ws13), torch_fake_quant_weight(ws2)
    for t in range(T):
        acc = torch.zeros(H, dtype=torch.float64)
        for j in range(k):
            e = idx[t, j]
            acc += expert(xq[t], Wq13[e], Wq2[e], float(gate[t, j]))
        acc += expert(xq[t], Sq13, Sq2, 1.0)
        ref[t] = acc.numpy()
    assert rel(y, ref) < 1e-12


# ------------------------------------------------------------------------------------
# backward
# ------------------------------------------------------------------------------------

def test_backward_matches_autograd():
    """Data and weight gradients of the folded expert MLP vs torch.autograd (fp64)."""
    T, H, E, k, F = 20, 32, 4, 2, 16
    x, w13, w2, idx, gate, _, _ = make(T, H, E, k, F, seed=8, dtype=torch.bfloat16)
    perm = oracle.permute(idx, gate, E)
    A = T * k
    xp = torch.from_numpy(oracle.gather_rows(x.view(torch.int16).numpy(), perm["pos"])).view(torch.bfloat16)
    g = torch.Generator().manual_seed(9)
    dy = torch.randn(A, H, generator=g).to(torch.bfloat16)
    offs = perm["offsets"]
    gp = perm["gate_perm"]
    # saved forward tensors, rounded to bf16 as a bf16 forward would store them
    zs, acts = [], []
    for r in range(A):
        e = int(np.searchsorted(offs, r, side="right") - 1)
        z = (w13[e].double() @ xp[r].double())
        zs.append(z)
    z_saved = torch.stack(zs).to(torch.bfloat16)
    zz = z_saved.double()
    act_saved = (torch.from_numpy(gp).double()[:, None] * Fn.silu(zz[:, :F]) * zz[:, F:]).to(torch.bfloat16)

    # autograd reference on the same saved values
    X = xp.double().requires_grad_(True)
    G = torch.from_numpy(gp).double().requires_grad_(True)
    W13 = w13.double().requires_grad_(True)
    W2 = w2.double().requires_grad_(True)
    Zs = zz.clone().requires_grad_(True)
    loss = 0
    dzs = []
    for r in range(A):
        e = int(np.searchsorted(offs, r, side="right") - 1)
        Zr = Zs[r]
        a = G[r] * Fn.silu(Zr[:F]) * Zr[F:]
        yr = W2[e] @ a
        loss = loss + (dy[r].double() * yr).sum()
    loss.backward()
    dZ = Zs.grad                                            # [A, 2F]
    dx_ref = torch.stack([w13[int(np.searchsorted(offs, r, side='right') - 1)].double().T @ dZ[r]
                          for r in range(A)])
    dx, dg = oracle.expert_bwd_rows(dy, z_saved, offs, gp, w13, w2, np.arange(A))
    assert rel(dx, dx_ref.numpy()) < 1e-12
    assert rel(dg, G.grad.numpy()) < 1e-12

    # weight gradients: dW2_e = dy^T act, dW13_e = dz^T x_perm (autograd through a fresh graph)
    for e in range(E):
        r0, r1 = int(offs[e]), int(offs[e + 1])
        if r1 == r0:
            continue
        W13e = w13[e].double().requires_grad_(True)
        W2e = w2[e].double().requires_grad_(True)
        # forward with the saved z treated as a function of W13 through a straight-through
        # identity: z = W13 x + (z_saved - W13 x).detach()
        Xe = xp[r0:r1].double()
        Z = Xe @ W13e.T
        Z = Z + (zz[r0:r1] - Z).detach()
        Ae = act_saved[r0:r1].double()
        a_fn = torch.from_numpy(gp[r0:r1]).double()[:, None] * Fn.silu(Z[:, :F]) * Z[:, F:]
        a_use = a_fn + (Ae - a_fn).detach()
        Y = a_use @ W2e.T
        (dy[r0:r1].double() * Y).sum().backward()
        rr = np.array([0, 5, 2 * F - 1, F, 7], np.int32)
        cc = np.array([0, H - 1, 3, 17, 9], np.int32)
        r2 = np.array([0, H - 1, 4, 11], np.int32)
        c2 = np.array([0, F - 1, 5, 2], np.int32)
        dw13, dw2 = oracle.expert_wgrad_entries(dy, z_saved, act_saved, xp, offs, e, gp, w2,
                                                (rr, cc), (r2, c2))
        np.testing.assert_allclose(dw13, W13e.grad.numpy()[rr, cc], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dw2, W2e.grad.numpy()[r2, c2], rtol=1e-11, atol=1e-12)


def test_backward_finite_differences():
    """dx and dg of the data-gradient path against central differences of the oracle's
    own forward (fp32 inputs; the actual perturbation is measured in fp64)."""
    H, F = 16, 8
    g = torch.Generator().manual_seed(10)
    w13 = (torch.randn(1, 2 * F, H, generator=g) * 0.3)
    w2 = (torch.randn(1, H, F, generator=g) * 0.3)
    x = torch.randn(1, H, generator=g)
    dy = torch.randn(1, H, generator=g)
    gate = np.array([0.7], np.float32)
    offs = np.array([0, 1], np.int32)
    z = torch.from_numpy((w13[0].double() @ x[0].double()).float().numpy()[None])

    def loss(xv, gv):
        zz, act, y = oracle.expert_rows(xv.numpy(), offs, np.array([gv], np.float32), w13, w2, [0],
                                        want_z=True)
        return float((dy.double().numpy() * y).sum())
    dx, dg = oracle.expert_bwd_rows(dy, z, offs, gate, w13, w2, [0])
    # the backward reads z rounded to fp32; compare with a forward that computes z exactly, so
    # use a loose tolerance that still catches a dropped term or a sign error
    for h in range(H):
        xp_, xm_ = x.clone(), x.clone()
        xp_[0, h] += 1e-2
        xm_[0, h] -= 1e-2
        d = float(xp_[0, h]) - float(xm_[0, h])
        fd = (loss(xp_, gate[0]) - loss(xm_, gate[0])) / d
        assert abs(fd - dx[0, h]) < 2e-4 * (1 + abs(fd))
    gp_, gm_ = np.float32(0.7 + 1e-3), np.float32(0.7 - 1e-3)
    fd = (loss(x, gp_) - loss(x, gm_)) / (float(gp_) - float(gm_))
    assert abs(fd - dg[0]) < 1e-5 * (1 + abs(fd))

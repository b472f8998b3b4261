"""Pins of the oracle's MXFP8 quantiser (oracle.mx_quant): a brute-force restatement of the
OCP Microscaling rule (shared exponent from frexp, nearest E4M3 value by scanning the code
table, ties to the even code, saturation at 448) on blocks with edge cases, and the
defining property that a block's largest magnitude scales into [256, 512)."""
import math

import numpy as np
import torch

import oracle

MAG = oracle.e4m3_decode_array(np.arange(127, dtype=np.uint8))   # codes 0..126, increasing


def brute_code(v):
    a = abs(v)
    if a >= 448.0:
        c = 126
    else:
        d = np.abs(MAG - a)
        best = np.flatnonzero(d == d.min())
        c = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
    return (0x80 if math.copysign(1.0, v) < 0 else 0) | c


def brute_block(vals):
    amax = max(abs(v) for v in vals)
    if amax == 0.0:
        X = -127
    else:
        X = min(127, max(-127, math.frexp(amax)[1] - 1 - 8))
    return [brute_code(math.ldexp(v, -X)) for v in vals], X + 127


def test_mx_quant_matches_brute_force():
    rng = np.random.default_rng(3)
    blocks = [rng.standard_normal(32) * 10.0 ** rng.integers(-6, 4) for _ in range(40)]
    blocks.append(np.zeros(32))
    edge = np.zeros(32)
    edge[:6] = [448.0, -2.0 ** 9 * 1.75, 2.0 ** -20, 3.0, -0.0, 2.0 ** 8]
    blocks.append(edge)
    ties = (MAG[1:40] + MAG[:39]) / 2.0          # midpoints between neighbouring codes
    blocks.append(np.concatenate([ties[:31], [256.0]]))
    x = torch.tensor(np.stack(blocks), dtype=torch.float32)
    q, s = oracle.mx_quant(x)
    for i, b in enumerate(x.numpy().astype(np.float64)):
        codes, sc = brute_block(list(b))
        assert int(s[i, 0]) == sc, i
        assert list(q[i]) == codes, i


def test_mx_block_maximum_scales_into_256_512():
    rng = np.random.default_rng(4)
    x = torch.from_numpy((rng.standard_normal((64, 256)) * 3.0).astype(np.float32)).to(
        torch.bfloat16)
    q, s = oracle.mx_quant(x)
    a = np.abs(x.double().numpy()).reshape(64, 8, 32).max(axis=2)
    scaled = a * np.exp2(-(s.astype(np.float64) - 127.0))
    assert np.all((scaled >= 256.0) & (scaled < 512.0))
    d = oracle.mx_dequant(q, s)
    # away from saturation, each value is within half a code step of its e4m3 rounding
    err = np.abs(d - x.double().numpy())
    sc = np.repeat(np.exp2(s.astype(np.float64) - 127.0), 32, axis=1)
    ok = np.abs(x.double().numpy()) / sc < 464.0     # 464: halfway past 448, where it saturates
    assert np.all(err[ok] <= 16.0 * sc[ok])          # half of the largest step (32) below 512
    assert np.all(np.abs(d[~ok]) == 448.0 * sc[~ok])


# ------------------------------------------------------------------------------------
# MXFP8 expert layer: the oracle's layer (fp8="mx") against a torch simulation written
# independently of it (frexp for the shared exponent, torch's float8_e4m3fn cast for the
# element rounding, fp64 matmuls)
# ------------------------------------------------------------------------------------

def torch_fake_mx(v):
    """MXFP8 quantise-dequantise along the last axis, 32 values per block (float64 out)."""
    v = v.double()
    b = v.reshape(*v.shape[:-1], v.shape[-1] // 32, 32)
    amax = b.abs().amax(-1, keepdim=True)
    _, e = torch.frexp(amax)
    X = torch.where(amax > 0, e - 1 - 8, torch.full_like(e, -127)).clamp(-127, 127).double()
    scaled = (b * torch.exp2(-X)).float().clamp(-448.0, 448.0)
    q = scaled.to(torch.float8_e4m3fn).double()
    return (q * torch.exp2(X)).reshape(v.shape)


def _make(T, H, E, k, F, sF, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    w13 = (torch.randn(E, 2 * F, H, generator=g) * 0.05).to(torch.bfloat16)
    w2 = (torch.randn(E, H, F, generator=g) * 0.05).to(torch.bfloat16)
    ws13 = (torch.randn(2 * sF, H, generator=g) * 0.05).to(torch.bfloat16)
    ws2 = (torch.randn(H, sF, generator=g) * 0.05).to(torch.bfloat16)
    idx, gate = oracle.route(torch.randn(T, E, generator=g).numpy(), k)
    return x, w13, w2, ws13, ws2, idx, gate


def test_mx_layer_equals_torch_simulation():
    T, H, E, k, F, sF = 12, 256, 4, 2, 96, 64
    x, w13, w2, ws13, ws2, idx, gate = _make(T, H, E, k, F, sF, seed=21)
    q13, s13 = oracle.mx_quant(w13)
    q2, s2 = oracle.mx_quant(w2)
    qs13, ss13 = oracle.mx_quant(ws13)
    qs2, ss2 = oracle.mx_quant(ws2)
    y = oracle.layer_tokens(x, idx, gate, q13, q2, np.arange(T), qs13, qs2, fp8="mx",
                            w13_scales=s13, w2_scales=s2, ws13_scales=ss13, ws2_scales=ss2)

    def expert(xrow, W13, W2, gt):
        z = W13 @ xrow
        a = gt * (torch.nn.functional.silu(z[:W13.shape[0] // 2]) * z[W13.shape[0] // 2:])
        return W2 @ torch_fake_mx(a.float())
    xq = torch_fake_mx(x.float())
    W13 = [torch_fake_mx(w13[e].float()) for e in range(E)]
    W2 = [torch_fake_mx(w2[e].float()) for e in range(E)]
    S13, S2 = torch_fake_mx(ws13.float()), torch_fake_mx(ws2.float())
    ref = np.zeros((T, H))
    for t in range(T):
        acc = expert(xq[t], S13, S2, 1.0)
        for j in range(k):
            acc = acc + expert(xq[t], W13[idx[t, j]], W2[idx[t, j]], float(gate[t, j]))
        ref[t] = acc.numpy()
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_mx_expert_rows_read_codes_and_scales_per_32_block():
    """expert_rows on MX codes of x (E8M0 scales per 1 x 32 block) equals the per-row torch
    simulation, including the quantised activation it exposes."""
    T, H, E, k, F, sF = 10, 128, 3, 1, 64, 32
    x, w13, w2, _, _, _, _ = _make(T, H, E, k, F, sF, seed=22)
    xq, xs = oracle.mx_quant(x)
    q13, s13 = oracle.mx_quant(w13)
    q2, s2 = oracle.mx_quant(w2)
    offsets = np.array([0, 4, 4, T], np.int32)            # an empty middle expert
    gate = np.linspace(0.1, 1.0, T).astype(np.float32)
    _, act, yp = oracle.expert_rows(xq, offsets, gate, q13, q2, np.arange(T), x_scales=xs,
                                    w13_scales=s13, w2_scales=s2, quant_act=True, mx=True)
    X = torch_fake_mx(x.float())
    for r in range(T):
        e = 0 if r < 4 else 2
        z = torch_fake_mx(w13[e].float()) @ X[r]
        a = float(gate[r]) * (torch.nn.functional.silu(z[:F]) * z[F:])
        a = torch_fake_mx(a.float())
        assert np.max(np.abs(act[r] - a.numpy())) <= 1e-12 * max(1e-30, a.abs().max().item())
        yr = torch_fake_mx(w2[e].float()) @ a
        assert np.max(np.abs(yp[r] - yr.numpy())) <= 1e-12 * yr.abs().max().item()

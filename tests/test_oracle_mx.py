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

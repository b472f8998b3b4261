"""Pins of the oracle's e4m3 arithmetic against the OCP FP8 specification and torch's
float8_e4m3fn cast (an independent library implementation of the same format)."""
import numpy as np
import pytest
import torch

import oracle


def torch_e4m3_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_all_codes_decode_like_torch():
    ref = torch_e4m3_decode_all()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}       # S.1111.111 is NaN, no infinities
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_spec_values():
    assert oracle.e4m3_value(0x7E) == 448.0               # largest finite
    assert oracle.e4m3_value(0x08) == 2.0 ** -6           # smallest normal
    assert oracle.e4m3_value(0x01) == 2.0 ** -9           # smallest subnormal
    assert oracle.e4m3_value(0x07) == 7 * 2.0 ** -9       # largest subnormal
    assert oracle.e4m3_value(0x38) == 1.0                 # exponent field 7 = bias
    assert oracle.e4m3_value(0xB8) == -1.0


def _grid():
    # every e4m3 value, every midpoint between neighbours, and points just either side
    mags = np.array([oracle.e4m3_value(c) for c in range(127)], dtype=np.float64)
    mids = (mags[:-1] + mags[1:]) / 2
    pts = np.concatenate([mags, mids])
    f32 = pts.astype(np.float32)
    up = np.nextafter(f32, np.float32(np.inf))
    dn = np.nextafter(f32, np.float32(0))
    rnd = np.random.default_rng(1).uniform(0, 463.0, 20000).astype(np.float32)
    g = np.concatenate([f32, up, dn, rnd])
    g = g[g < 464.0]
    return np.concatenate([g, -g])


def test_encode_matches_torch_in_range():
    g = _grid()
    ref = torch.from_numpy(g).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(v)) for v in g], dtype=np.uint8)
    bad = np.nonzero(ref != got)[0]
    assert bad.size == 0, [(g[i], ref[i], got[i]) for i in bad[:10]]


def test_encode_ties_to_even_and_saturates():
    # 2^-10 is halfway between 0 and the smallest subnormal: ties to the even code 0
    assert oracle.e4m3_encode(2.0 ** -10) == 0
    # 3 * 2^-10 is halfway between codes 1 and 2: even code 2
    assert oracle.e4m3_encode(3 * 2.0 ** -10) == 2
    # halfway between 1.0 (0x38) and 1.125 (0x39): even code 0x38
    assert oracle.e4m3_encode(1.0625) == 0x38
    # halfway between 1.125 (0x39) and 1.25 (0x3A): even code 0x3A
    assert oracle.e4m3_encode(1.1875) == 0x3A
    for v in (448.0, 464.0, 480.0, 1e6, 3.4e38):
        assert oracle.e4m3_encode(v) == 0x7E
        assert oracle.e4m3_encode(-v) == 0xFE
    assert oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(0.0) == 0x00


def _torch_quant_blocks(v32: torch.Tensor, s32: torch.Tensor):
    """torch reference of q = e4m3(fp32(v / s)) with the clamp to +-448 done first."""
    r = (v32 / s32).clamp(-448.0, 448.0)
    return r.to(torch.float8_e4m3fn).view(torch.uint8)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quant_rows_matches_definition(dtype):
    g = torch.Generator().manual_seed(3)
    v = (torch.randn(37, 384, generator=g) * torch.rand(37, 1, generator=g) * 50).to(dtype)
    v[5, 128:256] = 0.0                                  # all-zero block: scale 1
    v[6, 0] = 1e4                                        # an outlier dominates its block
    q, s = oracle.quant_rows(v)
    v32 = v.float().reshape(37, 3, 128)
    amax = v32.abs().amax(dim=2)
    s_ref = torch.where(amax == 0, torch.ones_like(amax), amax / 448.0)
    np.testing.assert_array_equal(s, s_ref.numpy())
    q_ref = _torch_quant_blocks(v32, s_ref[:, :, None]).reshape(37, 384).numpy()
    np.testing.assert_array_equal(q, q_ref)
    # the largest element of a block maps to +-448 (within one code)
    deq = oracle.e4m3_decode_array(q).reshape(37, 3, 128) * s[:, :, None]
    err = np.abs(deq - v32.double().numpy())
    # relative error of a normal e4m3 value is at most 2^-4; subnormals at most s * 2^-10
    bound = np.maximum(np.abs(v32.double().numpy()) * 2.0 ** -4, s[:, :, None] * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-12))


def test_quant_weight_matches_definition():
    g = torch.Generator().manual_seed(4)
    w = (torch.randn(2, 256, 384, generator=g) * 0.02).to(torch.bfloat16)
    q, s = oracle.quant_weight(w)
    assert q.shape == (2, 256, 384) and s.shape == (2, 2, 3)
    wb = w.float().reshape(2, 2, 128, 3, 128).permute(0, 1, 3, 2, 4)
    amax = wb.abs().amax(dim=(3, 4))
    s_ref = amax / 448.0
    np.testing.assert_array_equal(s, s_ref.numpy())
    q_ref = _torch_quant_blocks(wb, s_ref[:, :, :, None, None])
    q_ref = q_ref.permute(0, 1, 3, 2, 4).reshape(2, 256, 384).numpy()
    np.testing.assert_array_equal(q, q_ref)


def test_e4m3_rank_orders_codes_like_their_values():
    """The code-distance helper used for quantised tensors: sorting finite codes by rank
    sorts them by value, and neighbouring ranks are neighbouring representable values."""
    from helpers import e4m3_rank
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)   # no NaN
    vals = oracle.e4m3_decode_array(codes)
    r = e4m3_rank(codes)
    order = np.argsort(r, kind="stable")
    assert np.all(np.diff(vals[order]) >= 0)
    pos = codes[(codes & 0x80) == 0]
    assert np.all(np.diff(oracle.e4m3_decode_array(np.sort(pos))) > 0)


def test_e4m3_step_matches_the_code_table():
    """e4m3_step(v) is the gap between the two representable values around v."""
    from helpers import e4m3_step
    vals = np.sort(oracle.e4m3_decode_array(np.arange(0, 127, dtype=np.uint8)))
    gaps = np.diff(vals)
    np.testing.assert_array_equal(e4m3_step(vals[:-1]), gaps)

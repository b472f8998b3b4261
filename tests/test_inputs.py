"""The seeded input generator: deterministic, per-expert streams, bf16 by round-to-nearest-even."""
import numpy as np
import torch

import moe_inputs as mi


def test_deterministic_and_per_expert_streams():
    cfg = mi.CONFIGS["tiny_fp32"]
    a = mi.make_inputs(cfg)
    b = mi.make_inputs(cfg, threads=1)
    for n in ("x", "w_router", "w13", "w2"):
        assert torch.equal(getattr(a, n), getattr(b, n))
    # one expert can be regenerated alone (its own seeded stream)
    e3 = mi._normal_torch(cfg.cfg_id, mi.TAG_W13, 3, (2 * cfg.F, cfg.H), 0.02)
    assert torch.equal(a.w13[3], e3)
    assert not torch.equal(a.w13[3], a.w13[4])
    # bf16 storage of a weight is the round-to-nearest-even of the same fp32 draw
    c = mi.CONFIGS["qwen3_bf16"].replace(T=8, H=256, E=4, k=2, F=128)
    w = mi.make_inputs(c).w13
    assert torch.equal(w[2], mi._normal_torch(c.cfg_id, mi.TAG_W13, 2, (2 * c.F, c.H), 0.02).to(torch.bfloat16))
    assert a.x.dtype == torch.float32 and a.x.shape == (256, 128)


def test_distributions():
    cfg = mi.CONFIGS["tiny_fp32"]
    a = mi.make_inputs(cfg)
    assert abs(float(a.x.std()) - 1.0) < 0.02
    assert abs(float(a.w13.std()) - 0.02) < 0.001


def test_bf16_is_round_to_nearest_even():
    v = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -1.0 - 2 ** -8],
                 np.float32)
    got = mi._to_storage(v, mi.BF16).float().numpy()
    np.testing.assert_array_equal(got, [1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -1.0])


def test_sigmoid_config_has_selection_bias():
    cfg = mi.CONFIGS["dsv3_bf16"].replace(T=16, H=128, F=128)
    a = mi.make_inputs(cfg, weights=False)
    assert a.sel_bias.shape == (256,) and a.sel_bias.dtype == torch.float32
    assert a.logit_bias is None


def test_zipf_bias_shape():
    cfg = mi.CONFIGS["dsv3_fp8_skew"]
    b = mi.zipf_logit_bias(cfg, c=0.5)
    assert b.shape == (256,)
    # the bias is c * ln(E p_r): one expert per rank, hottest rank 1
    p = np.arange(1, 257, dtype=np.float64) ** -1.2
    p /= p.sum()
    np.testing.assert_allclose(np.sort(b)[::-1], (0.5 * np.log(256 * p)).astype(np.float32), rtol=1e-6)

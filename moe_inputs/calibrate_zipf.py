"""Calibrate the strength c of the Zipf-shaped logit bias of the skewed DeepSeek-V3-shaped
workload and record it in moe_inputs/zipf_scale.json.

Offline test-infrastructure script (not imported by the moe_inputs package): it routes the
seeded inputs with the CPU oracle (router logits, then the sigmoid + group-limited top-k
with bias[e] = c * ln(E * p_pi(e)) added to the logits) and bisects on c until the hottest
expert receives between 9.5x and 10.5x the mean number of token copies (T * k / E).

    python moe_inputs/calibrate_zipf.py [workload]
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import moe_inputs as mi  # noqa: E402
import oracle  # noqa: E402


def load_stats(cfg, logits, c, sel_bias):
    lb = mi.zipf_logit_bias(cfg, c)
    idx, _ = oracle.route_cfg(cfg, logits, lb, sel_bias)
    counts = np.bincount(idx.ravel(), minlength=cfg.E)
    mean = cfg.T * cfg.k / cfg.E
    return counts.max() / mean, counts


def main(name="dsv3_fp8_skew"):
    cfg = mi.CONFIGS[name]
    inp = mi.make_inputs(cfg, weights=False, zipf_c=0.0)
    print(f"[zipf] oracle router logits for {name} (T={cfg.T}, H={cfg.H}, E={cfg.E}) ...",
          flush=True)
    logits = oracle.router_logits(inp.x, inp.w_router)
    sb = None if inp.sel_bias is None else inp.sel_bias.numpy()
    lo, hi = 0.0, 2.0
    ratio_hi, _ = load_stats(cfg, logits, hi, sb)
    assert ratio_hi > 10.5, ratio_hi
    c = None
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        r, counts = load_stats(cfg, logits, mid, sb)
        print(f"[zipf] c={mid:.6f} max/mean={r:.3f}", flush=True)
        if 9.5 <= r <= 10.5 and abs(r - 10.0) < 0.25:
            c = mid
            break
        if r < 10.0:
            lo = mid
        else:
            hi = mid
    assert c is not None
    r, counts = load_stats(cfg, logits, c, sb)
    mean = cfg.T * cfg.k / cfg.E
    rec = {"c": round(c, 6), "max_over_mean": round(float(r), 4),
           "min_rows": int(counts.min()), "median_rows": float(np.median(counts)),
           "max_rows": int(counts.max()), "mean_rows": mean,
           "method": "bisection on the oracle's routing of the seeded inputs; target hottest "
                     "expert 9.5x..10.5x the mean load"}
    path = mi.zipf_scale_path()
    data = {}
    if os.path.exists(path):
        with open(path) as f:
            data = json.load(f)
    data[name] = rec
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(f"[zipf] recorded {rec} in {path}", flush=True)


if __name__ == "__main__":
    main(*sys.argv[1:])

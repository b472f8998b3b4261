"""Seeded synthetic inputs for the MoE-layer forward, shared by the GPU path's tests and
bench and by the CPU oracle.

This module holds no step of the method: it only draws random numbers and rounds them
to the storage type (fp32 -> bf16 by round-to-nearest-even, done by torch's cast).
Nothing here routes, permutes, multiplies or quantises.

Every tensor comes from its own seeded stream, keyed by
SeedSequence([BASE_SEED, config id, tensor tag, expert]): numpy PCG64 for x, the router
weight and the biases; for the expert weights (the bulk of the bytes) a torch CPU generator
seeded with that key's 63-bit state, one stream per expert, so a single expert can be
regenerated alone and generation can run in threads.

Layouts (row-major, K contiguous for both GEMM operands):
  x        [T, H]          activations, N(0, 1)
  w_router [E, H]          router weight, N(0, 0.02), in the activation dtype
  sel_bias [E]   fp32      sigmoid-router selection bias, N(0, 0.01) (sigmoid configs)
  w13      [E, 2F, H]      rows 0..F-1 gate projection, rows F..2F-1 up projection
  w2       [E, H, F]       down projection
  ws13     [2F_s, H], ws2 [H, F_s]   shared expert (configs that have one)
  dy       [T, H]          upstream gradient, N(0, 1) (backward config)
"""
from __future__ import annotations

import json
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, asdict

import numpy as np
import torch

BASE_SEED = 20261202

TAG_X, TAG_WR, TAG_SELB, TAG_W13, TAG_W2, TAG_WS13, TAG_WS2, TAG_DY, TAG_ZIPF = range(9)

F32, BF16, E4M3, MXFP8 = 0, 1, 2, 3   # dtype codes shared with the C interfaces
SOFTMAX_TOPK, SIGMOID_GROUP_TOPK = 0, 1


@dataclass(frozen=True)
class MoEConfig:
    name: str
    cfg_id: int
    T: int
    H: int
    E: int
    k: int
    F: int
    router: int = SOFTMAX_TOPK
    n_groups: int = 1
    topk_groups: int = 1
    route_scale: float = 1.0
    act_dtype: int = BF16
    w_dtype: int = BF16
    shared_F: int = 0
    zipf_alpha: float = 0.0        # > 0: add a Zipf-shaped per-expert logit bias
    backward: bool = False
    a_layout: int = 0              # 0 row-major, 1 K-blocked (expert-grouped activations)
    w_layout: int = 0              # 0 row-major, 1 K-blocked (expert weights)
    capacity_factor: float = 0.0   # 0 dropless; > 0: expert capacity ceil(cf * T * k / E)

    def replace(self, **kw) -> "MoEConfig":
        d = asdict(self)
        d.update(kw)
        return MoEConfig(**d)

    @property
    def A(self) -> int:
        return self.T * self.k


# The five workloads: a tiny fp32 layer and layers shaped like Mixtral-8x7B,
# Qwen3-235B-A22B and DeepSeek-V3 (bf16, and fp8 with a skewed expert load); plus the
# DeepSeek-V3 bf16 layer with MXFP8 expert GEMMs (the same seed family, hence the same x,
# router and weights as the bf16 layer: only the expert GEMMs' number format differs).
CONFIGS = {
    "tiny_fp32": MoEConfig("tiny_fp32", 0, T=256, H=128, E=8, k=2, F=256,
                           act_dtype=F32, w_dtype=F32),
    "mixtral_bf16": MoEConfig("mixtral_bf16", 1, T=4096, H=4096, E=8, k=2, F=14336),
    "qwen3_bf16": MoEConfig("qwen3_bf16", 2, T=8192, H=4096, E=128, k=8, F=1536),
    "dsv3_bf16": MoEConfig("dsv3_bf16", 3, T=8192, H=7168, E=256, k=8, F=2048,
                           router=SIGMOID_GROUP_TOPK, n_groups=8, topk_groups=4,
                           route_scale=2.5, shared_F=2048),
    "dsv3_fp8_skew": MoEConfig("dsv3_fp8_skew", 4, T=8192, H=7168, E=256, k=8, F=2048,
                               router=SIGMOID_GROUP_TOPK, n_groups=8, topk_groups=4,
                               route_scale=2.5, shared_F=2048, w_dtype=E4M3,
                               zipf_alpha=1.2, backward=True),
    "dsv3_mxfp8": MoEConfig("dsv3_mxfp8", 3, T=8192, H=7168, E=256, k=8, F=2048,
                            router=SIGMOID_GROUP_TOPK, n_groups=8, topk_groups=4,
                            route_scale=2.5, shared_F=2048, w_dtype=MXFP8),
}


def _rng(cfg_id: int, tag: int, expert: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [BASE_SEED, cfg_id, tag, expert])))


def _normal(cfg_id: int, tag: int, expert: int, shape, sigma: float) -> np.ndarray:
    a = _rng(cfg_id, tag, expert).standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return a


def _torch_seed(cfg_id: int, tag: int, expert: int) -> int:
    st = np.random.SeedSequence([BASE_SEED, cfg_id, tag, expert]).generate_state(1, np.uint64)
    return int(st[0]) & ((1 << 63) - 1)


def _normal_torch(cfg_id: int, tag: int, expert: int, shape, sigma: float) -> torch.Tensor:
    g = torch.Generator().manual_seed(_torch_seed(cfg_id, tag, expert))
    a = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    if sigma != 1.0:
        a.mul_(sigma)
    return a


def _to_storage(a: np.ndarray, dtype: int) -> torch.Tensor:
    t = torch.from_numpy(a)
    if dtype == F32:
        return t
    # fp8 weights are produced from the bf16 weights by the quantiser under test.
    return t.to(torch.bfloat16)


def _stacked(cfg_id, tag, n, shape, sigma, dtype, threads) -> torch.Tensor:
    tdt = torch.float32 if dtype == F32 else torch.bfloat16
    out = torch.empty((n,) + tuple(shape), dtype=tdt)

    def one(e):
        out[e].copy_(_normal_torch(cfg_id, tag, e, shape, sigma))

    if n == 1 or threads <= 1:
        for e in range(n):
            one(e)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(n)))
    return out


def storage_dtype(cfg: MoEConfig) -> int:
    """Storage dtype of x and of the generated (pre-quantisation) weights."""
    return F32 if cfg.act_dtype == F32 else BF16


def zipf_scale_path() -> str:
    return os.path.join(os.path.dirname(__file__), "zipf_scale.json")


def zipf_logit_bias(cfg: MoEConfig, c: float | None = None) -> np.ndarray:
    """Per-expert logit bias shaping a Zipf(alpha) load: a seeded ranking pi of the experts,
    p_r proportional to r^-alpha, bias[e] = c * ln(E * p_{pi(e)}). The strength c is a
    recorded constant (calibrated once so the hottest expert gets about 10x the mean load)."""
    E = cfg.E
    if c is None:
        with open(zipf_scale_path()) as f:
            table = json.load(f)
        key = cfg.name if cfg.name in table else cfg.name.split("_small")[0]
        c = float(table[key]["c"])
    ranks = _rng(cfg.cfg_id, TAG_ZIPF).permutation(E) + 1          # rank of expert e, 1-based
    p = np.arange(1, E + 1, dtype=np.float64) ** (-cfg.zipf_alpha)
    p /= p.sum()
    return (c * np.log(E * p[ranks - 1])).astype(np.float32)


@dataclass
class MoEInputs:
    cfg: MoEConfig
    x: torch.Tensor
    w_router: torch.Tensor
    logit_bias: torch.Tensor | None
    sel_bias: torch.Tensor | None
    w13: torch.Tensor | None = None
    w2: torch.Tensor | None = None
    ws13: torch.Tensor | None = None
    ws2: torch.Tensor | None = None
    dy: torch.Tensor | None = None
    extra: dict = field(default_factory=dict)


def make_inputs(cfg: MoEConfig, weights: bool = True, threads: int | None = None,
                zipf_c: float | None = None) -> MoEInputs:
    """Generate the seeded inputs of `cfg` as CPU tensors (fp32 or bf16)."""
    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    sd = storage_dtype(cfg)
    x = _to_storage(_normal(cfg.cfg_id, TAG_X, 0, (cfg.T, cfg.H), 1.0), sd)
    wr = _to_storage(_normal(cfg.cfg_id, TAG_WR, 0, (cfg.E, cfg.H), 0.02), sd)
    sel_bias = None
    if cfg.router == SIGMOID_GROUP_TOPK:
        sel_bias = torch.from_numpy(_normal(cfg.cfg_id, TAG_SELB, 0, (cfg.E,), 0.01))
    logit_bias = None
    if cfg.zipf_alpha > 0:
        logit_bias = torch.from_numpy(zipf_logit_bias(cfg, zipf_c))
    inp = MoEInputs(cfg, x, wr, logit_bias, sel_bias)
    if weights:
        inp.w13 = _stacked(cfg.cfg_id, TAG_W13, cfg.E, (2 * cfg.F, cfg.H), 0.02, sd, threads)
        inp.w2 = _stacked(cfg.cfg_id, TAG_W2, cfg.E, (cfg.H, cfg.F), 0.02, sd, threads)
        if cfg.shared_F:
            inp.ws13 = _stacked(cfg.cfg_id, TAG_WS13, 1, (2 * cfg.shared_F, cfg.H), 0.02, sd, 1)[0]
            inp.ws2 = _stacked(cfg.cfg_id, TAG_WS2, 1, (cfg.H, cfg.shared_F), 0.02, sd, 1)[0]
    if cfg.backward:
        inp.dy = _to_storage(_normal(cfg.cfg_id, TAG_DY, 0, (cfg.T, cfg.H), 1.0), BF16)
    return inp


def scaled(cfg: MoEConfig, **kw) -> MoEConfig:
    """A smaller copy of a workload for element-by-element parity (same router, dtypes and
    structure, fewer tokens / narrower matrices). The config id is kept so that the
    distributions are drawn from the same family of streams."""
    return cfg.replace(name=cfg.name + "_small", **kw)


def raw_u16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 view of its bit patterns (no copy for contiguous CPU)."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)

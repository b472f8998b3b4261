"""Benchmark of the MoE-layer forward on one MI355X.

One step = one moe_layer_forward call over one batch of seeded synthetic inputs already
resident in HBM: router GEMM -> top-k routing -> permute -> grouped GEMM up (gate/up +
SwiGLU, gate folded) -> grouped GEMM down -> combine, for the routed experts and the shared
expert. The expert weights are stored in the library's K-blocked layout (moe_pack_kblock,
run once before timing, like loading a checkpoint); the step itself starts from x. The
default workload is the DeepSeek-V3-shaped bf16 layer (T=8192 tokens, hidden 7168, 256
routed experts in 8 groups, top-8, SwiGLU width 2048, one shared expert).

Prints progress to stderr and ONE JSON line to stdout.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--cpu-sample S] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12          # MI355X HBM3E, bytes/s
PEAK_MFMA = {"bf16": 2.5e15, "fp32": 157.3e12, "fp8": 5.0e15}   # dense, FLOP/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(cfg):
    """Algorithmic bytes / FLOPs of every step of the path, from the shapes alone."""
    T, H, E, k, F, sF = cfg.T, cfg.H, cfg.E, cfg.k, cfg.F, cfg.shared_F
    A = T * k
    b = 4 if cfg.act_dtype == 0 else 2
    wb = 1 if cfg.w_dtype == 2 else b
    d = {}
    d["router_logits"] = dict(bytes=T * H * b + E * H * b + T * E * 4, flops=2 * T * H * E)
    d["route"] = dict(bytes=T * E * 4 + 2 * A * 4, flops=0)
    # x read once, written k times; idx/gate read; pos/src/gate_perm written
    d["permute"] = dict(bytes=T * H * b + A * H * wb + 2 * A * 4 + 3 * A * 4, flops=0)
    up_b = E * 2 * F * H * wb + A * H * wb + A * F * wb + A * 4
    up_f = 2 * A * 2 * F * H
    dn_b = E * H * F * wb + A * F * wb + A * H * b
    dn_f = 2 * A * H * F
    if sF:
        up_b += 2 * sF * H * wb + T * H * wb + T * sF * wb
        up_f += 2 * T * 2 * sF * H
        dn_b += H * sF * wb + T * sF * wb + T * H * b
        dn_f += 2 * T * H * sF
    d["grouped_gemm_up"] = dict(bytes=up_b, flops=up_f)
    d["grouped_gemm_down"] = dict(bytes=dn_b, flops=dn_f)
    d["combine"] = dict(bytes=A * H * b + (T * H * b if sF else 0) + T * H * b + A * 4, flops=0)
    return d


def cpu_baseline(cfg, inp, sample: int):
    """The oracle, as it stands, end to end on `sample` seeded tokens of the same workload."""
    import numpy as np
    import oracle

    rng = np.random.default_rng(7)
    toks = np.sort(rng.choice(cfg.T, size=min(sample, cfg.T), replace=False))
    sub = cfg.replace(T=len(toks))
    xs = inp.x[toks]
    oracle.lib()
    t0 = time.perf_counter()
    logits = oracle.router_logits(xs, inp.w_router)
    lb = None if inp.logit_bias is None else inp.logit_bias.numpy()
    sb = None if inp.sel_bias is None else inp.sel_bias.numpy()
    idx, gate = oracle.route_cfg(sub, logits, lb, sb)
    oracle.permute(idx, gate, cfg.E)
    oracle.layer_tokens(xs, idx, gate, inp.w13, inp.w2, np.arange(len(toks)), inp.ws13, inp.ws2)
    dt = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": len(toks) / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(toks)} seeded tokens of the same workload, end to end (router "
                      f"logits, routing, permutation of the sub-batch, expert MLPs, shared "
                      f"expert) in {dt:.1f} s; tokens are independent, so tokens/s scales"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dsv3_bf16")
    ap.add_argument("--cpu-sample", type=int, default=1024)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--stage-reps", type=int, default=5)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (this build "
              "has no multi-GPU path; the expert-parallel design is described in DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_inputs as mi
    import routing_grouped_expert_softmax_amd as moe

    cfg = mi.CONFIGS[args.workload]
    if cfg.act_dtype != mi.F32:
        cfg = cfg.replace(a_layout=1, w_layout=1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log(f"[bench] generating {cfg.name} inputs ...")
    t0 = time.time()
    inp = mi.make_inputs(cfg)
    log(f"[bench] inputs generated in {time.time() - t0:.1f} s; copying to HBM")
    g = lambda t: None if t is None else t.to(dev, non_blocking=False)  # noqa: E731
    x, wr, w13, w2 = g(inp.x), g(inp.w_router), g(inp.w13), g(inp.w2)
    ws13, ws2, lb, sb = g(inp.ws13), g(inp.ws2), g(inp.logit_bias), g(inp.sel_bias)
    if cfg.w_layout:
        pk = lambda t: None if t is None else moe.pack_kblock(t)  # noqa: E731
        w13, w2, ws13, ws2 = pk(w13), pk(w2), pk(ws13), pk(ws2)
        torch.cuda.synchronize()
    y = torch.empty(cfg.T, cfg.H, dtype=moe.act_torch_dtype(cfg), device=dev)
    ws = moe.workspace(cfg, moe.OP_LAYER_FORWARD, dev)
    counts = torch.empty(cfg.E, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    def step():
        moe.layer_forward(cfg, x, wr, w13, w2, lb, sb, None, ws13=ws13, ws2=ws2, y=y, ws=ws)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = e0.elapsed_time(e1) / args.steps
    log(f"[bench] {ms:.3f} ms/step (wall {wall * 1e3 / args.steps:.3f} ms/step)")

    # ---- per-stage times: the same work as one step, one C-ABI call per stage, each
    # bracketed by events on the stream the library launches on
    A = cfg.T * cfg.k
    logits = torch.empty(cfg.T, cfg.E, dtype=torch.float32, device=dev)
    idx = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device=dev)
    gate = torch.empty(cfg.T, cfg.k, dtype=torch.float32, device=dev)
    pws = moe.workspace(cfg, moe.OP_PERMUTE, dev)
    gws = moe.workspace(cfg, moe.OP_GROUPED_GEMM, dev)
    gd, ad = moe.gemm_torch_dtype(cfg), moe.act_torch_dtype(cfg)
    act = torch.empty(A, cfg.F, dtype=gd, device=dev)
    y_perm = torch.empty(A, cfg.H, dtype=ad, device=dev)
    sh_act = torch.empty(cfg.T, cfg.shared_F, dtype=gd, device=dev) if cfg.shared_F else None
    sh_y = torch.empty(cfg.T, cfg.H, dtype=ad, device=dev) if cfg.shared_F else None
    perm = {}
    stages = {
        "router_logits": lambda: moe.router_logits(cfg, x, wr, logits),
        "route": lambda: moe.route(cfg, logits, lb, sb, idx, gate),
        "permute": lambda: perm.update(moe.permute(cfg, x, idx, gate, ws=pws)),
        "grouped_gemm_up": lambda: moe.grouped_gemm_up(
            cfg, perm["x_perm"], perm["offsets"], perm["gate_perm"], w13, act,
            x_shared=x if cfg.shared_F else None, ws13=ws13, shared_act=sh_act, ws=gws),
        "grouped_gemm_down": lambda: moe.grouped_gemm_down(
            cfg, act, perm["offsets"], w2, y_perm, shared_act=sh_act, ws2=ws2, shared_y=sh_y,
            ws=gws),
        "combine": lambda: moe.unpermute_combine(cfg, y_perm, perm["pos"], sh_y, y),
    }
    times = {k: 0.0 for k in stages}
    for rep in range(args.stage_reps + 1):
        for name, fn in stages.items():
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            if rep > 0:
                times[name] += a.elapsed_time(b) / args.stage_reps
    moe.layer_forward(cfg, x, wr, w13, w2, lb, sb, None, ws13=ws13, ws2=ws2, y=y, ws=ws,
                      want=("counts",))
    _, ex = moe.layer_forward(cfg, x, wr, w13, w2, lb, sb, None, ws13=ws13, ws2=ws2, y=y,
                              ws=ws, want=("counts",))
    cnt = ex["counts"].cpu().double()
    torch.cuda.synchronize()

    alg = algorithmic(cfg)
    dtype = {0: "fp32", 1: "bf16", 2: "fp8"}[cfg.w_dtype]
    per_stage = {}
    for name, t in times.items():
        s = t * 1e-3
        per_stage[name] = {"ms": round(t, 4),
                           "GB/s": round(alg[name]["bytes"] / s / 1e9, 1),
                           "TFLOP/s": round(alg[name]["flops"] / s / 1e12, 1)}
    # dominant kernel: the grouped GEMM up (gate/up projection + SwiGLU)
    dom = "grouped_gemm_up"
    t_dom = times[dom] * 1e-3
    t_hbm = alg[dom]["bytes"] / PEAK_HBM
    t_mfma = alg[dom]["flops"] / PEAK_MFMA[dtype]
    if t_hbm >= t_mfma:
        achieved, peak, unit = alg[dom]["bytes"] / t_dom / 1e9, PEAK_HBM / 1e9, "GB/s"
        bound = "hbm"
    else:
        achieved, peak, unit = alg[dom]["flops"] / t_dom / 1e12, PEAK_MFMA[dtype] / 1e12, "TFLOP/s"
        bound = "mfma"
    gemm_t = (times["grouped_gemm_up"] + times["grouped_gemm_down"]) * 1e-3
    gemm_flops = alg["grouped_gemm_up"]["flops"] + alg["grouped_gemm_down"]["flops"]

    result = {
        "metric": "MoE layer tokens/s; grouped-GEMM TFLOPS & % MFMA peak; permute GB/s",
        "value": round(cfg.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights)",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "E": cfg.E, "k": cfg.k,
                   "F": cfg.F, "shared_F": cfg.shared_F,
                   "router": "softmax_topk" if cfg.router == 0 else
                   f"sigmoid_group_topk(groups={cfg.n_groups},keep={cfg.topk_groups},"
                   f"scale={cfg.route_scale})",
                   "weights": "K-blocked" if cfg.w_layout else "row-major",
                   "parallelism": "single GPU"},
        "roofline": {"kernel": "grouped GEMM up (gate/up + SwiGLU, gate folded)",
                     "bound": bound, "achieved": round(achieved, 1), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": None},
        "grouped_gemm": {"TFLOP/s": round(gemm_flops / gemm_t / 1e12, 1),
                         "frac_mfma_peak": round(gemm_flops / gemm_t / PEAK_MFMA[dtype], 4)},
        "permute_GB/s": per_stage["permute"]["GB/s"],
        "stages": per_stage,
        "load": {"max_over_mean": round(float(cnt.max() / cnt.mean()), 3),
                 "min_over_mean": round(float(cnt.min() / cnt.mean()), 3)},
    }
    if not args.no_cpu:
        log(f"[bench] cpu baseline: oracle on {args.cpu_sample} tokens ...")
        result["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_sample)
        log(f"[bench] cpu baseline {result['cpu_baseline']['value']:.2f} tokens/s")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

"""Shared test helpers: the error metric and the small parity workloads."""
import numpy as np
import torch

import moe_inputs as mi

TOL = {mi.F32: 1e-5, mi.BF16: 2e-2, mi.E4M3: 6e-2, mi.MXFP8: 6e-2}


def rel_err(got, ref) -> float:
    """max_i |got_i - ref_i| / max_i |ref_i| over the whole checked tensor (fp64)."""
    g = got.detach().cpu().double().numpy() if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    r = ref.detach().cpu().double().numpy() if isinstance(ref, torch.Tensor) else np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    den = np.max(np.abs(r))
    return float(np.max(np.abs(g - r)) / (den if den > 0 else 1.0))


def tol(cfg) -> float:
    return TOL[cfg.w_dtype if cfg.w_dtype in (mi.E4M3, mi.MXFP8) else cfg.act_dtype]


# Small copies of each workload: same router, dtypes and structure, sizes the oracle finishes
# in seconds, several M and N tiles per GEMM and ragged per-expert tails.
SMALL = {
    "tiny_fp32": mi.CONFIGS["tiny_fp32"],
    "mixtral_small": mi.scaled(mi.CONFIGS["mixtral_bf16"], T=1000, H=512, F=512),
    "qwen3_small": mi.scaled(mi.CONFIGS["qwen3_bf16"], T=520, H=512, F=256),
    "dsv3_small": mi.scaled(mi.CONFIGS["dsv3_bf16"], T=520, H=512, F=256, shared_F=256),
    "dsv3_small_wide_shared": mi.scaled(mi.CONFIGS["dsv3_bf16"], T=300, H=256, F=128,
                                        shared_F=384),
}

# Small copies of the skewed e4m3 workload (same Zipf-biased router, e4m3 expert GEMMs).
SMALL_FP8 = {
    "dsv3_fp8_small": mi.scaled(mi.CONFIGS["dsv3_fp8_skew"], T=520, H=512, F=256,
                                shared_F=256),
    "dsv3_fp8_small_kblock": mi.scaled(mi.CONFIGS["dsv3_fp8_skew"], T=300, H=768, F=384,
                                       shared_F=128, a_layout=1, w_layout=1),
    # one token: one live row per GEMM tile, most experts empty
    "dsv3_fp8_one_token": mi.scaled(mi.CONFIGS["dsv3_fp8_skew"], T=1, H=256, F=128,
                                    shared_F=128),
}


# Small copies of the DeepSeek-V3 layer with MXFP8 expert GEMMs (1 x 32 E8M0 scales): several
# M and N tiles, ragged tails, a shared expert in the same launch (shared_F == F) and in a
# launch of its own, K of 2 to 6 stages, one token.
SMALL_MX = {
    "dsv3_mx_small": mi.scaled(mi.CONFIGS["dsv3_mxfp8"], T=520, H=512, F=256, shared_F=256),
    "dsv3_mx_wide": mi.scaled(mi.CONFIGS["dsv3_mxfp8"], T=300, H=768, F=384, shared_F=128),
    # 16 experts: 300+ rows per expert, i.e. two M tiles of 256 with a ragged second one
    "dsv3_mx_deep": mi.scaled(mi.CONFIGS["dsv3_mxfp8"], T=1500, H=256, F=128, E=16, k=4,
                              n_groups=4, topk_groups=2, shared_F=128),
    "dsv3_mx_one_token": mi.scaled(mi.CONFIGS["dsv3_mxfp8"], T=1, H=256, F=128, shared_F=128),
    # K-blocked weight codes (scales row-major)
    "dsv3_mx_wkblock": mi.scaled(mi.CONFIGS["dsv3_mxfp8"], T=300, H=512, F=256, shared_F=256,
                                 w_layout=1),
}


def to_dev(t):
    return None if t is None else t.cuda()


def sample_rows(offsets, extra_per_group=1, seed=0):
    """First, last and a random row of every non-empty group."""
    rng = np.random.default_rng(seed)
    rows = []
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            rows += [a, b - 1] + list(rng.integers(a, b, extra_per_group))
    return np.unique(np.array(rows, np.int64))


def unblock(t, rows: int, cols: int):
    """K-blocked [rows, cols] tensor -> row-major copy (torch, any device): the inverse of
    the layout [cols * eb / 64][rows][64 bytes], written with plain reshapes."""
    eb = t.element_size()
    b = t.contiguous().view(torch.uint8).reshape(-1)
    n = b.numel() // (rows * cols * eb)
    b = b.reshape(n, cols * eb // 64, rows, 64).permute(0, 2, 1, 3).reshape(n, rows, cols * eb)
    out = b.contiguous().view(t.dtype).reshape(n, rows, cols)
    return out[0] if t.dim() == 2 else out


def block(t):
    """Row-major [.., rows, cols] tensor -> K-blocked copy (the forward re-layout, reshapes)."""
    eb = t.element_size()
    rows, cols = t.shape[-2], t.shape[-1]
    b = t.contiguous().view(torch.uint8).reshape(-1, rows, cols * eb // 64, 64)
    b = b.permute(0, 2, 1, 3).contiguous().reshape(-1)
    return b.view(t.dtype).reshape(t.shape)


def e4m3_rank(q):
    """Signed position of an e4m3 code on the number line (codes are sign-magnitude)."""
    q = np.asarray(q).astype(np.int32)
    mag = q & 0x7F
    return np.where(q & 0x80, -mag, mag)


def e4m3_step(v):
    """Spacing of e4m3 values at |v| (v in units of the block scale): 2^(e - 3) for normal
    values (2^-6 <= |v| < 448, e = floor(log2 |v|)), 2^-9 below."""
    a = np.minimum(np.abs(np.asarray(v, np.float64)), 448.0)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (e - 3))


def e4m3_codes_close(q_gpu, s_gpu, act_ref_f64, err=1e-3):
    """Compare quantised rows (codes + 1 x 128 scales) with the oracle's unquantised
    activation act_ref. The GPU quantises its own fp32 value, which differs from the
    oracle's by accumulation rounding, so each dequantised element must lie within one e4m3
    step of act_ref (the quantisation error) plus err of the block's scale range (the
    propagated rounding). Returns (max |error| / bound, fraction of codes differing from the
    oracle's own quantisation, max scale rel diff)."""
    import oracle
    ref32 = np.asarray(act_ref_f64, np.float64).astype(np.float32)
    q_ref, s_ref = oracle.quant_rows(ref32)
    s_ref_e = np.repeat(np.asarray(s_ref, np.float64), 128, axis=1)
    s_gpu_e = np.repeat(np.asarray(s_gpu, np.float64), 128, axis=1)
    v_ref = ref32.astype(np.float64) / s_ref_e
    v_gpu = oracle.e4m3_decode_array(np.asarray(q_gpu)) * s_gpu_e / s_ref_e
    bound = e4m3_step(v_ref) + err * 448.0
    ratio = float(np.max(np.abs(v_gpu - v_ref) / bound))
    frac = float((np.asarray(q_gpu) != q_ref).mean())
    srel = float(np.max(np.abs(np.asarray(s_gpu, np.float64) - s_ref) / np.maximum(np.abs(s_ref), 1e-30)))
    return ratio, frac, srel


def mx_codes_close(q_gpu, s_gpu, act_ref_f64, err=1e-3):
    """Compare MXFP8-quantised rows (codes + E8M0 scale codes per 1 x 32 block) with the
    oracle's unquantised activation act_ref, as e4m3_codes_close does for 1 x 128 blocks:
    each dequantised element must lie within one e4m3 step (at the oracle's own block scale)
    of act_ref, plus its saturation error, plus err of that block's range. The MX rule maps a
    block's largest value into [256, 512) and clamps [448, 512) to 448; when a block's
    maximum sits at a power of two, the GPU's fp32 value may fall on the other side of it
    and take the scale one below the oracle's, and then elements of the block saturate at
    the GPU's scale, so the saturation allowance is taken at both scales. Returns
    (max |error| / bound, fraction of codes differing from the oracle's own quantisation,
    max |scale code difference|, fraction of scale codes differing)."""
    import oracle
    ref32 = np.asarray(act_ref_f64, np.float64).astype(np.float32)
    q_ref, s_ref = oracle.mx_quant(ref32)
    sc_ref = np.repeat(np.exp2(np.asarray(s_ref, np.float64) - 127.0), 32, axis=-1)
    sc_gpu = np.repeat(np.exp2(np.asarray(s_gpu, np.float64) - 127.0), 32, axis=-1)
    v_ref = ref32.astype(np.float64)
    v_gpu = oracle.e4m3_decode_array(np.asarray(q_gpu)) * sc_gpu
    u = np.abs(v_ref / sc_ref)
    ug = np.abs(v_ref / sc_gpu)
    bound = ((e4m3_step(u) + np.maximum(u - 448.0, 0.0) + err * 448.0) * sc_ref
             + np.maximum(ug - 448.0, 0.0) * sc_gpu)
    ratio = float(np.max(np.abs(v_gpu - v_ref) / bound))
    frac = float((np.asarray(q_gpu) != q_ref).mean())
    ds = np.asarray(s_gpu, np.int32) - np.asarray(s_ref, np.int32)
    return ratio, frac, int(np.max(np.abs(ds))), float((ds != 0).mean())


def routing_margin(cfg, logits, logit_bias=None, sel_bias=None):
    """Per token, how close the oracle's selection is to a tie, relative to max|key| of the
    token: the smallest of (a) the key gap between the k-th selected expert and the best
    unselected candidate and, for the group-limited router, (b) the score gap between the
    last kept group and the best dropped group. Keys are the oracle's own: l + logit_bias
    (softmax router), or fp32(s + sel_bias) with the oracle's s (sigmoid router). A token
    whose expert set changes under a small perturbation of the logits must have a small
    margin."""
    import oracle
    lg = np.asarray(logits, np.float32)
    T, E = lg.shape
    lb = None if logit_bias is None else np.asarray(logit_bias, np.float32)
    l = lg if lb is None else (lg + lb[None, :]).astype(np.float32)
    k = cfg.k
    if cfg.router == oracle.SOFTMAX_TOPK:
        key = l.astype(np.float64)
        srt = -np.sort(-key, axis=1)
        gap = srt[:, k - 1] - srt[:, k] if k < E else np.full(T, np.inf)
    else:
        _, _, s = oracle.route_cfg(cfg, lg, lb, sel_bias, return_scores=True)
        sb = np.zeros(E, np.float32) if sel_bias is None else np.asarray(sel_bias, np.float32)
        key32 = (s + sb[None, :]).astype(np.float32)
        key = key32.astype(np.float64)
        G, TG, per = cfg.n_groups, cfg.topk_groups, E // cfg.n_groups
        grp = -np.sort(-key32.reshape(T, G, per), axis=2)
        gs = (grp[:, :, 0] + grp[:, :, 1]).astype(np.float32).astype(np.float64)
        gsrt = -np.sort(-gs, axis=1)
        ggap = gsrt[:, TG - 1] - gsrt[:, TG] if TG < G else np.full(T, np.inf)
        # expert gap inside the oracle's kept groups
        gorder = np.argsort(-gs, axis=1, kind="stable")[:, :TG]
        allowed = np.zeros((T, G), bool)
        np.put_along_axis(allowed, gorder, True, axis=1)
        masked = np.where(np.repeat(allowed, per, axis=1), key, -np.inf)
        srt = -np.sort(-masked, axis=1)
        egap = srt[:, k - 1] - srt[:, k] if k < TG * per else np.full(T, np.inf)
        gap = np.minimum(ggap, egap)
    return gap / np.maximum(np.max(np.abs(key), axis=1), 1e-30)

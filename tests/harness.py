"""Shared helpers of the GPU parity tests: seeded inputs on both sides, oracle
calls, error measures. Imports the oracle (tests may) and the product binding."""
from __future__ import annotations

import functools
import sys

import numpy as np

from oracle import qlayer_ref as ref
from transformer_decoder_layer_qwen_amd import configs, synth

BF16_TOL = 2e-2     # max|err| <= 2e-2 * RMS(output) for bf16 paths (the layer output Y)
# Branch self-checks, so the residual cannot hide an error in a branch. The
# FFN branch Y - R is measured through Y after removing Y's own rounding
# (branch_err) against its RMS over all rows, with the 2e-2 bar. The
# attention branch R - X is measured row by row: row t's largest error over
# row t's own branch RMS (rowwise_err), so the bound does not depend on which
# rows are compared. Its floor is the bf16 storage of q, k and v that the
# cache format imposes: the oracle fed bf16-rounded q, k, v (nothing else
# rounded) reads 1.2e-2 (d=256 test layer), 1.9e-2 (Qwen2.5-7B, 512 rows)
# and 1.4e-2 (Qwen3-8B, 512 rows) at the worst row, medians 0.7-1.3e-2; the
# bound is twice the largest of them.
ATT_ROW_TOL = 4e-2
FFN_BRANCH_TOL = 2e-2
# The MoE FFN branch is small beside the residual (RMS 0.14 against RMS(Y)
# 1.0 at Qwen3-30B-A3B) and passes three bf16 stores of its own: z (the
# experts' input), h and each expert's output (kept in slot order before the
# weighted sum). The oracle with exactly those roundings and nothing else, on
# identical R, reads 2.6e-2 over 4096 tokens; the bound is about twice that.
MOE_BRANCH_TOL = 5e-2
F32_TOL = 1e-5      # relative, fp32 toy
GAP_MIN = 1e-3      # routing sets must match where the k-th/(k+1)-th gap exceeds this


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def spec_of(cfg: configs.LayerConfig, **kw) -> ref.LayerSpec:
    s = dict(d=cfg.d, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
             head_dim=cfg.head_dim, ffn_dim=cfg.ffn_dim, n_experts=cfg.n_experts,
             top_k=cfg.top_k, norm_topk_prob=cfg.norm_topk_prob,
             shared_ffn_dim=cfg.shared_ffn_dim, qkv_bias=cfg.qkv_bias,
             qk_norm=cfg.qk_norm, eps=cfg.rms_eps, theta=cfg.rope_theta)
    s.update(kw)
    return ref.LayerSpec(**s)


def widen(w_np):
    """Stored weights -> float64, once (the oracle would otherwise widen every
    matrix at every call)."""
    return {k: synth.to_f32(v).astype(np.float64) for k, v in w_np.items()}


def rel_err(got, want) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    rms = float(np.sqrt(np.mean(want * want)))
    return float(np.max(np.abs(got - want))) / max(rms, 1e-30)


def rounding_err(got, want, rel=2.0 ** -8, noise=1e-3) -> float:
    """Largest |got - want| in units of the allowance rel*|want| + noise*RMS(want).

    A tensor stored in bf16 with round-to-nearest-even is off by at most 2^-9
    of its magnitude, so rel = 2^-8 leaves a factor of two; `noise` covers the
    fp32 accumulation and upstream differences. <= 1 passes."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    rms = float(np.sqrt(np.mean(want * want)))
    allow = rel * np.abs(want) + noise * max(rms, 1e-30)
    return float(np.max(np.abs(got - want) / allow))


def attention_err(got, want, v) -> float:
    """Attention output against the oracle fed the same q, k, v, in units of
    its rounding bound. The kernels round each probability p to bf16 (relative
    error <= 2^-9) and normalise by the sum of the rounded values, so the
    weights w~ = p~ / sum p~ differ from w = p / sum p by at most 2 * 2^-9 * w
    and |o - o_ref| = |sum (w~ - w) v| <= 2^-8 * max|v|; the allowance is twice
    that plus fp32 noise. <= 1 passes."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    rms = float(np.sqrt(np.mean(want * want)))
    allow = 2.0 ** -7 * float(np.max(np.abs(v))) + 1e-4 * rms
    return float(np.max(np.abs(got - want))) / allow


def excess_err(got_bf16, want) -> float:
    """max|got - want| less got's own bf16 rounding (half an ulp of each
    stored value), over RMS(want): the output bar with the output format's
    storage error taken out."""
    g = np.asarray(got_bf16, np.float64)
    w = np.asarray(want, np.float64)
    _, e = np.frexp(g)                       # |g| in [2^(e-1), 2^e): ulp = 2^(e-8)
    half = np.where(g != 0, np.ldexp(1.0, e - 9), 0.0)
    rms = float(np.sqrt(np.mean(w * w)))
    return float(np.max(np.maximum(np.abs(g - w) - half, 0.0))) / max(rms, 1e-30)


# Layers whose output cannot meet max|err| <= 2e-2 * RMS(Y) in bf16 at all:
# rounding Y alone (the oracle's exact Y stored in bf16, nothing else
# rounded) already reads the value below on the prefill workload, because
# max|Y| / RMS(Y) is 5.6 (Mixtral-like) and 7.0 (Qwen2-57B-A14B) and half an
# ulp of bf16 in [8, 16) is 2^-5; the bf16 K/V cache then adds its own share.
# For these the bar is applied to the error in excess of Y's own rounding
# (excess_err); the plain figure is still reported.
Y_ROUNDING_FLOOR = {"mixtral-like": 1.91e-2, "qwen2-57b-a14b": 1.75e-2}


def rowwise_err(got, want) -> float:
    """Largest over rows (leading axes flattened) of max|got - want| in the row
    over RMS(want) of the same row."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    d = got.shape[-1]
    g = got.reshape(-1, d)
    w = want.reshape(-1, d)
    rms = np.sqrt(np.mean(w * w, axis=1))
    return float(np.max(np.max(np.abs(g - w), axis=1) / np.maximum(rms, 1e-30)))


def branch_err(y_bf16, r, f_ref) -> float:
    """Error of a residual branch F seen through the stored bf16 output
    y = bf16(r + F): |y - r - F_ref| less y's own rounding (at most half an
    ulp, <= 2^-8 |y|), relative to RMS(F_ref). Keeps a small branch from
    hiding behind a large residual."""
    y = np.asarray(y_bf16, np.float64)
    f = np.asarray(f_ref, np.float64)
    excess = np.maximum(np.abs(y - np.asarray(r, np.float64) - f) - 2.0 ** -8 * np.abs(y), 0.0)
    return float(np.max(excess)) / max(float(np.sqrt(np.mean(f * f))), 1e-30)


def bf16_round(a) -> np.ndarray:
    """Round to the nearest bf16 (ties to even), as stored by the kernels."""
    return synth.to_f32(synth.f32_to_bf16_bits(np.asarray(a, np.float32))).astype(np.float64)


def small_cfg(**kw) -> configs.LayerConfig:
    base = dict(name="small-bf16", d=256, n_q_heads=4, n_kv_heads=2, head_dim=128, ffn_dim=384,
                qkv_bias=True, qk_norm=True, rope_theta=1e4)
    base.update(kw)
    return configs.LayerConfig(**base)


def small_moe_cfg(**kw) -> configs.LayerConfig:
    base = dict(name="small-moe", d=256, n_q_heads=4, n_kv_heads=2, head_dim=128, ffn_dim=128,
                n_experts=32, top_k=4, qk_norm=True, router_std=0.1)
    base.update(kw)
    return configs.LayerConfig(**base)


@functools.lru_cache(maxsize=4)
def weights_for(cfg: configs.LayerConfig, seed: int):
    """(stored numpy weights, weights widened to float64)."""
    w = synth.make_weights(cfg, seed)
    return w, widen(w)


def flip_report(logits_gpu, logits_ref, k, edges=(1e-3, 1e-2)):
    """Tokens whose top-k expert set from the GPU's router logits differs from
    the oracle's, binned by the oracle's k-th/(k+1)-th logit gap: a dict
    "lo..hi" -> (flipped, tokens)."""
    lr = np.asarray(logits_ref, np.float64)
    srt = -np.sort(-lr, axis=-1)
    gap = srt[:, k - 1] - srt[:, k]
    want = np.sort(ref.topk_select(lr, k), axis=-1)
    got = np.sort(ref.topk_select(np.asarray(logits_gpu, np.float64), k), axis=-1)
    diff = np.any(want != got, axis=-1)
    bounds = (0.0,) + tuple(edges) + (np.inf,)
    out = {}
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        sel = (gap >= lo) & (gap < hi)
        out[f"{lo:g}..{hi:g}"] = (int(diff[sel].sum()), int(sel.sum()))
    return out


def routing_mismatch(idx_gpu, logits_ref, k, gap_min=GAP_MIN):
    """Tokens whose selected set differs from the oracle's where its
    k-th/(k+1)-th logit gap exceeds gap_min. Returns (bad tokens, checked)."""
    l = np.asarray(logits_ref, np.float64)
    srt = -np.sort(-l, axis=-1)
    gap = srt[:, k - 1] - srt[:, k] if l.shape[1] > k else np.full(l.shape[0], np.inf)
    want = np.sort(ref.topk_select(l, k), axis=-1)
    got = np.sort(np.asarray(idx_gpu), axis=-1)
    check = gap > gap_min
    bad = np.nonzero(check & np.any(want != got, axis=-1))[0]
    return bad, int(check.sum())


def oracle_gaps(logits_ref, k) -> np.ndarray:
    """The oracle's k-th minus (k+1)-th largest logit per token."""
    l = np.asarray(logits_ref, np.float64)
    if l.shape[-1] <= k:
        return np.full(l.shape[0], np.inf)
    srt = -np.sort(-l, axis=-1)
    return srt[:, k - 1] - srt[:, k]


def moe_rerouted(o, logits_gpu, w, spec):
    """Whole-layer MoE rows: the bf16 roundings upstream of the router move
    the GPU's logits by ~1e-3 from the oracle's, so a token whose k-th/(k+1)-th
    gap is that small may select another expert set; its FFN output is then a
    different (equally valid) sum. For every such token this returns the
    oracle's own FFN output for the GPU's selection (the oracle's z, its gate
    weights over the oracle's logits at those experts), so every row can be
    compared. o: the oracle's layer outputs flattened to [N, ...] ("z", "f",
    "logits", "idx"). Returns (f [N, d], flipped [N] bool)."""
    k = spec.top_k
    lg = np.asarray(logits_gpu, np.float64).reshape(-1, spec.n_experts)
    idx_g = ref.topk_select(lg, k)
    flipped = np.any(np.sort(idx_g, -1) != np.sort(np.asarray(o["idx"]).reshape(-1, k), -1), -1)
    f = np.array(o["f"], np.float64).reshape(lg.shape[0], -1)
    z = np.asarray(o["z"], np.float64).reshape(lg.shape[0], -1)
    lr = np.asarray(o["logits"], np.float64).reshape(lg.shape[0], -1)
    for t in np.nonzero(flipped)[0]:
        wts = ref.gate_weights(lr[t:t + 1], idx_g[t:t + 1], spec.norm_topk_prob)[0]
        acc = np.zeros(f.shape[1])
        for i in range(k):
            e = int(idx_g[t, i])
            acc = acc + wts[i] * ref.swiglu_ffn(z[t:t + 1], w["we_gate"][e], w["we_up"][e],
                                                w["we_down"][e])[0]
        if spec.shared_ffn_dim:
            acc = acc + ref.shared_expert(z[t:t + 1], w)[0][0]
        f[t] = acc
    return f, flipped

"""Shared helpers of the GPU parity tests: seeded inputs on both sides, oracle
calls, error measures. Imports the oracle (tests may) and the product binding."""
from __future__ import annotations

import functools
import sys

import numpy as np

from oracle import qlayer_ref as ref
from transformer_decoder_layer_qwen_amd import configs, synth

BF16_TOL = 2e-2     # max|err| <= 2e-2 * RMS(output) for bf16 paths (the layer output Y)
# Branch self-checks (R - X and Y - R on their own scale). The attention branch
# inherits the bf16 rounding of q, k, v (K and V live in the bf16 cache); a
# bf16-rounding emulation of the oracle puts that floor at ~2.8% on the small
# test layer, so its bound is 4e-2. The FFN branch is measured through Y after
# removing Y's own rounding (branch_err) and keeps the 2e-2 bound.
ATT_BRANCH_TOL = 4e-2
FFN_BRANCH_TOL = 2e-2
F32_TOL = 1e-5      # relative, fp32 toy
GAP_MIN = 1e-3      # routing sets must match where the k-th/(k+1)-th gap exceeds this


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def spec_of(cfg: configs.LayerConfig, **kw) -> ref.LayerSpec:
    s = dict(d=cfg.d, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
             head_dim=cfg.head_dim, ffn_dim=cfg.ffn_dim, n_experts=cfg.n_experts,
             top_k=cfg.top_k, norm_topk_prob=cfg.norm_topk_prob, qkv_bias=cfg.qkv_bias,
             qk_norm=cfg.qk_norm, eps=cfg.rms_eps, theta=cfg.rope_theta)
    s.update(kw)
    return ref.LayerSpec(**s)


def widen(w_np):
    return {k: synth.to_f32(v) for k, v in w_np.items()}


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
    its rounding bound. The kernel rounds each probability p to bf16 before
    the P*V product (relative error <= 2^-9) and divides by the unrounded sum,
    so |o - o_ref| <= 2^-9 * sum_u p_u |v_u| / sum_u p_u <= 2^-9 * max|v|; the
    allowance is twice that plus fp32 noise. <= 1 passes."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    rms = float(np.sqrt(np.mean(want * want)))
    allow = 2.0 ** -8 * float(np.max(np.abs(v))) + 1e-4 * rms
    return float(np.max(np.abs(got - want))) / allow


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
    """(stored numpy weights, widened fp32 weights)."""
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

"""Rounding floor of the bf16 GPU path on a dense prefill layer (CPU, fp64).

Not a test: a measurement behind the precision choices of the HIP path. The
layer is computed twice in float64 with the oracle's own step functions: once
exactly, once rounding to bf16 exactly the tensors a given kernel design
stores (q, the K/V cache rows, the attention probabilities -- normalised by
the sum of their rounded values -- and the layer output Y always; the
RMSNorm1 output x-hat, the attention output O, the RMSNorm2 output z and the
SwiGLU hidden h only when the variant says so). It prints max|err| / RMS(Y)
over every element for each variant, the figure the 2e-2 bar applies to.

    python tests/rounding_floor.py 3 1024    # Qwen2.5-7B, one sequence of 1024
    python tests/rounding_floor.py 4 2048    # Qwen3-8B, one sequence of 2048
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from oracle import qlayer_ref as ref                             # noqa: E402
from transformer_decoder_layer_qwen_amd import configs, synth    # noqa: E402

# (x-hat, O, z, h) rounded to bf16 before their projections
VARIANTS = [(0, 0, 0, 0), (1, 0, 0, 0), (0, 1, 0, 0), (1, 1, 0, 0), (0, 0, 1, 0),
            (0, 0, 0, 1), (1, 1, 1, 1)]


def bf16(a):
    a32 = np.asarray(a, dtype=np.float32)
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(a32)).astype(np.float64)


def run(cid: int, S: int) -> None:
    cfg = configs.CONFIGS[cid]
    assert not cfg.is_moe
    W = {k: synth.to_f32(v).astype(np.float64)
         for k, v in synth.make_weights(cfg, configs.weight_seed(cid)).items()}
    x = synth.to_f32(synth.make_prefill_input(cfg, 1000 * cid + 1, 1, S)).astype(np.float64)[0]
    Hq, Hkv, dh, eps = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps
    pos = np.arange(S, dtype=np.float64)
    causal = np.tril(np.ones((S, S), bool))

    def layer(rx, ro, rz, rh, stored_bf16):
        xh = ref.rmsnorm(x, W["ln1_g"], eps)
        if rx:
            xh = bf16(xh)
        q = ref.linear(xh, W["wq"], W.get("bq") if cfg.qkv_bias else None)
        k = ref.linear(xh, W["wk"], W.get("bk") if cfg.qkv_bias else None)
        v = ref.linear(xh, W["wv"], W.get("bv") if cfg.qkv_bias else None)
        q, k, v = (ref.split_heads(q, Hq, dh), ref.split_heads(k, Hkv, dh),
                   ref.split_heads(v, Hkv, dh))
        if cfg.qk_norm:
            q = ref.head_rmsnorm(q, W["q_norm_g"], eps)
            k = ref.head_rmsnorm(k, W["k_norm_g"], eps)
        q = ref.rope_rotate_half(q, pos, cfg.rope_theta)
        k = ref.rope_rotate_half(k, pos, cfg.rope_theta)
        if stored_bf16:
            q, k, v = bf16(q), bf16(k), bf16(v)
        o = np.empty((S, Hq, dh))
        for h in range(Hq):
            g = ref.kv_group(h, Hq, Hkv)
            s = np.where(causal, (q[:, h] @ k[:, g].T) / np.sqrt(dh), -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            if stored_bf16:
                p = bf16(p)
            o[:, h] = (p @ v[:, g]) / p.sum(axis=1, keepdims=True)
        o = o.reshape(S, Hq * dh)
        if ro:
            o = bf16(o)
        r = x + ref.linear(o, W["wo"])
        z = ref.rmsnorm(r, W["ln2_g"], eps)
        if rz:
            z = bf16(z)
        hid = ref.swiglu_hidden(z, W["w_gate"], W["w_up"])
        if rh:
            hid = bf16(hid)
        y = r + ref.linear(hid, W["w_down"])
        return bf16(y) if stored_bf16 else y

    t0 = time.time()
    y0 = layer(0, 0, 0, 0, False)
    rms = float(np.sqrt(np.mean(y0 * y0)))
    print(f"{cfg.name} S={S}: exact layer in {time.time() - t0:.1f}s, RMS(Y) {rms:.4f}, "
          f"max|Y| {np.abs(y0).max():.3f}", flush=True)
    for var in VARIANTS:
        e = np.abs(layer(*var, True) - y0)
        print(f"  bf16 (x-hat, O, z, h) = {var}: max|err|/RMS(Y) = {e.max() / rms:.4e}", flush=True)


if __name__ == "__main__":
    run(int(sys.argv[1]), int(sys.argv[2]))

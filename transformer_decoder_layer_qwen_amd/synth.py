"""Seeded synthetic weights and inputs, shared by the tests, the oracle checks
and the benchmark.

This module holds no arithmetic of the layer: it only draws normal numbers in a
fixed, documented order and stores them either as float32 (the f32 toy) or as
bfloat16 bit patterns (round-to-nearest-even of the float32 draw).

Draw order for the weights of one config (seed ``1000*cfg``), one
``numpy.random.Generator(PCG64(seed))`` stream, float32 standard normals scaled
as ``mean + std*z``:

    ln1_g[d], ln2_g[d],                        N(gamma_mean, gamma_std)
    wq[q,d], wk[kv,d], wv[kv,d], wo[d,q],      N(0, w_std)
    bq[q], bk[kv], bv[kv]        (qkv_bias)    N(0, b_std)
    q_norm_g[dh], k_norm_g[dh]   (qk_norm)     N(gamma_mean, gamma_std)
    dense: w_gate[f,d], w_up[f,d], w_down[d,f] N(0, w_std)
    MoE:   w_router[E,d]                       N(0, router_std)
           we_gate[E,mf,d], we_up[E,mf,d], we_down[E,d,mf]  (expert by expert,
           gate then up then down inside an expert)         N(0, w_std)
           shared expert (shared_ffn_dim sf > 0): ws_gate[sf,d], ws_up[sf,d],
           ws_down[d,sf], w_shared_gate[1,d]                N(0, w_std)

A tensor whose std is 0 is filled with its mean and consumes no draws.  All
weights follow the ``[out, in]`` storage convention.

Inputs of a workload (seed ``1000*cfg + index``):

    prefill: x[B,S,d]                                  N(0, x_std)
    decode:  x[B,d] N(0, x_std); then k_cache, v_cache [B,T_max,Hkv,dh], rows
             0..cache_len-1 N(0, cache_std) (K first, then V, batch by batch);
             rows >= cache_len hold a canary (NaN unless ``canary=None``).
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .configs import LayerConfig

BF16_NAN_BITS = np.uint16(0x7FC0)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def to_f32(a: np.ndarray) -> np.ndarray:
    """Float32 view of a stored tensor (bf16 bits are widened exactly)."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a)
    return np.asarray(a, dtype=np.float32)


def _draw(rng: np.random.Generator, shape, mean: float, std: float,
          dtype: str, chunk: int = 1 << 24) -> np.ndarray:
    n = int(np.prod(shape)) if len(shape) else 1
    store = np.uint16 if dtype == "bf16" else np.float32
    out = np.empty(n, dtype=store)
    if std == 0.0:
        out[:] = f32_to_bf16_bits(np.full(1, mean, np.float32))[0] if dtype == "bf16" \
            else np.float32(mean)
        return out.reshape(shape)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        z = rng.standard_normal(e - s, dtype=np.float32)
        z *= np.float32(std)
        z += np.float32(mean)
        out[s:e] = f32_to_bf16_bits(z) if dtype == "bf16" else z
    return out.reshape(shape)


def weight_shapes(cfg: LayerConfig) -> Dict[str, tuple]:
    """Shapes of every tensor one layer holds, in draw order ([out, in])."""
    d, q, kv, dh, f = cfg.d, cfg.q_dim, cfg.kv_dim, cfg.head_dim, cfg.ffn_dim
    s = {"ln1_g": (d,), "ln2_g": (d,),
         "wq": (q, d), "wk": (kv, d), "wv": (kv, d), "wo": (d, q)}
    if cfg.qkv_bias:
        s.update(bq=(q,), bk=(kv,), bv=(kv,))
    if cfg.qk_norm:
        s.update(q_norm_g=(dh,), k_norm_g=(dh,))
    if cfg.is_moe:
        E = cfg.n_experts
        s.update(w_router=(E, d), we_gate=(E, f, d), we_up=(E, f, d), we_down=(E, d, f))
        if cfg.shared_ffn_dim:
            sf = cfg.shared_ffn_dim
            s.update(ws_gate=(sf, d), ws_up=(sf, d), ws_down=(d, sf), w_shared_gate=(1, d))
    else:
        s.update(w_gate=(f, d), w_up=(f, d), w_down=(d, f))
    return s


def make_weights(cfg: LayerConfig, seed: int) -> Dict[str, np.ndarray]:
    rng = np.random.Generator(np.random.PCG64(seed))
    shapes = weight_shapes(cfg)
    dt = cfg.dtype
    w: Dict[str, np.ndarray] = {}
    for name in ("ln1_g", "ln2_g"):
        w[name] = _draw(rng, shapes[name], cfg.gamma_mean, cfg.gamma_std, dt)
    for name in ("wq", "wk", "wv", "wo"):
        w[name] = _draw(rng, shapes[name], 0.0, cfg.w_std, dt)
    if cfg.qkv_bias:
        for name in ("bq", "bk", "bv"):
            w[name] = _draw(rng, shapes[name], 0.0, cfg.b_std, dt)
    if cfg.qk_norm:
        for name in ("q_norm_g", "k_norm_g"):
            w[name] = _draw(rng, shapes[name], cfg.gamma_mean, cfg.gamma_std, dt)
    if cfg.is_moe:
        w["w_router"] = _draw(rng, shapes["w_router"], 0.0, cfg.router_std, dt)
        E, mf, d = cfg.n_experts, cfg.ffn_dim, cfg.d
        store = np.uint16 if dt == "bf16" else np.float32
        g = np.empty((E, mf, d), store)
        u = np.empty((E, mf, d), store)
        dn = np.empty((E, d, mf), store)
        for e in range(E):
            g[e] = _draw(rng, (mf, d), 0.0, cfg.w_std, dt)
            u[e] = _draw(rng, (mf, d), 0.0, cfg.w_std, dt)
            dn[e] = _draw(rng, (d, mf), 0.0, cfg.w_std, dt)
        w.update(we_gate=g, we_up=u, we_down=dn)
        if cfg.shared_ffn_dim:
            for name in ("ws_gate", "ws_up", "ws_down", "w_shared_gate"):
                w[name] = _draw(rng, shapes[name], 0.0, cfg.w_std, dt)
    else:
        for name in ("w_gate", "w_up", "w_down"):
            w[name] = _draw(rng, shapes[name], 0.0, cfg.w_std, dt)
    return w


def make_prefill_input(cfg: LayerConfig, seed: int, B: int, S: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return _draw(rng, (B, S, cfg.d), 0.0, cfg.x_std, cfg.dtype)


def make_decode_input(cfg: LayerConfig, seed: int, B: int, cache_len: int,
                      T_max: Optional[int] = None, canary: Optional[str] = "nan"):
    """Returns (x[B,d], k_cache, v_cache, cache_len[B] int32)."""
    if T_max is None:
        T_max = cache_len + 1
    rng = np.random.Generator(np.random.PCG64(seed))
    x = _draw(rng, (B, cfg.d), 0.0, cfg.x_std, cfg.dtype)
    store = np.uint16 if cfg.dtype == "bf16" else np.float32
    Hkv, dh = cfg.n_kv_heads, cfg.head_dim
    kc = np.empty((B, T_max, Hkv, dh), store)
    vc = np.empty((B, T_max, Hkv, dh), store)
    fill = BF16_NAN_BITS if cfg.dtype == "bf16" else np.float32(np.nan)
    if canary is None:
        fill = store(0)
    for b in range(B):
        kc[b, :cache_len] = _draw(rng, (cache_len, Hkv, dh), 0.0, cfg.cache_std, cfg.dtype)
        vc[b, :cache_len] = _draw(rng, (cache_len, Hkv, dh), 0.0, cfg.cache_std, cfg.dtype)
        kc[b, cache_len:] = fill
        vc[b, cache_len:] = fill
    lens = np.full(B, cache_len, np.int32)
    return x, kc, vc, lens


def make_moe_input(cfg: LayerConfig, seed: int, N: int) -> np.ndarray:
    """Residual-stream rows r[N,d] fed straight to the MoE FFN entry point."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _draw(rng, (N, cfg.d), 0.0, cfg.x_std, cfg.dtype)

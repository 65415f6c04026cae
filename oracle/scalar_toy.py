"""Brute-force scalar-loop layer for tiny shapes (pure Python + ``math``).

TEST INFRASTRUCTURE, like the rest of ``oracle/``: it exists to pin the NumPy
oracle on small inputs with an implementation that shares no code with it
(no NumPy, every sum an explicit loop). Only ``tests/`` use it.

Follows the same pages as ``qlayer_ref`` ([P3] "推理系统 03：逐项算清一个真实
Qwen3 Transformer 层" §2-§10 for the layer; [P1] "Qwen2.5-7B 结构拆解" §03.1
for the [out, in] weight convention), one scalar at a time:

  x_hat[t][j] = g1[j] * x[t][j] / sqrt(sum_j x[t][j]^2 / d + eps)
  q[t][n]     = sum_j x_hat[t][j] * Wq[n][j] (+ bq[n]);  same for k, v
  per head: optional RMSNorm over dh, then rotation of (i, i + dh/2) pairs
  s[t][u]     = sum_i q[t][h*dh+i] * k[u][g*dh+i] / sqrt(dh), u <= t
  a[t][u]     = exp(s - max) / sum exp(s - max);  o[t][h*dh+i] = sum_u a v
  r[t][j]     = x[t][j] + sum_n o[t][n] * Wo[j][n]
  y[t][j]     = r[t][j] + sum_m silu(gate[t][m]) * up[t][m] * Wd[j][m]
"""
from __future__ import annotations

import math
from typing import List, Optional

Vec = List[float]
Mat = List[List[float]]


def _matvec_out_in(W: Mat, x: Vec, bias: Optional[Vec] = None) -> Vec:
    out = []
    for n in range(len(W)):
        acc = 0.0
        row = W[n]
        for j in range(len(x)):
            acc += x[j] * row[j]
        if bias is not None:
            acc += bias[n]
        out.append(acc)
    return out


def _rms(x: Vec, g: Vec, eps: float) -> Vec:
    ss = 0.0
    for v in x:
        ss += v * v
    den = math.sqrt(ss / len(x) + eps)
    return [g[j] * x[j] / den for j in range(len(x))]


def _rotate(vec: Vec, pos: float, theta: float) -> Vec:
    dh = len(vec)
    half = dh // 2
    out = list(vec)
    for i in range(half):
        w = theta ** (-2.0 * i / dh)
        a = pos * w
        c, s = math.cos(a), math.sin(a)
        x0, x1 = vec[i], vec[i + half]
        out[i] = c * x0 - s * x1
        out[i + half] = s * x0 + c * x1
    return out


def toy_layer(x: Mat, W: dict, Hq: int, Hkv: int, dh: int, eps: float = 1e-6,
              theta: float = 1e6, pos_offset: int = 0, qk_norm: bool = False,
              qkv_bias: bool = False) -> Mat:
    """One sequence x[T][d] -> y[T][d]; W holds nested lists in [out, in]."""
    T = len(x)
    group = Hq // Hkv
    qs, ks, vs = [], [], []
    for t in range(T):
        xh = _rms(x[t], W["ln1_g"], eps)
        q = _matvec_out_in(W["wq"], xh, W["bq"] if qkv_bias else None)
        k = _matvec_out_in(W["wk"], xh, W["bk"] if qkv_bias else None)
        v = _matvec_out_in(W["wv"], xh, W["bv"] if qkv_bias else None)
        qh, kh = [], []
        for h in range(Hq):
            seg = q[h * dh:(h + 1) * dh]
            if qk_norm:
                seg = _rms(seg, W["q_norm_g"], eps)
            qh.extend(_rotate(seg, t + pos_offset, theta))
        for h in range(Hkv):
            seg = k[h * dh:(h + 1) * dh]
            if qk_norm:
                seg = _rms(seg, W["k_norm_g"], eps)
            kh.extend(_rotate(seg, t + pos_offset, theta))
        qs.append(qh)
        ks.append(kh)
        vs.append(v)
    y = []
    for t in range(T):
        o = [0.0] * (Hq * dh)
        for h in range(Hq):
            g = h // group
            scores = []
            for u in range(t + 1):
                acc = 0.0
                for i in range(dh):
                    acc += qs[t][h * dh + i] * ks[u][g * dh + i]
                scores.append(acc / math.sqrt(dh))
            m = max(scores)
            ex = [math.exp(s - m) for s in scores]
            tot = sum(ex)
            for u in range(t + 1):
                a = ex[u] / tot
                for i in range(dh):
                    o[h * dh + i] += a * vs[u][g * dh + i]
        attn = _matvec_out_in(W["wo"], o)
        r = [x[t][j] + attn[j] for j in range(len(x[t]))]
        z = _rms(r, W["ln2_g"], eps)
        gate = _matvec_out_in(W["w_gate"], z)
        up = _matvec_out_in(W["w_up"], z)
        hid = [gate[m] / (1.0 + math.exp(-gate[m])) * up[m] for m in range(len(gate))]
        f = _matvec_out_in(W["w_down"], hid)
        y.append([r[j] + f[j] for j in range(len(r))])
    return y

"""Plain float64 CPU oracle of one Qwen-style pre-norm decoder layer (forward).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The product path
(the HIP library and its Python binding) never imports, links or calls it, and
this module imports nothing from the product package.

Every step is the plain definition written out in NumPy float64, with no
blocking, fusion or reordering beyond what the definition states. Inputs may
be any float dtype (bf16 values arrive widened exactly to float32); everything
is converted to float64 before use and never rounded afterwards.

Sources (page title, then the section each function follows):

[P1] "Qwen2.5-7B 结构拆解" (daleiyang.github.io, llm-inference-anatomy)
[P2] "MoE 初步：参数量计算、Qwen3-30B-A3B、GQA 与 Sparse MoE"
     (hqhq1025.github.io, ai-course-notes lecture01)
[P3] "推理系统 03：逐项算清一个真实 Qwen3 Transformer 层" (marvinlee.cn)
[P4] "Transformer 的 Infra 视角" (inference-learning-path.pages.dev)
[P5] "第七章 模型容量与参数量推导" (starbuckoverflow.cn)

Readings where the pages are silent or disagree:

* RoPE pairs coordinate i with i + dh/2 (rotate_half, [P3 §6]); [P1 §05.3]
  pairs (2i, 2i+1). ``rope_adjacent`` keeps the [P1] form only to pin the
  two against each other under a fixed coordinate permutation.
* SiLU goes on the gate branch: SiLU(gate) * up ([P1 §07.1], [P3 §10]);
  [P2 "Expert 的 FFN 结构"] writes it on the up branch but names the other
  matrix the gating branch.
* Router weights: with norm_topk_prob the k selected probabilities are
  renormalised ([P1 §10.2]); equal in exact arithmetic to a softmax over the k
  selected logits ([P2 "Router 机制"]). The oracle computes the softmax over
  the selected logits; ``gate_weights_via_full_softmax`` is the [P1] route,
  kept to pin the two equal.
* Top-k ties (not on the pages): descending logit, ties to the lower index.
* The shared expert's gate row W_sg ([P1 §10.1]) is stored [1, d] like every
  [out, in] weight; its sigmoid scales the shared SwiGLU's output, which is
  added to the routed sum with no further normalisation ([P1 §10.2]).
* epsilon = 1e-6 everywhere, QK-norm included (the only value printed, [P3 §1]).
* QKV bias only (Qwen2.5, [P1 §11]); no O-projection bias.
* Decode-cache rows are stored after QK-norm and RoPE ([P3 §12]) and are
  never rotated again; the new token sits at cache row ``cache_len``.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional, Sequence

import numpy as np


def f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


@dataclass(frozen=True)
class LayerSpec:
    """Hyper-parameters of one layer, as named in a model's config.json
    ([P1 §11]; [P2 configuration table])."""
    d: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    n_experts: int = 0
    top_k: int = 0
    norm_topk_prob: bool = True
    shared_ffn_dim: int = 0
    qkv_bias: bool = False
    qk_norm: bool = False
    eps: float = 1e-6
    theta: float = 1e6


# --------------------------------------------------------------------------
# matrix products
# --------------------------------------------------------------------------

def gemm(a, b) -> np.ndarray:
    """C = A @ B, C[i,j] = sum_p A[i,p] B[p,j] ([P1 §03.4])."""
    return f64(a) @ f64(b)


def linear(x, w, bias=None) -> np.ndarray:
    """y = x @ W^T (+ b) with W stored [out, in] ([P1 §03.1]; [P3 §4]).

    Leading axes of x are flattened into rows; rows never interact ([P1 §03.2]).
    """
    y = f64(x) @ f64(w).T
    if bias is not None:
        y = y + f64(bias)
    return y


# --------------------------------------------------------------------------
# normalisation
# --------------------------------------------------------------------------

def rmsnorm(x, gamma, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: gamma_j x_j / sqrt(mean_k x_k^2 + eps).

    [P3 §3]: mean of squares along the feature axis only, per position, no
    mean subtraction.
    """
    x = f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return f64(gamma) * x / np.sqrt(ms + eps)


# --------------------------------------------------------------------------
# heads, QK-norm, RoPE
# --------------------------------------------------------------------------

def split_heads(t, n_heads: int, head_dim: int) -> np.ndarray:
    """[..., H*dh] -> [..., H, dh]; head h owns columns [h*dh, (h+1)*dh)
    ([P1 §05.1])."""
    t = f64(t)
    return t.reshape(t.shape[:-1] + (n_heads, head_dim))


def head_rmsnorm(t, gamma, eps: float) -> np.ndarray:
    """QK-norm: RMSNorm over each head's dh values with one gamma shared by
    all heads of Q (or of K) ([P3 §5])."""
    return rmsnorm(t, gamma, eps)


def rope_frequencies(head_dim: int, theta: float) -> np.ndarray:
    """omega_r = theta^(-2r/dh), r = 0 .. dh/2-1 ([P3 §6]; [P1 §05.3])."""
    r = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * r / head_dim)


def rope_rotate_half(t, pos, theta: float) -> np.ndarray:
    """Rotate each pair (x_i, x_{i+dh/2}) by angle pos*omega_i ([P3 §6]).

    t: [T, H, dh]; pos: [T]. The 2-D rotation is R(a) = [[cos a, -sin a],
    [sin a, cos a]] acting on the column (x_i, x_{i+dh/2}).
    """
    t = f64(t)
    dh = t.shape[-1]
    half = dh // 2
    ang = f64(pos)[:, None] * rope_frequencies(dh, theta)[None, :]     # [T, dh/2]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1 = t[..., :half]
    x2 = t[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def rope_adjacent(t, pos, theta: float) -> np.ndarray:
    """[P1 §05.3] form: pairs (x_{2i}, x_{2i+1}) rotated by pos*theta_i."""
    t = f64(t)
    dh = t.shape[-1]
    ang = f64(pos)[:, None] * rope_frequencies(dh, theta)[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    xe = t[..., 0::2]
    xo = t[..., 1::2]
    out = np.empty_like(t)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


def kv_group(h: int, n_q_heads: int, n_kv_heads: int) -> int:
    """GQA: query head h reads KV head floor(h / (Hq/Hkv)) ([P3 §7];
    [P2 "GQA 的动机与机制"]; [P1 §05.2] repeat_interleave)."""
    return h // (n_q_heads // n_kv_heads)


# --------------------------------------------------------------------------
# attention core
# --------------------------------------------------------------------------

def softmax(z, axis: int = -1) -> np.ndarray:
    """Stable softmax: exp(z - max) / sum exp(z - max) ([P3 §8])."""
    z = f64(z)
    m = np.max(z, axis=axis, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def attention(q, k, v, q_idx, k_idx, n_kv_heads: int, return_probs: bool = False):
    """Masked GQA attention for one sequence.

    q: [Tq, Hq, dh] (already normed and rotated), k, v: [Tk, Hkv, dh];
    q_idx / k_idx: sequence indices of the rows. Key u is visible to query t
    iff k_idx[u] <= q_idx[t] (causal mask, [P3 §8]). For each head:
    scores = q k^T / sqrt(dh) + M, a = softmax(scores), o = a v ([P3 §7-§9];
    [P1 §05]).  Returns o: [Tq, Hq, dh] (and the per-head probabilities).
    """
    q, k, v = f64(q), f64(k), f64(v)
    Tq, Hq, dh = q.shape
    mask = f64(k_idx)[None, :] > f64(q_idx)[:, None]                  # [Tq, Tk]
    o = np.empty((Tq, Hq, dh))
    probs = []
    for h in range(Hq):
        g = kv_group(h, Hq, n_kv_heads)
        s = (q[:, h, :] @ k[:, g, :].T) / np.sqrt(dh)
        s = np.where(mask, -np.inf, s)
        a = softmax(s, axis=-1)
        o[:, h, :] = a @ v[:, g, :]
        if return_probs:
            probs.append(a)
    if return_probs:
        return o, np.stack(probs)
    return o


# --------------------------------------------------------------------------
# feed-forward
# --------------------------------------------------------------------------

def silu(z) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + e^-z) ([P1 §07.1]; [P3 §10])."""
    z = f64(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def sigmoid(z) -> np.ndarray:
    """sigmoid(z) = 1 / (1 + e^-z), the (0, 1) squashing that [P1 §07.1]
    uses inside SiLU and [P1 §10.1] applies to the shared expert's gate."""
    z = f64(z)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def swiglu_ffn(z, w_gate, w_up, w_down) -> np.ndarray:
    """F = (SiLU(z W_gate^T) * (z W_up^T)) W_down^T, no bias ([P3 §10];
    [P1 §07.1])."""
    g = linear(z, w_gate)
    u = linear(z, w_up)
    return linear(silu(g) * u, w_down)


def swiglu_hidden(z, w_gate, w_up) -> np.ndarray:
    """The gated hidden H = SiLU(z W_gate^T) * (z W_up^T) ([P3 §10])."""
    return silu(linear(z, w_gate)) * linear(z, w_up)


# --------------------------------------------------------------------------
# sparse MoE FFN
# --------------------------------------------------------------------------

def router_logits(z, w_router) -> np.ndarray:
    """logits = z W_router^T over all E experts ([P1 §10.2]; [P2 "Router
    机制"]; [P5 §3])."""
    return linear(z, w_router)


def topk_select(logits, k: int) -> np.ndarray:
    """Indices of the k largest logits per row, by descending logit, ties to
    the lower expert index (the pages do not say how ties break)."""
    l = f64(logits)
    order = np.argsort(-l, axis=-1, kind="stable")
    return order[..., :k].astype(np.int64)


def gate_weights(logits, idx, norm_topk_prob: bool = True) -> np.ndarray:
    """Gate weights of the selected experts.

    norm_topk_prob: softmax over the k selected logits ([P2 "Router 机制"]).
    Otherwise the raw probabilities of a softmax over all E logits
    ([P1 §10.2], Qwen2 setting).
    """
    l = f64(logits)
    sel = np.take_along_axis(l, idx, axis=-1)
    if norm_topk_prob:
        return softmax(sel, axis=-1)
    return np.take_along_axis(softmax(l, axis=-1), idx, axis=-1)


def gate_weights_via_full_softmax(logits, idx) -> np.ndarray:
    """[P1 §10.2] route: probs = softmax over all E, keep the k selected,
    renormalise them to sum 1."""
    p = np.take_along_axis(softmax(logits, axis=-1), idx, axis=-1)
    return p / np.sum(p, axis=-1, keepdims=True)


def shared_expert(z, w):
    """Qwen2's shared expert ([P1 §10.1]): an ordinary SwiGLU of width sf run
    on every token, its whole output vector scaled by the token's own gate
    g = sigmoid(z W_sg^T), W_sg a single row [1, d] without bias.
    Returns (g * SwiGLU_shared(z) [N, d], g [N, 1])."""
    g = sigmoid(linear(z, w["w_shared_gate"]))
    return g * swiglu_ffn(z, w["ws_gate"], w["ws_up"], w["ws_down"]), g


def moe_ffn_output(z, w, top_k: int, norm_topk_prob: bool = True, shared: bool = False):
    """MoE(z) = sum_i w_i Expert_{idx_i}(z), i over the k selected experts in
    rank order, a plain elementwise weighted sum ([P1 §10.2]; [P2 "MoE 的最终
    输出"]). Each expert is a SwiGLU with its own gate/up/down. With
    ``shared`` (Qwen2, [P1 §10.1-§10.2]) the gated shared expert is added
    elementwise as the ninth term.

    z: [N, d]. Returns (F [N, d], idx [N, k], weights [N, k], logits [N, E]).
    """
    z = f64(z)
    N = z.shape[0]
    logits = router_logits(z, w["w_router"])
    idx = topk_select(logits, top_k)
    wts = gate_weights(logits, idx, norm_topk_prob)
    d = z.shape[1]
    per_rank = np.zeros((N, top_k, d))
    E = np.asarray(w["we_gate"]).shape[0]
    for e in range(E):
        tok, rank = np.nonzero(idx == e)
        if tok.size == 0:
            continue
        out = swiglu_ffn(z[tok], w["we_gate"][e], w["we_up"][e], w["we_down"][e])
        per_rank[tok, rank] = out
    F = np.zeros((N, d))
    for i in range(top_k):
        F = F + wts[:, i:i + 1] * per_rank[:, i, :]
    if shared:
        F = F + shared_expert(z, w)[0]
    return F, idx, wts, logits


def moe_ffn(r, w, spec: LayerSpec) -> Dict[str, np.ndarray]:
    """The MoE half of a layer: Y = R + MoE(RMSNorm2(R)) ([P1 §10, §10.2])."""
    r = f64(r)
    z = rmsnorm(r, w["ln2_g"], spec.eps)
    F, idx, wts, logits = moe_ffn_output(z, w, spec.top_k, spec.norm_topk_prob,
                                         spec.shared_ffn_dim > 0)
    return {"y": r + F, "z": z, "f": F, "idx": idx, "w": wts, "logits": logits}


# --------------------------------------------------------------------------
# the layer
# --------------------------------------------------------------------------

def _ffn(z, w, spec: LayerSpec):
    if spec.n_experts:
        F, idx, wts, logits = moe_ffn_output(z, w, spec.top_k, spec.norm_topk_prob,
                                             spec.shared_ffn_dim > 0)
        return F, {"idx": idx, "w": wts, "logits": logits}
    h = swiglu_hidden(z, w["w_gate"], w["w_up"])
    return linear(h, w["w_down"]), {"h": h}


def _project_qkv(xhat, w, spec: LayerSpec, pos):
    """Q/K/V projections (+QKV bias), head split, QK-norm, RoPE
    ([P3 §4-§6]; [P1 §04, §05.1, §05.3])."""
    Hq, Hkv, dh = spec.n_q_heads, spec.n_kv_heads, spec.head_dim
    q = linear(xhat, w["wq"], w.get("bq") if spec.qkv_bias else None)
    k = linear(xhat, w["wk"], w.get("bk") if spec.qkv_bias else None)
    v = linear(xhat, w["wv"], w.get("bv") if spec.qkv_bias else None)
    q = split_heads(q, Hq, dh)
    k = split_heads(k, Hkv, dh)
    v = split_heads(v, Hkv, dh)
    if spec.qk_norm:
        q = head_rmsnorm(q, w["q_norm_g"], spec.eps)
        k = head_rmsnorm(k, w["k_norm_g"], spec.eps)
    q = rope_rotate_half(q, pos, spec.theta)
    k = rope_rotate_half(k, pos, spec.theta)
    return q, k, v


def layer_prefill(x, w, spec: LayerSpec, pos_offset: int = 0,
                  rows: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Full-sequence (prefill) forward of one layer, per independent sequence.

    R = X + Attn(RMSNorm1(X)),  Y = R + FFN(RMSNorm2(R))  ([P3 §2]; [P1 §02]).
    x: [B, S, d]. Position of sequence row t is t + pos_offset.
    ``rows`` restricts the attention/O/FFN part to those query rows (every
    row's K and V are still computed, since they are what the rows attend to);
    the returned per-row tensors then have S' = len(rows) rows.

    Returns y [B,S',d], r [B,S',d], xhat [B,S,d], q [B,S',Hq,dh], k/v
    [B,S,Hkv,dh] (the cache rows: post-norm, post-RoPE K and plain V,
    [P3 §12]), attn [B,S',Hq*dh] (heads concatenated, before W_O), z, ffn
    intermediates.
    """
    x = f64(x)
    B, S, d = x.shape
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    Hq, dh = spec.n_q_heads, spec.head_dim
    out = {k: [] for k in ("y", "r", "xhat", "q", "k", "v", "attn", "z", "f", "h",
                           "idx", "w", "logits")}
    pos = np.arange(S, dtype=np.float64) + pos_offset
    for b in range(B):
        xhat = rmsnorm(x[b], w["ln1_g"], spec.eps)
        q, k, v = _project_qkv(xhat, w, spec, pos)
        o = attention(q[rows], k, v, rows, np.arange(S), spec.n_kv_heads)
        attn = o.reshape(len(rows), Hq * dh)                    # concat heads [P3 §9]
        r = x[b, rows] + linear(attn, w["wo"])
        z = rmsnorm(r, w["ln2_g"], spec.eps)
        F, extra = _ffn(z, w, spec)
        y = r + F
        for name, val in (("y", y), ("r", r), ("xhat", xhat), ("q", q[rows]), ("k", k),
                          ("v", v), ("attn", attn), ("z", z), ("f", F)):
            out[name].append(val)
        for name, val in extra.items():
            out[name].append(val)
    return {k: np.stack(v) for k, v in out.items() if v}


def layer_decode(x, k_cache, v_cache, cache_len, w, spec: LayerSpec,
                 pos_offset: int = 0) -> Dict[str, np.ndarray]:
    """One decode step ([P1 §09.1]).

    x: [B, d] new-token hidden rows; k_cache/v_cache: [B, T_max, Hkv, dh]
    holding rows 0..cache_len[b]-1 as stored (post-norm, post-RoPE keys);
    the new token is cache row cache_len[b] at position cache_len[b] +
    pos_offset and attends to all cache_len[b]+1 rows.

    The projections and the FFN take the B rows as one matrix (rows never
    interact, [P1 §03.2]); only attention is per sequence.

    Returns y [B, d], k_new/v_new [B, Hkv, dh] (the row written to the cache),
    r, attn, q, z and FFN intermediates.
    """
    x = f64(x)
    B, d = x.shape
    Hq, dh = spec.n_q_heads, spec.head_dim
    lens = np.asarray(cache_len, dtype=np.int64).reshape(B)
    xhat = rmsnorm(x, w["ln1_g"], spec.eps)
    q, k, v = _project_qkv(xhat, w, spec, lens.astype(np.float64) + pos_offset)
    attn = np.empty((B, Hq * dh))
    for b in range(B):
        L = int(lens[b])
        K = np.concatenate([f64(k_cache[b, :L]), k[b:b + 1]], axis=0)
        V = np.concatenate([f64(v_cache[b, :L]), v[b:b + 1]], axis=0)
        o = attention(q[b:b + 1], K, V, np.array([L]), np.arange(L + 1), spec.n_kv_heads)
        attn[b] = o.reshape(Hq * dh)                                  # concat heads [P3 §9]
    r = x + linear(attn, w["wo"])
    z = rmsnorm(r, w["ln2_g"], spec.eps)
    F, extra = _ffn(z, w, spec)
    out = {"y": r + F, "r": r, "xhat": xhat, "q": q, "k_new": k, "v_new": v, "attn": attn,
           "z": z, "f": F}
    out.update(extra)
    return out


def layer_prefill_chunk(x_new, k_cache, v_cache, cache_len, w, spec: LayerSpec,
                        pos_offset: int = 0) -> Dict[str, np.ndarray]:
    """Prefill of new tokens over an existing cache prefix, one sequence
    ([P1 §09.1]: the cache grows by the new rows; [P3 §8]: causal).

    x_new: [S, d] new-token hidden rows; k_cache/v_cache: [T_max, Hkv, dh]
    holding rows 0..cache_len-1 as stored (post-norm, post-RoPE keys). New
    row t sits at cache row cache_len + t, position cache_len + t +
    pos_offset, and attends to cache rows 0..cache_len-1 and new rows 0..t.

    The projections and the FFN take the S rows as one matrix (rows never
    interact, [P1 §03.2]). Returns y, r, q, attn, z, f [S, ...] and the new
    cache rows k_new, v_new [S, Hkv, dh].
    """
    x = f64(x_new)
    S, d = x.shape
    Hq, dh = spec.n_q_heads, spec.head_dim
    P = int(cache_len)
    pos = np.arange(S, dtype=np.float64) + P + pos_offset
    xhat = rmsnorm(x, w["ln1_g"], spec.eps)
    q, k, v = _project_qkv(xhat, w, spec, pos)
    K = np.concatenate([f64(k_cache[:P]), k], axis=0)
    V = np.concatenate([f64(v_cache[:P]), v], axis=0)
    o = attention(q, K, V, np.arange(S) + P, np.arange(P + S), spec.n_kv_heads)
    attn = o.reshape(S, Hq * dh)                                      # concat heads [P3 §9]
    r = x + linear(attn, w["wo"])
    z = rmsnorm(r, w["ln2_g"], spec.eps)
    F, extra = _ffn(z, w, spec)
    out = {"y": r + F, "r": r, "q": q, "k_new": k, "v_new": v, "attn": attn, "z": z, "f": F}
    out.update(extra)
    return out

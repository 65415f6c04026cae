"""Parameter, FLOP and byte accounting of one layer, written from the pages'
formulas. TEST INFRASTRUCTURE (see ``qlayer_ref``); ``bench.py`` reads the
algorithmic work of a workload from here only for its ``cpu_baseline`` leg.

[P1] "Qwen2.5-7B 结构拆解": §03.4 (2mkn vs m·n·(2k-1)), §03.8 (per-token
     FLOPs = 2 x matmul params), §05.4-§05.5 (attention FLOPs), §09.1 (KV
     bytes), §10.1 (shared expert), §11 (parameter formulas), §11.1 (MoE).
[P3] "推理系统 03：逐项算清一个真实 Qwen3 Transformer 层" §11-§12.
[P4] "Transformer 的 Infra 视角" §3.
[P5] "第七章 模型容量与参数量推导" §1-§3.
"""
from __future__ import annotations


def gemm_flops(m: int, k: int, n: int) -> int:
    """Conventional count 2·m·k·n ([P1 §03.4])."""
    return 2 * m * k * n


def gemm_exact_ops(m: int, k: int, n: int) -> int:
    """k multiplies and k-1 adds per output: m·n·(2k-1) ([P1 §03.4])."""
    return m * n * (2 * k - 1)


def attn_params(d: int, q_dim: int, kv_dim: int) -> int:
    """Q, K, V, O projections: d·q + 2·d·kv + q·d ([P4 §3]; [P5 §1])."""
    return d * q_dim + 2 * d * kv_dim + q_dim * d


def qkv_bias_params(q_dim: int, kv_dim: int) -> int:
    """q + 2·kv ([P1 §11])."""
    return q_dim + 2 * kv_dim


def mlp_params(d: int, f: int) -> int:
    """SwiGLU: 3·d·f ([P1 §11]; [P3 §11])."""
    return 3 * d * f


def norm_params(d: int) -> int:
    """Two RMSNorm gammas per layer ([P1 §11])."""
    return 2 * d


def model_params(n_layers: int, layer_params: int, vocab: int, d: int,
                 tied: bool) -> int:
    """L·layer + (1 or 2)·V·d + d (final norm) ([P1 §11]; [P5 §2])."""
    return n_layers * layer_params + (1 if tied else 2) * vocab * d + d


def moe_block_params(d: int, n_experts: int, mf: int, sf: int = 0) -> int:
    """router d·e + experts e·3·d·mf (+ shared 3·d·sf + d) ([P1 §11.1])."""
    p = d * n_experts + n_experts * 3 * d * mf
    if sf:
        p += 3 * d * sf + d
    return p


def moe_active_params(d: int, n_experts: int, top_k: int, mf: int, sf: int = 0) -> int:
    """router d·e + k·3·d·mf (+ shared) ([P1 §11.1])."""
    p = d * n_experts + top_k * 3 * d * mf
    if sf:
        p += 3 * d * sf + d
    return p


def experts_touched(n_experts: int, top_k: int, batch: int) -> float:
    """Expected distinct experts under uniform routing: e·(1-(1-k/e)^B)
    ([P1 §11.1])."""
    return n_experts * (1.0 - (1.0 - top_k / n_experts) ** batch)


def attn_prefill_flops_half(S: int, n_q_heads: int, head_dim: int) -> float:
    """[P1 §05.4]: 4·dh·S² per head, × Hq, ÷ 2 for the causal triangle."""
    return 4 * head_dim * S * S * n_q_heads / 2


def attn_prefill_flops_exact(S: int, n_q_heads: int, head_dim: int) -> int:
    """Visible (query, key) pairs S(S+1)/2, 4·dh FLOPs per pair per head
    (QK^T and PV, [P1 §05.4])."""
    return 4 * head_dim * n_q_heads * S * (S + 1) // 2


def attn_decode_flops(T: int, n_q_heads: int, head_dim: int) -> int:
    """One query over T keys: 4·dh·T per head ([P1 §05.5])."""
    return 4 * head_dim * n_q_heads * T


def kv_bytes_per_token(n_kv_heads: int, head_dim: int, dtype_bytes: int = 2) -> int:
    """K and V rows of one layer: 2·Hkv·dh·bytes ([P1 §09.1]; [P3 §12])."""
    return 2 * n_kv_heads * head_dim * dtype_bytes


def dense_layer_gemm_flops(tokens: int, d: int, q_dim: int, kv_dim: int, f: int) -> dict:
    """2·m·k·n for each weight GEMM of a dense layer at m = tokens."""
    return {
        "qkv": gemm_flops(tokens, d, q_dim + 2 * kv_dim),
        "o": gemm_flops(tokens, q_dim, d),
        "gate_up": gemm_flops(tokens, d, 2 * f),
        "down": gemm_flops(tokens, f, d),
    }

"""Layer shapes and workloads used by the tests and the benchmark.

Pure data: no arithmetic of the layer lives here. The dimensions are the ones
the pages print for each model:

* Qwen2.5-7B -- "Qwen2.5-7B 结构拆解" (daleiyang.github.io), §04 and §11
  (d=3584, 28 query heads, 4 KV heads, head_dim 128, f=18944, QKV bias).
* Qwen3-8B -- "推理系统 03：逐项算清一个真实 Qwen3 Transformer 层"
  (marvinlee.cn), opening paragraph and §4-§5 (d=4096, 32/8 heads, f=12288,
  no bias, QK-norm).
* Qwen3-30B-A3B -- "MoE 初步：参数量计算、Qwen3-30B-A3B、GQA 与 Sparse MoE"
  (hqhq1025.github.io), configuration table and "Sparse MoE 架构详解"
  (d=2048, 32/4 heads, head_dim 128, 128 experts of width 768, top-8,
  norm_topk_prob true).
* The toy layer -- same Qwen3 page, §1 (3 positions, d=4, 2 query heads,
  1 KV head, head_dim 2, MLP width 6, gamma=1, eps=1e-6).
* Qwen3-32B -- "MoE 初步" configuration table (d=5120, 64 query heads,
  8 KV groups, head_dim 128, FFN 25600; QK-norm as every Qwen3 layer).
* Qwen2-57B-A14B -- "Qwen2.5-7B 结构拆解" §10-§10.2: the Qwen2.5-7B attention
  unchanged (d=3584, 28/4 heads, QKV bias), the MLP replaced by 64 SwiGLU
  experts of width 2560, top-8 with raw (not renormalised) probabilities,
  plus one shared SwiGLU expert of width 20480 scaled by sigmoid(x W_sg).
* A Mixtral-like layer -- "第七章 模型容量与参数量推导" §3 gives only the
  routing (8 FFN experts per layer, 2 chosen per token); the rest is
  Qwen3-8B's attention (d=4096, 32/8 heads, QK-norm) and experts of width
  4096.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class LayerConfig:
    name: str
    d: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int                 # dense SwiGLU width f, or per-expert width mf
    n_experts: int = 0           # 0 -> dense SwiGLU FFN
    top_k: int = 0
    norm_topk_prob: bool = True
    shared_ffn_dim: int = 0      # width of an always-on shared SwiGLU expert (0: none)
    qkv_bias: bool = False
    qk_norm: bool = False
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    dtype: str = "bf16"          # "bf16" (bf16 storage, fp32 math) or "f32"
    # distributions of the synthetic tensors (std of a normal)
    w_std: float = 0.02
    b_std: float = 0.02
    gamma_mean: float = 1.0
    gamma_std: float = 0.05
    router_std: float = 0.05
    x_std: float = 1.0
    cache_std: float = 1.0

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def is_moe(self) -> bool:
        return self.n_experts > 0


@dataclass(frozen=True)
class Workload:
    cfg_id: int
    index: int          # workload number inside the config (seed = 1000*cfg + index)
    kind: str           # "prefill" or "decode"
    batch: int
    seq: int            # prefill: tokens per sequence; decode: cache length before the step
    label: str = ""

    @property
    def seed(self) -> int:
        return 1000 * self.cfg_id + self.index

    @property
    def tokens(self) -> int:
        return self.batch * self.seq if self.kind == "prefill" else self.batch


TOY = LayerConfig(
    name="toy-f32", d=4, n_q_heads=2, n_kv_heads=1, head_dim=2, ffn_dim=6,
    dtype="f32", w_std=0.5, b_std=0.0, gamma_mean=1.0, gamma_std=0.0,
    x_std=0.5, cache_std=0.5,
)

QWEN25_7B = LayerConfig(
    name="qwen2.5-7b", d=3584, n_q_heads=28, n_kv_heads=4, head_dim=128,
    ffn_dim=18944, qkv_bias=True,
)

QWEN3_8B = LayerConfig(
    name="qwen3-8b", d=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
    ffn_dim=12288, qk_norm=True,
)

QWEN3_30B_A3B = LayerConfig(
    name="qwen3-30b-a3b", d=2048, n_q_heads=32, n_kv_heads=4, head_dim=128,
    ffn_dim=768, n_experts=128, top_k=8, norm_topk_prob=True, qk_norm=True,
)

QWEN3_32B = LayerConfig(
    name="qwen3-32b", d=5120, n_q_heads=64, n_kv_heads=8, head_dim=128,
    ffn_dim=25600, qk_norm=True,
)

QWEN2_57B_A14B = LayerConfig(
    name="qwen2-57b-a14b", d=3584, n_q_heads=28, n_kv_heads=4, head_dim=128,
    ffn_dim=2560, n_experts=64, top_k=8, norm_topk_prob=False, shared_ffn_dim=20480,
    qkv_bias=True,
)

MIXTRAL_LIKE = LayerConfig(
    name="mixtral-like", d=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
    ffn_dim=4096, n_experts=8, top_k=2, norm_topk_prob=True, qk_norm=True,
)

CONFIGS = {1: TOY, 2: QWEN25_7B, 3: QWEN25_7B, 4: QWEN3_8B, 5: QWEN3_30B_A3B,
           6: QWEN3_32B, 7: MIXTRAL_LIKE, 8: QWEN2_57B_A14B}

WORKLOADS = {
    1: [Workload(1, 1, "prefill", 1, 3, "toy prefill T=3")],
    2: [Workload(2, 1, "decode", 1, 1024, "qwen2.5-7b decode B=1 cache=1024"),
        Workload(2, 2, "decode", 32, 1024, "qwen2.5-7b decode B=32 cache=1024")],
    3: [Workload(3, 1, "prefill", 1, 1024, "qwen2.5-7b prefill B=1 S=1024"),
        Workload(3, 2, "prefill", 4, 512, "qwen2.5-7b prefill B=4 S=512")],
    4: [Workload(4, 1, "prefill", 1, 2048, "qwen3-8b prefill B=1 S=2048"),
        Workload(4, 2, "decode", 64, 4096, "qwen3-8b decode B=64 cache=4096")],
    5: [Workload(5, 1, "prefill", 1, 4096, "qwen3-30b-a3b prefill 4096 tokens"),
        Workload(5, 2, "decode", 128, 4096, "qwen3-30b-a3b decode B=128 cache=4096"),
        Workload(5, 3, "decode", 128, 1024, "qwen3-30b-a3b decode B=128 cache=1024")],
    # shape variants beyond the graded configs
    6: [Workload(6, 1, "prefill", 1, 2048, "qwen3-32b prefill B=1 S=2048"),
        Workload(6, 2, "decode", 32, 4096, "qwen3-32b decode B=32 cache=4096")],
    7: [Workload(7, 1, "prefill", 1, 2048, "mixtral-like prefill 2048 tokens"),
        Workload(7, 2, "decode", 64, 2048, "mixtral-like decode B=64 cache=2048")],
    8: [Workload(8, 1, "prefill", 1, 2048, "qwen2-57b-a14b prefill 2048 tokens"),
        Workload(8, 2, "decode", 64, 1024, "qwen2-57b-a14b decode B=64 cache=1024")],
}


def weight_seed(cfg_id: int) -> int:
    """Seed of a config's weights; inputs use 1000*cfg + workload index."""
    return 1000 * cfg_id


def with_dims(cfg: LayerConfig, **kw) -> LayerConfig:
    return replace(cfg, **kw)

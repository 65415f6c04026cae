/*
 * qlayer.h -- C ABI of a forward pass of one Qwen-style pre-norm decoder layer
 * on an AMD Instinct MI355X (gfx950).
 *
 * The layer computes, per token row ("推理系统 03：逐项算清一个真实 Qwen3
 * Transformer 层", §2; "Qwen2.5-7B 结构拆解", §02):
 *
 *     R = X + Attn(RMSNorm1(X))          Y = R + FFN(RMSNorm2(R))
 *
 * Attn = Q/K/V projections (+ optional QKV bias, "Qwen2.5-7B 结构拆解" §11),
 * optional per-head QK-RMSNorm ("推理系统 03" §5), rotate_half RoPE with
 * omega_r = theta^(-2r/dh) ("推理系统 03" §6), causal GQA softmax attention
 * with head h reading KV head floor(h / (Hq/Hkv)) ("推理系统 03" §7-§9), head
 * concatenation and the O projection. FFN is either a dense SwiGLU
 * (SiLU(gate) * up, then down; "推理系统 03" §10) or a top-k sparse MoE of
 * SwiGLU experts with gate weights softmax-renormalised over the k selected
 * logits ("MoE 初步：参数量计算、Qwen3-30B-A3B、GQA 与 Sparse MoE", Router 机制,
 * MoE 的最终输出; "Qwen2.5-7B 结构拆解" §10.2).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are row-major and dense. Weights use the [out, in] storage
 *   convention and are applied as y = x W^T ("Qwen2.5-7B 结构拆解" §03.1).
 * - Every data pointer is a DEVICE pointer on the current HIP device unless
 *   stated otherwise. The caller owns all of them: weights must outlive the
 *   handle, activations / caches must outlive the call's stream work. The
 *   library never frees or reallocates caller memory.
 * - Element type: QL_BF16 -> bfloat16 weights, inputs, outputs and caches,
 *   fp32 arithmetic, one round-to-nearest-even rounding when a bf16 tensor is
 *   stored; the residual stream between the two halves, the RMSNorm1 output
 *   and the attention output are kept in fp32 (the last two enter their bf16
 *   MFMA projections as a bf16 hi + lo pair), and so are, in a dense
 *   prefill, the RMSNorm2 output and the SwiGLU hidden. QL_F32 -> fp32
 *   storage and arithmetic (small shapes only, generic kernels).
 * - Work is enqueued on `stream` (a hipStream_t; NULL = default stream) with
 *   no host synchronisation and no device-to-host copy. Argument errors
 *   return before anything is enqueued. A failed launch returns QL_EHIP;
 *   faults inside kernels surface at the caller's next synchronisation.
 * - A handle owns one device workspace. Calls on one handle must not overlap
 *   in time (issue them on one stream, or synchronise between streams).
 * - On any non-OK status qlayer_last_error() returns a message (thread-local).
 */
#ifndef QLAYER_H
#define QLAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QLAYER_ABI_VERSION 2

typedef enum {
  QL_OK = 0,
  QL_EINVAL = -1,        /* bad argument: NULL pointer, non-positive size, size above the handle's maximum */
  QL_EUNSUPPORTED = -2,  /* shape/dtype combination no kernel of this build handles */
  QL_ENOMEM = -3,        /* workspace allocation failed at create */
  QL_EHIP = -4,          /* a HIP runtime call or launch failed */
  QL_ECACHE_FULL = -5    /* decode: cache_len[b] + 1 > T_max (checked when a host copy is given) */
} ql_status;

typedef enum { QL_BF16 = 0, QL_F32 = 1 } ql_dtype;

/* Layer hyper-parameters, named as in a model's config.json ("Qwen2.5-7B
 * 结构拆解" §11; "MoE 初步" configuration table).
 *
 * d            hidden size
 * n_q_heads    query heads Hq;  n_kv_heads: KV heads Hkv (Hq % Hkv == 0)
 * head_dim     dh (QL_BF16 requires 128; QL_F32 a power of two in [2, 128])
 * ffn_dim      dense SwiGLU width f, or per-expert width mf when n_experts > 0
 * n_experts    0 -> dense SwiGLU FFN; otherwise E routed experts (QL_BF16 only)
 * top_k        experts per token (1 <= top_k <= min(E, 32))
 * norm_topk_prob  1: gate weights = softmax over the k selected logits;
 *                 0: raw probabilities of a softmax over all E logits
 * qkv_bias     1: bq/bk/bv are added after the projections
 * qk_norm      1: per-head RMSNorm of Q and K over dh with shared gammas
 * rms_eps      epsilon of every RMSNorm (including QK-norm)
 * rope_theta   RoPE base theta
 * dtype        ql_dtype of weights, activations and caches
 * max_tokens   largest B*S of qlayer_prefill and largest N of qlayer_moe_ffn
 * max_batch    largest B of qlayer_decode
 * shared_ffn_dim  width sf of an always-on shared SwiGLU expert whose output is
 *              scaled per token by sigmoid(z W_sg^T) and added to the routed
 *              sum (Qwen2 MoE, "Qwen2.5-7B 结构拆解" §10.1-§10.2); 0 = none.
 *              MoE layers only; sf % 128 == 0.
 *
 * QL_BF16 shape limits: head_dim == 128, d % 256 == 0, Hq and Hkv even,
 * ffn_dim % 128 == 0, Hq/Hkv <= 16, max_batch <= 1024, and with experts
 * n_experts <= 256.
 */
typedef struct {
  int d;
  int n_q_heads;
  int n_kv_heads;
  int head_dim;
  int ffn_dim;
  int n_experts;
  int top_k;
  int norm_topk_prob;
  int qkv_bias;
  int qk_norm;
  float rms_eps;
  float rope_theta;
  int dtype;
  int max_tokens;
  int max_batch;
  int shared_ffn_dim;
} ql_config;

/* Device pointers to the layer's weights, all in the config dtype, [out, in]:
 *   ln1_g[d], ln2_g[d]                      RMSNorm gammas
 *   wq[Hq*dh, d], wk[Hkv*dh, d], wv[Hkv*dh, d], wo[d, Hq*dh]
 *   bq[Hq*dh], bk[Hkv*dh], bv[Hkv*dh]       only when qkv_bias (else NULL)
 *   q_norm_g[dh], k_norm_g[dh]              only when qk_norm (else NULL)
 *   dense: w_gate[f, d], w_up[f, d], w_down[d, f]
 *   MoE:   w_router[E, d], we_gate[E, mf, d], we_up[E, mf, d], we_down[E, d, mf]
 *   shared expert (shared_ffn_dim sf > 0): ws_gate[sf, d], ws_up[sf, d],
 *          ws_down[d, sf], w_shared_gate[1, d] (W_sg, no bias)
 */
typedef struct {
  const void *ln1_g, *ln2_g;
  const void *wq, *wk, *wv, *wo;
  const void *bq, *bk, *bv;
  const void *q_norm_g, *k_norm_g;
  const void *w_gate, *w_up, *w_down;
  const void *w_router, *we_gate, *we_up, *we_down;
  const void *ws_gate, *ws_up, *ws_down, *w_shared_gate;
} ql_weights;

typedef struct ql_handle ql_handle;

/* Validates the config and the weight pointers, allocates the workspace for
 * max_tokens / max_batch rows on the current device and returns a handle.
 * Synchronous. Errors: QL_EINVAL, QL_EUNSUPPORTED, QL_ENOMEM, QL_EHIP. */
ql_status qlayer_create(const ql_config* cfg, const ql_weights* w, ql_handle** out);

/* Frees the workspace (synchronises the device first). NULL is a no-op. */
ql_status qlayer_destroy(ql_handle* h);

/* Bytes of device workspace the handle holds. */
size_t qlayer_workspace_bytes(const ql_handle* h);

/* Prefill: the full forward of B independent sequences of S tokens
 * ("Qwen2.5-7B 结构拆解" §09.1: prefill writes all S cache rows at once).
 *
 * x        [B, S, d]                input hidden rows
 * pos_offset  RoPE position of sequence row s is s + pos_offset
 * k_cache, v_cache  [B, T_max, Hkv, dh]  rows 0..S-1 of each sequence are
 *          written: K after QK-norm and RoPE, V as projected ("推理系统 03"
 *          §12); other rows are untouched. Attention reads only these S rows.
 * T_max    rows per sequence in the caches (S <= T_max; one sequence's K or V
 *          cache, T_max * Hkv * dh * 2 bytes, must stay below 4 GiB and T_max
 *          below 2^24 on the bf16 path)
 * y        [B, S, d]                output hidden rows (may not alias x)
 * Errors: QL_EINVAL (NULL, B*S > max_tokens, S > T_max), QL_EUNSUPPORTED
 * (T_max beyond the limit above), QL_EHIP. */
ql_status qlayer_prefill(ql_handle* h, const void* x, int B, int S, int pos_offset,
                         void* k_cache, void* v_cache, int T_max, void* y, void* stream);

/* Prefill of new rows over existing cache prefixes, for a batch of
 * sequences of different lengths (chunked prefill: "Qwen2.5-7B 结构拆解"
 * §09.1, the cache grows by the new rows; causal as in "推理系统 03" §8).
 *
 * x          [N, d]  the new rows of every sequence, concatenated
 * seq_start  [B + 1] int32 DEVICE: sequence b's new rows are x rows
 *            seq_start[b] .. seq_start[b + 1] - 1 (seq_start[0] = 0,
 *            non-decreasing, N = seq_start[B]; a sequence may have none)
 * cache_len  [B] int32 DEVICE: rows 0 .. cache_len[b] - 1 of sequence b's
 *            cache hold earlier keys/values (keys normed and rotated). New
 *            row t is written at cache row cache_len[b] + t, has RoPE position
 *            cache_len[b] + t + pos_offset and attends to cache rows
 *            0 .. cache_len[b] + t. The caller advances cache_len afterwards.
 * seq_start_host, cache_len_host  HOST copies of both (required): the
 *            launch shapes come from them and the bounds are checked there.
 * k_cache, v_cache [B, T_max, Hkv, dh];  y [N, d] (may not alias x); T_max
 *            within the limit of qlayer_prefill
 * Errors: QL_EINVAL (NULL, bad seq_start, N = 0 or > max_tokens),
 * QL_ECACHE_FULL (cache_len[b] + new rows > T_max), QL_EUNSUPPORTED
 * (QL_F32, T_max beyond the limit), QL_EHIP. */
ql_status qlayer_prefill_varlen(ql_handle* h, const void* x, int B, const int* seq_start,
                                const int* cache_len, const int* seq_start_host,
                                const int* cache_len_host, int pos_offset, void* k_cache,
                                void* v_cache, int T_max, void* y, void* stream);

/* Decode: one new token per sequence ("Qwen2.5-7B 结构拆解" §09.1).
 *
 * x          [B, d]     hidden row of the new token of each sequence
 * cache_len  [B] int32, DEVICE: rows 0..cache_len[b]-1 of sequence b hold
 *            earlier keys/values (keys already normed and rotated). The new
 *            K/V row is written at row cache_len[b]; the token's RoPE position
 *            is cache_len[b] + pos_offset; it attends to rows 0..cache_len[b].
 *            The caller advances cache_len afterwards.
 * cache_len_host  optional HOST copy of cache_len (may be NULL); when given,
 *            any cache_len[b] < 0 or cache_len[b] + 1 > T_max returns
 *            QL_ECACHE_FULL before any launch. Without it the bound is a
 *            precondition; kernels still never touch rows outside [0, T_max)
 *            and write NaN outputs for a sequence whose length is out of range.
 * y          [B, d]     output hidden rows
 * Errors: QL_EINVAL (NULL, B > max_batch), QL_ECACHE_FULL, QL_EHIP. */
ql_status qlayer_decode(ql_handle* h, const void* x, int B, const int* cache_len,
                        const int* cache_len_host, int pos_offset, void* k_cache,
                        void* v_cache, int T_max, void* y, void* stream);

/* One decode step through a stack of L layers (a model's trunk, "Qwen2.5-7B
 * 结构拆解" §02 and §11: the layers run one after another, each reading the
 * previous one's output rows and its own KV cache).
 *
 * layers     [L] handles (same d and dtype; B <= each max_batch)
 * x          [B, d] input rows of layer 0;  y [B, d] output rows of layer L-1
 * cache_len, cache_len_host, pos_offset, T_max  as qlayer_decode, shared by
 *            every layer (each layer appends its row at cache_len[b])
 * k_caches, v_caches  [L] HOST arrays of DEVICE pointers, layer l's caches
 *            [B, T_max, Hkv_l, dh]
 * tmp        [B, d] device scratch for the rows between layers (caller-owned;
 *            layers alternate between tmp and y so the last one writes y)
 * The whole step is enqueued on `stream` (capturable as one graph).
 * Errors: as qlayer_decode; QL_EINVAL for mismatched layers or aliasing. */
ql_status qlayer_decode_stack(ql_handle* const* layers, int L, const void* x, int B,
                              const int* cache_len, const int* cache_len_host, int pos_offset,
                              void* const* k_caches, void* const* v_caches, int T_max, void* y,
                              void* tmp, void* stream);

/* Largest workspace, in bytes, of a qlayer_decode_noalloc call. */
#define QLAYER_NOALLOC_MAX_WORKSPACE (64u << 20)

/* Decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, results and errors as qlayer_decode, with the config and
 * weights passed directly instead of a handle. The workspace is a
 * file-scope device array of QLAYER_NOALLOC_MAX_WORKSPACE bytes that every
 * GPU the library runs on holds from module load until the process ends;
 * no hipMalloc / hipFree or other allocating call is made. The array is
 * laid out afresh for each call (cfg->max_tokens and cfg->max_batch are
 * ignored; B is the call's size) and keeps the last call's contents.
 * Calls on one GPU share that GPU's array: calls that overlap in time on
 * one GPU (two streams, two threads) race and must be serialised by the
 * caller. Errors: as qlayer_decode; QL_EUNSUPPORTED also when the call's
 * workspace would exceed the array (the message gives the bytes needed). */
ql_status qlayer_decode_noalloc(const ql_config* cfg, const ql_weights* w, const void* x, int B,
                                const int* cache_len, const int* cache_len_host, int pos_offset,
                                void* k_cache, void* v_cache, int T_max, void* y, void* stream);

/* The sparse-MoE FFN half of a layer on N residual rows ("Qwen2.5-7B 结构拆解"
 * §10.2; "MoE 初步" Sparse MoE 架构详解):
 *     y = r + sum_{i<k} w_i * Expert_{idx_i}(z) [+ sigmoid(z W_sg^T) SharedExpert(z)],
 *     z = RMSNorm2(r)
 * Router logits are computed from an fp32 RMSNorm2 output; top-k order is by
 * descending logit, ties to the lower expert index; the sum runs in rank order.
 *
 * r [N, d], y [N, d] in the config dtype (QL_BF16); topk_idx [N, k] int32 and
 * topk_w [N, k] fp32 receive the routing when not NULL.
 * Errors: QL_EINVAL (NULL, N > max_tokens), QL_EUNSUPPORTED (dense handle), QL_EHIP. */
ql_status qlayer_moe_ffn(ql_handle* h, const void* r, int N, void* y, int* topk_idx,
                         float* topk_w, void* stream);

/* Optional copies of intermediate tensors, for stage-by-stage checks. Each
 * non-NULL device pointer receives, after every later prefill/decode call on
 * the handle, its tensor for the call's N rows (N = B*S or B):
 *   q      [N, Hq*dh]  dtype   queries after QK-norm and RoPE
 *   attn   [N, Hq*dh]  fp32    attention output, heads concatenated (before W_O)
 *   r      [N, d]      fp32    residual stream after the attention half
 *   z      [N, d]      fp32    RMSNorm2(r) as the FFN's GEMMs see it (the
 *                              hi + lo of a pair, or the stored value widened)
 *   h      [N, f]      fp32    dense SwiGLU hidden SiLU(gate)*up, likewise
 *                              (dense only)
 *   logits [N, E]      fp32    router logits (MoE only)
 * qlayer_moe_ffn fills the z and logits taps for its N rows.
 * Passing NULL (or a struct of NULLs) turns taps off. */
typedef struct {
  void* q;
  void* attn;
  float* r;
  void* z;
  void* h;
  float* logits;
} ql_taps;

ql_status qlayer_set_taps(ql_handle* h, const ql_taps* taps);

/* Stages of a call, for qlayer_set_stage_events. */
typedef enum {
  QL_STAGE_NONE = 0,
  QL_STAGE_RMSNORM1 = 1,     /* RMSNorm of the input rows */
  QL_STAGE_QKV = 2,          /* Q/K/V projection (+bias) */
  QL_STAGE_QKV_POST = 3,     /* QK-norm, RoPE, cache write */
  QL_STAGE_ATTENTION = 4,    /* attention core (decode: split + combine) */
  QL_STAGE_O_PROJ = 5,       /* O projection + residual */
  QL_STAGE_RMSNORM2 = 6,     /* RMSNorm of the residual rows */
  QL_STAGE_GATE_UP = 7,      /* dense gate/up + SwiGLU */
  QL_STAGE_DOWN = 8,         /* dense down + residual */
  QL_STAGE_ROUTER = 9,       /* router logits + top-k */
  QL_STAGE_PERMUTE = 10,     /* histogram, scan, scatter */
  QL_STAGE_EXPERT_GATE_UP = 11,
  QL_STAGE_EXPERT_DOWN = 12,
  QL_STAGE_COMBINE = 13,     /* weighted combine + residual */
  QL_STAGE_SHARED_GATE_UP = 14,  /* shared expert gate/up + SwiGLU */
  QL_STAGE_SHARED_DOWN = 15      /* shared expert down, gated, + residual */
} ql_stage;

/* Timing aid: after this call, every prefill / decode / moe_ffn call on the
 * handle records `start_event` on its stream immediately before the first
 * kernel of `stage` and `stop_event` immediately after its last kernel (both
 * hipEvent_t created by the caller; recorded again on every call).
 * stage = QL_STAGE_NONE (or NULL events) turns it off. Errors: QL_EINVAL. */
ql_status qlayer_set_stage_events(ql_handle* h, int stage, void* start_event, void* stop_event);

/* Thread-local description of the last non-OK status on this thread. */
const char* qlayer_last_error(void);

/* QLAYER_ABI_VERSION of the built library. */
int qlayer_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QLAYER_H */

// Host side of the C ABI declared in include/qlayer.h: argument checks, the
// per-handle device workspace and the order of kernel launches for one layer.
//
// Prefill / decode, per call on the caller's stream:
//   RMSNorm1 -> QKV projection (+bias) -> QK-norm + RoPE + cache write ->
//   attention -> O projection + residual (R, fp32) -> RMSNorm2 ->
//   dense: gate/up + SwiGLU -> down + residual (Y)
//   MoE:   router + top-k -> permutation -> grouped gate/up + SwiGLU ->
//          grouped down -> weighted combine + residual (Y)
// ("推理系统 03：逐项算清一个真实 Qwen3 Transformer 层" §2-§10; "Qwen2.5-7B 结构
// 拆解" §09.1 for the decode step and §10.2 for the MoE FFN.)
#include "../../include/qlayer.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>
#include <string>

#include "kernels.h"

namespace {

thread_local std::string g_last_error;

ql_status fail(ql_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

constexpr int kMinMoeTile = 32;
constexpr int kBigMoeTile = 128;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

}  // namespace

struct ql_handle {
  ql_config cfg;
  ql_weights w;
  int device;
  int es;  // element bytes of the config dtype
  int q_dim, kv_dim, qkv_dim, G;
  int rows;  // workspace rows: max(max_tokens, max_batch)
  char* ws;
  size_t ws_bytes;
  // workspace slices
  void* xhat;
  float* qkv;
  void* q;
  void* attn;
  float* r;
  void* z;
  float* zf;
  void* h;
  float* part_o;
  float* part_ml;
  float* inv_rms;   // [rows] RMSNorm1 1/rms handed from the QKV GEMV to attention
  void* g2part;     // split-K / stream-K partial tiles of the MFMA GEMMs
  size_t g2part_bytes;
  bool attn_hilo;   // the attention buffer holds a [hi | lo] bf16 pair (prefill)
  bool ffn_pair;    // the last call kept RMSNorm2's output (in xhat) and h as [hi | lo] pairs
  double* rope_omega;  // [head_dim / 2] RoPE frequencies
  float* logits;
  int* idx;
  float* topw;
  int* hist;
  int* blkoff;
  int* offsets;
  int* tile_expert;
  int* tile_row0;
  int* tile_rows;
  int* num_tiles;
  int* slot_token;
  int* pos_of;
  void* hm;
  float* out_slot;  // [N*k, d] expert outputs in slot order
  void* hs;         // shared expert hidden: [N, 2 sf] pair (prefill) or [N, sf]
  float* rs;        // [N, d] residual + gated shared expert output (fp32)
  int max_tiles;
  ql_taps taps;
  int ev_stage;
  hipEvent_t ev_start, ev_stop;
};

namespace {

#define QL_HIP(call)                                                                  \
  do {                                                                                \
    hipError_t e_ = (call);                                                           \
    if (e_ != hipSuccess)                                                             \
      return fail(QL_EHIP, "%s failed: %s", #call, hipGetErrorString(e_));            \
  } while (0)

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// The bf16 prefill attention addresses one sequence's cache rows with 32-bit
// offsets from 24-bit factors.
bool prefill_cache_fits(const ql_config& c, int T_max) {
  return T_max < (1 << 24) && (long long)T_max * c.n_kv_heads * c.head_dim * 2 < (1LL << 32);
}

// Stage markers for qlayer_set_stage_events.
ql_status mark(ql_handle* h, int stage, bool begin, hipStream_t s) {
  if (h->ev_stage == QL_STAGE_NONE || h->ev_stage != stage) return QL_OK;
  QL_HIP(hipEventRecord(begin ? h->ev_start : h->ev_stop, s));
  return QL_OK;
}

#define QL_STAGE(h, st, s, body)               \
  do {                                         \
    ql_status m_ = mark(h, st, true, s);       \
    if (m_ != QL_OK) return m_;                \
    body;                                      \
    m_ = mark(h, st, false, s);                \
    if (m_ != QL_OK) return m_;                \
  } while (0)

ql_status validate(const ql_config* c, const ql_weights* w) {
  if (!c || !w) return fail(QL_EINVAL, "config and weights must not be NULL");
  if (c->d <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
      c->ffn_dim <= 0)
    return fail(QL_EINVAL, "dimensions must be positive");
  if (c->n_q_heads % c->n_kv_heads)
    return fail(QL_EINVAL, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", c->n_q_heads,
                c->n_kv_heads);
  if (c->max_tokens < 0 || c->max_batch < 0 || (c->max_tokens == 0 && c->max_batch == 0))
    return fail(QL_EINVAL, "max_tokens / max_batch must be non-negative and not both 0");
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f))
    return fail(QL_EINVAL, "rms_eps must be >= 0 and rope_theta > 0");
  if (c->dtype != QL_BF16 && c->dtype != QL_F32) return fail(QL_EINVAL, "unknown dtype %d", c->dtype);
  if (!w->ln1_g || !w->ln2_g || !w->wq || !w->wk || !w->wv || !w->wo)
    return fail(QL_EINVAL, "attention weights and norm gammas must not be NULL");
  if (c->qkv_bias && (!w->bq || !w->bk || !w->bv))
    return fail(QL_EINVAL, "qkv_bias set but a bias pointer is NULL");
  if (c->qk_norm && (!w->q_norm_g || !w->k_norm_g))
    return fail(QL_EINVAL, "qk_norm set but a QK-norm gamma is NULL");
  const int G = c->n_q_heads / c->n_kv_heads;
  if (c->n_experts > 0) {
    if (c->dtype != QL_BF16) return fail(QL_EUNSUPPORTED, "MoE layers need dtype QL_BF16");
    if (c->n_experts > kMaxExperts)
      return fail(QL_EUNSUPPORTED, "n_experts must be <= %d", kMaxExperts);
    if (c->top_k < 1 || c->top_k > std::min(c->n_experts, kMaxTopK))
      return fail(QL_EINVAL, "top_k must be in [1, min(n_experts, %d)]", kMaxTopK);
    if (!w->w_router || !w->we_gate || !w->we_up || !w->we_down)
      return fail(QL_EINVAL, "MoE weights must not be NULL");
    if (c->shared_ffn_dim < 0) return fail(QL_EINVAL, "shared_ffn_dim must be >= 0");
    if (c->shared_ffn_dim > 0) {
      if (c->shared_ffn_dim % 128)
        return fail(QL_EUNSUPPORTED, "shared_ffn_dim %% 128 must be 0");
      if (!w->ws_gate || !w->ws_up || !w->ws_down || !w->w_shared_gate)
        return fail(QL_EINVAL, "shared expert weights must not be NULL");
    }
  } else {
    if (c->n_experts < 0) return fail(QL_EINVAL, "n_experts must be >= 0");
    if (c->shared_ffn_dim != 0)
      return fail(QL_EINVAL, "shared_ffn_dim needs a MoE layer (n_experts > 0)");
    if (!w->w_gate || !w->w_up || !w->w_down)
      return fail(QL_EINVAL, "dense FFN weights must not be NULL");
  }
  if (c->dtype == QL_BF16) {
    if (c->head_dim != 128) return fail(QL_EUNSUPPORTED, "QL_BF16 needs head_dim == 128");
    if (c->d % 256) return fail(QL_EUNSUPPORTED, "QL_BF16 needs d %% 256 == 0");
    if (c->n_q_heads % 2 || c->n_kv_heads % 2)
      return fail(QL_EUNSUPPORTED, "QL_BF16 needs even n_q_heads and n_kv_heads");
    if (c->ffn_dim % 128) return fail(QL_EUNSUPPORTED, "QL_BF16 needs ffn_dim %% 128 == 0");
    if (G > 16) return fail(QL_EUNSUPPORTED, "QL_BF16 needs n_q_heads / n_kv_heads <= 16");
    if (c->max_batch > 1024) return fail(QL_EUNSUPPORTED, "QL_BF16 decode needs max_batch <= 1024");
  } else {
    if (!is_pow2(c->head_dim) || c->head_dim < 2 || c->head_dim > 128)
      return fail(QL_EUNSUPPORTED, "QL_F32 needs a power-of-two head_dim in [2, 128]");
  }
  return QL_OK;
}

// Partial-tile bytes one call of M rows needs: the pair-input QKV and O
// GEMMs and the two dense FFN GEMMs (prefill: the split-K plans; decode with
// rows past the VALU GEMV: the stream-K cut). The bytes are not monotone in M
// (fewer row tiles can mean more splits), so the workspace takes the maximum
// over every M a handle accepts.
size_t gemm2_call_part_bytes(const ql_config& c, int q_dim, int qkv_dim, int M, bool decode) {
  if (M <= 0) return 0;
  size_t b = 0;
  if (!decode) {
    b = std::max(b, ql_gemm2_pair_part_bytes(M, qkv_dim, c.d));
    b = std::max(b, ql_gemm2_pair_part_bytes(M, c.d, q_dim));
    // dense FFN or shared expert: [hi | lo] pair inputs, planned as Q/K/V and O
    const int f = c.n_experts == 0 ? c.ffn_dim : c.shared_ffn_dim;
    if (f > 0) {
      b = std::max(b, ql_gemm2_pair_part_bytes(M, 2 * f, c.d));
      b = std::max(b, ql_gemm2_pair_part_bytes(M, c.d, f));
    }
    return b;
  }
  const bool gemv_attn = M <= kGemvMaxRows && ql_gemv_ok(M, qkv_dim, c.d) && ql_gemv_ok(M, c.d, q_dim);
  if (!gemv_attn) {
    b = std::max(b, ql_gemm2_decode_part_bytes(M, qkv_dim, c.d, true));
    b = std::max(b, ql_gemm2_decode_part_bytes(M, c.d, q_dim, true));
  }
  const bool gemv_ffn = M <= kGemvMaxRows && ql_gemv_ok(M, c.ffn_dim, c.d) &&
                        ql_gemv_ok(M, c.d, c.ffn_dim);
  // dense FFN past the GEMV, or the shared expert: [hi | lo] pair inputs
  const int f = c.n_experts == 0 ? (gemv_ffn ? 0 : c.ffn_dim) : c.shared_ffn_dim;
  if (f > 0) {
    b = std::max(b, ql_gemm2_decode_part_bytes(M, 2 * f, c.d, true));
    b = std::max(b, ql_gemm2_decode_part_bytes(M, c.d, f, true));
  }
  return b;
}
size_t gemm2_part_bytes(const ql_config& c, int q_dim, int qkv_dim) {
  size_t b = 0;
  for (int M = 1; M <= c.max_tokens; ++M)
    b = std::max(b, gemm2_call_part_bytes(c, q_dim, qkv_dim, M, false));
  for (int M = 1; M <= c.max_batch; ++M)
    b = std::max(b, gemm2_call_part_bytes(c, q_dim, qkv_dim, M, true));
  return b;
}

// Decode attention launch shape: about `target` waves over (key split, KV
// head, sequence); splits of `chunk` keys (a whole number of `tile`-key
// steps), the last split running to T_max (fewer than 2 chunks), so the
// longest split is about as short as the step size allows.
constexpr int kDecodeTargetWaves = 3072;      // fused-prologue kernel, 16-key steps
constexpr int kDecodeMfmaTargetWaves = 2048;  // MFMA kernel, 32-key steps
int decode_splits(int groups, int T_max, int tile, int target, int* chunk) {
  int ns = (target + groups - 1) / groups;
  ns = std::max(1, std::min({ns, kMaxDecodeSplits, T_max / tile}));
  int ch = std::max(tile, T_max / ns / tile * tile);
  int n = std::max(1, T_max / ch);
  if (n > ns) {  // rounding the chunk down would add splits: round it up
    ch = ((T_max + ns - 1) / ns + tile - 1) / tile * tile;
    n = (T_max + ch - 1) / ch;
  }
  *chunk = ch;
  return n;
}
// Upper bound of B * nsplit over every batch size (sizes the split partials).
size_t decode_split_slots(const ql_config& c) {
  const int hkv = std::max(c.n_kv_heads, 1);
  const int target = std::max(kDecodeTargetWaves, kDecodeMfmaTargetWaves);
  return (size_t)std::max(c.max_batch, 0) + (target + hkv - 1) / hkv;
}

struct Carve {
  char* base;
  size_t off = 0;
  template <class T>
  T* take(size_t bytes) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += align_up(std::max<size_t>(bytes, 1));
    return p;
  }
};

// Lays the workspace out (base == nullptr only measures it). exact_rows > 0
// sizes the GEMM partials for a decode of exactly that many rows (the
// allocation-free entry point lays its array out per call) instead of every
// row count the handle accepts.
size_t layout(ql_handle* h, char* base, int exact_rows = 0) {
  const ql_config& c = h->cfg;
  const size_t N = (size_t)h->rows;
  const size_t es = (size_t)h->es;
  Carve k{base};
  h->xhat = k.take<void>(N * c.d * 4);  // [hi | lo] bf16 pair of the fp32 RMSNorm1 output
  h->qkv = k.take<float>(N * h->qkv_dim * 4);
  h->q = k.take<void>(N * h->q_dim * es);
  h->attn = k.take<void>(N * h->q_dim * 4);  // [hi | lo] bf16 pair, or fp32 (GEMV decode)
  h->r = k.take<float>(N * c.d * 4);
  h->z = k.take<void>(N * c.d * es);
  const size_t slots = decode_split_slots(c);
  h->part_o = k.take<float>(slots * c.n_q_heads * c.head_dim * 4);
  h->part_ml = k.take<float>(slots * c.n_q_heads * 2 * 4);
  h->rope_omega = k.take<double>((size_t)std::max(c.head_dim / 2, 1) * 8);
  h->inv_rms = k.take<float>(N * 4);
  if (c.dtype == QL_BF16 && !base)
    h->g2part_bytes = exact_rows > 0
                          ? gemm2_call_part_bytes(c, h->q_dim, h->qkv_dim, exact_rows, true)
                          : gemm2_part_bytes(c, h->q_dim, h->qkv_dim);
  h->g2part = c.dtype == QL_BF16 ? k.take<void>(h->g2part_bytes) : nullptr;
  if (c.n_experts > 0) {
    const size_t E = c.n_experts, K = c.top_k, NK = N * K;
    const size_t nblk = (N + 255) / 256;
    h->max_tiles = (int)((NK + kMinMoeTile - 1) / kMinMoeTile + E);
    h->zf = k.take<float>(N * c.d * 4);
    h->logits = k.take<float>(N * (E + (c.shared_ffn_dim > 0 ? 1 : 0)) * 4);
    h->idx = k.take<int>(NK * 4);
    h->topw = k.take<float>(NK * 4);
    h->hist = k.take<int>(nblk * E * 4);
    h->blkoff = k.take<int>(nblk * E * 4);
    h->offsets = k.take<int>((E + 1) * 4);
    h->tile_expert = k.take<int>(h->max_tiles * 4);
    h->tile_row0 = k.take<int>(h->max_tiles * 4);
    h->tile_rows = k.take<int>(h->max_tiles * 4);
    h->num_tiles = k.take<int>(4);
    h->slot_token = k.take<int>(NK * 4);
    h->pos_of = k.take<int>(NK * 4);
    h->hm = k.take<void>(NK * c.ffn_dim * 4);  // [hi | lo] bf16 pair, or fp32
    h->out_slot = k.take<float>(NK * c.d * 4);
    if (c.shared_ffn_dim > 0) {
      h->hs = k.take<void>(N * 2 * (size_t)c.shared_ffn_dim * 2);
      h->rs = k.take<float>(N * c.d * 4);
    }
  } else {
    h->h = k.take<void>(N * c.ffn_dim * es * (c.dtype == QL_BF16 ? 2 : 1));  // bf16: [hi | lo]
  }
  return k.off;
}

float scale_log2(int dh) { return 1.4426950408889634f / std::sqrt((float)dh); }

ql_status copy_logits(ql_handle* h, int N, float* dst, hipStream_t s);

ql_status copy_taps(ql_handle* h, int N, hipStream_t s) {
  const ql_config& c = h->cfg;
  const size_t es = h->es;
  const bool f32 = c.dtype == QL_F32;
  if (h->taps.q)
    QL_HIP(hipMemcpyAsync(h->taps.q, h->q, (size_t)N * h->q_dim * es, hipMemcpyDeviceToDevice, s));
  if (h->taps.attn) {
    if (h->attn_hilo)
      QL_HIP(ql_hilo_to_f32(static_cast<const bf16*>(h->attn), N, h->q_dim,
                            static_cast<float*>(h->taps.attn), s));
    else
      QL_HIP(hipMemcpyAsync(h->taps.attn, h->attn, (size_t)N * h->q_dim * 4,
                            hipMemcpyDeviceToDevice, s));
  }
  if (h->taps.r)
    QL_HIP(hipMemcpyAsync(h->taps.r, h->r, (size_t)N * c.d * 4, hipMemcpyDeviceToDevice, s));
  // z and h taps are fp32: the pair's hi + lo, or the stored value widened
  if (h->taps.z) {
    float* tz = static_cast<float*>(h->taps.z);
    if (h->ffn_pair)
      QL_HIP(ql_hilo_to_f32(static_cast<const bf16*>(h->xhat), N, c.d, tz, s));
    else if (c.n_experts > 0)
      QL_HIP(hipMemcpyAsync(tz, h->zf, (size_t)N * c.d * 4, hipMemcpyDeviceToDevice, s));
    else if (f32)
      QL_HIP(hipMemcpyAsync(tz, h->z, (size_t)N * c.d * 4, hipMemcpyDeviceToDevice, s));
    else
      QL_HIP(ql_bf16_to_f32(static_cast<const bf16*>(h->z), (size_t)N * c.d, tz, s));
  }
  if (h->taps.h && c.n_experts == 0) {
    float* th = static_cast<float*>(h->taps.h);
    if (h->ffn_pair)
      QL_HIP(ql_hilo_to_f32(static_cast<const bf16*>(h->h), N, c.ffn_dim, th, s));
    else if (f32)
      QL_HIP(hipMemcpyAsync(th, h->h, (size_t)N * c.ffn_dim * 4, hipMemcpyDeviceToDevice, s));
    else
      QL_HIP(ql_bf16_to_f32(static_cast<const bf16*>(h->h), (size_t)N * c.ffn_dim, th, s));
  }
  if (h->taps.logits && c.n_experts > 0) {
    ql_status st = copy_logits(h, N, h->taps.logits, s);
    if (st != QL_OK) return st;
  }
  return QL_OK;
}

// y = resid + MoE(z). RMSNorm2 of the residual rows is in zf (fp32: the
// router and the 32-row expert tiles) and in h->xhat as a [hi | lo] bf16
// pair (the 128-row expert tiles and the shared expert). `decode`: the
// shared expert runs on the decode tiles.
ql_status moe_core(ql_handle* h, int N, const void* resid, int resid_is_f32, bf16* y,
                   bool decode, hipStream_t s) {
  const ql_config& c = h->cfg;
  const ql_weights& w = h->w;
  const int sf = c.shared_ffn_dim;
  RouterArgs ra{};
  ra.zf = h->zf;
  ra.wr = static_cast<const bf16*>(w.w_router);
  ra.w_extra = sf > 0 ? static_cast<const bf16*>(w.w_shared_gate) : nullptr;  // logit column E
  ra.n_extra = sf > 0 ? 1 : 0;
  ra.N = N;
  ra.d = c.d;
  ra.E = c.n_experts;
  ra.k = c.top_k;
  ra.norm_topk = c.norm_topk_prob;
  ra.logits = h->logits;
  ra.idx = h->idx;
  ra.w = h->topw;
  QL_STAGE(h, QL_STAGE_ROUTER, s, QL_HIP(ql_router_topk(ra, s)));

  // Expert tiles: 128 token rows on the 8-wave MFMA tiles when experts see
  // many rows (the prefill), 32 rows on the small-tile kernel for
  // decode-sized batches. (A tile's stages cost the same however few of its
  // rows are live; around 256 rows per expert, 256-row tiles leave a third
  // of the tile rows empty, 128-row tiles a fifth.)
  const bool big = (long long)N * c.top_k >= 64LL * c.n_experts;
  const int bm = big ? kBigMoeTile : kMinMoeTile;
  const int max_tiles = (int)(((long long)N * c.top_k + bm - 1) / bm + c.n_experts);
  PermuteArgs pa{};
  pa.idx = h->idx;
  pa.N = N;
  pa.k = c.top_k;
  pa.E = c.n_experts;
  pa.bm = bm;
  pa.hist = h->hist;
  pa.blkoff = h->blkoff;
  pa.offsets = h->offsets;
  pa.tile_expert = h->tile_expert;
  pa.tile_row0 = h->tile_row0;
  pa.tile_rows = h->tile_rows;
  pa.num_tiles = h->num_tiles;
  pa.slot_token = h->slot_token;
  pa.pos_of = h->pos_of;
  QL_STAGE(h, QL_STAGE_PERMUTE, s, QL_HIP(ql_moe_permute(pa, s)));

  // The experts see z at fp32 precision and keep h and their outputs so:
  // 128-row tiles read the [hi | lo] pair of z (x-hat buffer), hi and lo
  // rows sharing each weight tile, and store h as a pair; 32-row tiles stage
  // fp32 z and h as pairs themselves. Outputs are fp32 in slot order.
  const bf16* z2 = static_cast<const bf16*>(h->xhat);
  const bf16* wg = static_cast<const bf16*>(w.we_gate);
  const bf16* wu = static_cast<const bf16*>(w.we_up);
  const bf16* wd = static_cast<const bf16*>(w.we_down);
  if (big) {
    bf16* hm = static_cast<bf16*>(h->hm);
    QL_STAGE(h, QL_STAGE_EXPERT_GATE_UP, s,
             QL_HIP(ql_gemm2_moe_gu(z2, h->slot_token, wg, wu, c.ffn_dim, c.d, h->tile_expert,
                                    h->tile_row0, h->tile_rows, h->num_tiles, max_tiles, bm, hm,
                                    s)));
    QL_STAGE(h, QL_STAGE_EXPERT_DOWN, s,
             QL_HIP(ql_gemm2_moe_down(hm, wd, c.ffn_dim, c.d, h->tile_expert, h->tile_row0,
                                      h->tile_rows, h->num_tiles, max_tiles, bm, h->out_slot, s)));
  } else {
    float* hm = static_cast<float*>(h->hm);
    QL_STAGE(h, QL_STAGE_EXPERT_GATE_UP, s,
             QL_HIP(ql_gemm_moe_gu(h->zf, h->slot_token, wg, wu, c.ffn_dim, c.d, h->tile_expert,
                                   h->tile_row0, h->tile_rows, h->num_tiles, max_tiles, hm, s)));
    QL_STAGE(h, QL_STAGE_EXPERT_DOWN, s,
             QL_HIP(ql_gemm_moe_down(hm, wd, c.ffn_dim, c.d, h->tile_expert, h->tile_row0,
                                     h->tile_rows, h->num_tiles, max_tiles, h->out_slot, s)));
  }
  if (sf > 0) {
    // Shared expert ("Qwen2.5-7B 结构拆解" §10.1): SwiGLU of width sf on every
    // row from the pair of z, h_s kept as a pair, then rs = resid +
    // sigmoid(gate logit) * (h_s W_sd^T); the gate logit is the router's
    // column E. Prefill tiles with split-K plans, or the decode tiles.
    bf16* hs = static_cast<bf16*>(h->hs);
    const bf16* sg = static_cast<const bf16*>(w.ws_gate);
    const bf16* su = static_cast<const bf16*>(w.ws_up);
    const bf16* sd = static_cast<const bf16*>(w.ws_down);
    // (pair inputs: the launchers plan tile shape and split count themselves)
    QL_STAGE(h, QL_STAGE_SHARED_GATE_UP, s,
             QL_HIP(ql_gemm2_swiglu(z2, N, sg, su, sf, c.d, hs, decode, 1, h->g2part, s, true)));
    QL_STAGE(h, QL_STAGE_SHARED_DOWN, s,
             QL_HIP(ql_gemm2_gated_out(
                 hs, N, sd, c.d, sf, h->logits + c.n_experts, c.n_experts + 1,
                 resid_is_f32 ? static_cast<const float*>(resid) : nullptr,
                 resid_is_f32 ? nullptr : static_cast<const bf16*>(resid), h->rs, decode, 1,
                 h->g2part, s, true)));
    resid = h->rs;
    resid_is_f32 = 1;
  }
  CombineArgs ca{};
  ca.out_slot = h->out_slot;
  ca.pos_of = h->pos_of;
  ca.w = h->topw;
  ca.N = N;
  ca.k = c.top_k;
  ca.d = c.d;
  ca.y = y;
  QL_STAGE(h, QL_STAGE_COMBINE, s, QL_HIP(ql_moe_combine(ca, resid, resid_is_f32, s)));
  return QL_OK;
}

// router logits [N, E] of the last MoE call -> dst (the handle keeps a gate
// column E beside them when the layer has a shared expert)
ql_status copy_logits(ql_handle* h, int N, float* dst, hipStream_t s) {
  const ql_config& c = h->cfg;
  const size_t E = c.n_experts, ld = E + (c.shared_ffn_dim > 0 ? 1 : 0);
  if (ld == E)
    QL_HIP(hipMemcpyAsync(dst, h->logits, (size_t)N * E * 4, hipMemcpyDeviceToDevice, s));
  else
    QL_HIP(hipMemcpy2DAsync(dst, E * 4, h->logits, ld * 4, E * 4, (size_t)N,
                            hipMemcpyDeviceToDevice, s));
  return QL_OK;
}

// ---- bf16 layer -------------------------------------------------------------

ql_status ffn_dense_or_moe(ql_handle* h, int N, bool decode, bf16* y, hipStream_t s) {
  const ql_config& c = h->cfg;
  const ql_weights& w = h->w;
  const bf16* g2 = static_cast<const bf16*>(w.ln2_g);
  bf16* hh = static_cast<bf16*>(h->h);
  const bf16* wg = static_cast<const bf16*>(w.w_gate);
  const bf16* wu = static_cast<const bf16*>(w.w_up);
  const bf16* wd = static_cast<const bf16*>(w.w_down);
  h->ffn_pair = false;
  // Dense decode of a few rows: RMSNorm2 rides inside the gate/up GEMV, whose
  // z is never rounded (it is only formed, in bf16, when a tap asks for it).
  const bool gemv = decode && c.n_experts == 0 && N <= kGemvMaxRows &&
                    ql_gemv_ok(N, c.ffn_dim, c.d) && ql_gemv_ok(N, c.d, c.ffn_dim);
  if (gemv) {
    if (h->taps.z)
      QL_STAGE(h, QL_STAGE_RMSNORM2, s,
               QL_HIP(ql_rmsnorm_f32in_bf16(h->r, g2, static_cast<bf16*>(h->z), nullptr, N, c.d,
                                            c.rms_eps, s)));
    QL_STAGE(h, QL_STAGE_GATE_UP, s,
             QL_HIP(ql_gemv_rmsnorm_swiglu(h->r, g2, c.rms_eps, N, wg, wu, c.ffn_dim, c.d, hh, s)));
    QL_STAGE(h, QL_STAGE_DOWN, s,
             QL_HIP(ql_gemv_resid_out(hh, N, wd, c.d, c.ffn_dim, h->r, y, s)));
    return QL_OK;
  }
  // Otherwise RMSNorm2's output and the FFN hidden stay fp32 as [hi | lo]
  // bf16 pairs (the x-hat buffer is free once Q/K/V exist): gate/up and down
  // read them over a doubled K (prefill tiles) or with hi and lo rows sharing
  // each weight tile (decode tiles); the MoE router also gets fp32 z.
  bf16* z2 = static_cast<bf16*>(h->xhat);
  QL_STAGE(h, QL_STAGE_RMSNORM2, s,
           QL_HIP(ql_rmsnorm_f32_to_hilo(h->r, g2, z2, N, c.d, c.rms_eps, s,
                                         c.n_experts > 0 ? h->zf : nullptr)));
  h->ffn_pair = c.n_experts == 0;
  if (c.n_experts > 0) return moe_core(h, N, h->r, 1, y, decode, s);
  // (pair inputs: the launchers plan tile shape and split count themselves)
  QL_STAGE(h, QL_STAGE_GATE_UP, s,
           QL_HIP(ql_gemm2_swiglu(z2, N, wg, wu, c.ffn_dim, c.d, hh, decode, 1, h->g2part, s,
                                  true)));
  QL_STAGE(h, QL_STAGE_DOWN, s,
           QL_HIP(ql_gemm2_resid_out(hh, N, wd, c.d, c.ffn_dim, h->r, y, decode, 1, h->g2part, s,
                                     true)));
  return QL_OK;
}

// A varlen prefill: sequence b's new rows are rows seq_start[b] ..
// seq_start[b + 1] - 1 of the call, written after prefix[b] cache rows.
struct Varlen {
  const int* seq_start;  // [B + 1] device, or NULL: B sequences of S rows each
  const int* prefix;     // [B] device, or NULL: no prefix
  int N;                 // total new rows
};

// Prefill: RMSNorm1 -> QKV GEMM (+bias) -> QK-norm/RoPE/cache -> attention ->
// O GEMM + residual -> FFN half. S is the rows per sequence, or with a
// varlen batch the most new rows of any sequence.
ql_status prefill_bf16(ql_handle* h, const bf16* x, int B, int S, int pos_offset, void* kc,
                       void* vc, int T_max, bf16* y, hipStream_t s, const Varlen& vl = Varlen{}) {
  const ql_config& c = h->cfg;
  const ql_weights& w = h->w;
  const int N = vl.seq_start ? vl.N : B * S;
  if (gemm2_call_part_bytes(c, h->q_dim, h->qkv_dim, N, false) > h->g2part_bytes)
    return fail(QL_EUNSUPPORTED, "prefill: %d rows need more GEMM partial space than the handle holds",
                N);
  bf16* xhat = static_cast<bf16*>(h->xhat);  // [N, 2d]: hi | lo
  QL_STAGE(h, QL_STAGE_RMSNORM1, s,
           QL_HIP(ql_rmsnorm_bf16_to_hilo(x, static_cast<const bf16*>(w.ln1_g), xhat, N, c.d,
                                          c.rms_eps, s)));
  const bf16* bq = c.qkv_bias ? static_cast<const bf16*>(w.bq) : nullptr;
  const bf16* bk = c.qkv_bias ? static_cast<const bf16*>(w.bk) : nullptr;
  const bf16* bv = c.qkv_bias ? static_cast<const bf16*>(w.bv) : nullptr;
  // QKV projection with QK-norm, RoPE and the cache write in its epilogue
  QkvFinish f{};
  f.S = S;
  f.pos_offset = pos_offset;
  f.T_max = T_max;
  f.eps = c.rms_eps;
  f.omega = h->rope_omega;
  f.q_norm_g = c.qk_norm ? static_cast<const bf16*>(w.q_norm_g) : nullptr;
  f.k_norm_g = c.qk_norm ? static_cast<const bf16*>(w.k_norm_g) : nullptr;
  f.q_out = static_cast<bf16*>(h->q);
  f.k_cache = static_cast<bf16*>(kc);
  f.v_cache = static_cast<bf16*>(vc);
  f.seq_start = vl.seq_start;
  f.prefix = vl.prefix;
  f.nseq = B;
  QL_STAGE(h, QL_STAGE_QKV, s,
           QL_HIP(ql_gemm2_qkv(xhat, N, static_cast<const bf16*>(w.wq),
                               static_cast<const bf16*>(w.wk), static_cast<const bf16*>(w.wv),
                               h->q_dim, h->kv_dim, c.d, bq, bk, bv, f, false, 0, h->g2part,
                               s)));
  AttnPrefillArgs pa{};
  pa.q = static_cast<const bf16*>(h->q);
  pa.k_cache = static_cast<const bf16*>(kc);
  pa.v_cache = static_cast<const bf16*>(vc);
  pa.out = static_cast<bf16*>(h->attn);  // [N, 2q]: hi | lo
  pa.lo_off = h->q_dim;
  pa.ldq = h->q_dim;
  pa.ldo = 2 * h->q_dim;
  pa.B = B;
  pa.S = S;
  pa.T_max = T_max;
  pa.n_q_heads = c.n_q_heads;
  pa.n_kv_heads = c.n_kv_heads;
  pa.head_dim = c.head_dim;
  pa.scale_log2 = scale_log2(c.head_dim);
  pa.seq_start = vl.seq_start;
  pa.prefix = vl.prefix;
  QL_STAGE(h, QL_STAGE_ATTENTION, s, QL_HIP(ql_attn_prefill_bf16(pa, s)));
  h->attn_hilo = true;
  QL_STAGE(h, QL_STAGE_O_PROJ, s,
           QL_HIP(ql_gemm2_resid_f32(static_cast<const bf16*>(h->attn), N,
                                     static_cast<const bf16*>(w.wo), c.d, h->q_dim, x, h->r,
                                     false, 0, h->g2part, s)));
  return ffn_dense_or_moe(h, N, false, y, s);
}

// Decode, up to kGemvMaxRows sequences: QKV projection of x * gamma1 (raw
// sums) -> attention with RMSNorm1 scale, QK-norm, RoPE and the cache append
// fused in -> O projection + residual -> FFN half.
// More sequences: RMSNorm1 -> QKV on MFMA tiles with QK-norm, RoPE and the
// cache append in the epilogue -> attention -> O projection + residual ->
// FFN half; the hi/lo activation pairs share each weight tile.
ql_status decode_bf16(ql_handle* h, const bf16* x, int B, const int* cache_len, int pos_offset,
                      void* kc, void* vc, int T_max, bf16* y, hipStream_t s) {
  const ql_config& c = h->cfg;
  const ql_weights& w = h->w;
  const bool gemv = B <= kGemvMaxRows && ql_gemv_ok(B, h->qkv_dim, c.d) &&
                    ql_gemv_ok(B, c.d, h->q_dim);
  if (gemm2_call_part_bytes(c, h->q_dim, h->qkv_dim, B, true) > h->g2part_bytes)
    return fail(QL_EUNSUPPORTED, "decode: %d rows need more GEMM partial space than the handle holds",
                B);
  const bf16* g1 = static_cast<const bf16*>(w.ln1_g);
  const bf16* wq = static_cast<const bf16*>(w.wq);
  const bf16* wk = static_cast<const bf16*>(w.wk);
  const bf16* wv = static_cast<const bf16*>(w.wv);
  const bf16* wo = static_cast<const bf16*>(w.wo);
  const bf16* bq = c.qkv_bias ? static_cast<const bf16*>(w.bq) : nullptr;
  const bf16* bk = c.qkv_bias ? static_cast<const bf16*>(w.bk) : nullptr;
  const bf16* bv = c.qkv_bias ? static_cast<const bf16*>(w.bv) : nullptr;
  AttnDecodeArgs da{};
  da.k_cache = static_cast<const bf16*>(kc);
  da.v_cache = static_cast<const bf16*>(vc);
  da.cache_len = cache_len;
  da.B = B;
  da.T_max = T_max;
  da.n_q_heads = c.n_q_heads;
  da.n_kv_heads = c.n_kv_heads;
  da.head_dim = c.head_dim;
  int chunk = 0;
  da.nsplit = gemv ? decode_splits(B * c.n_kv_heads, T_max, 16, kDecodeTargetWaves, &chunk)
                   : decode_splits(B * c.n_kv_heads, T_max, 32, kDecodeMfmaTargetWaves, &chunk);
  da.chunk = chunk;
  da.part_o = h->part_o;
  da.part_ml = h->part_ml;
  da.scale_log2 = scale_log2(c.head_dim);
  if (!gemv) {
    bf16* xhat = static_cast<bf16*>(h->xhat);  // [B, 2d]: hi | lo
    QL_STAGE(h, QL_STAGE_RMSNORM1, s,
             QL_HIP(ql_rmsnorm_bf16_to_hilo(x, g1, xhat, B, c.d, c.rms_eps, s)));
    QkvFinish f{};
    f.S = 1;
    f.pos_offset = pos_offset;
    f.T_max = T_max;
    f.cache_len = cache_len;
    f.eps = c.rms_eps;
    f.omega = h->rope_omega;
    f.q_norm_g = c.qk_norm ? static_cast<const bf16*>(w.q_norm_g) : nullptr;
    f.k_norm_g = c.qk_norm ? static_cast<const bf16*>(w.k_norm_g) : nullptr;
    f.q_out = static_cast<bf16*>(h->q);
    f.k_cache = static_cast<bf16*>(kc);
    f.v_cache = static_cast<bf16*>(vc);
    QL_STAGE(h, QL_STAGE_QKV, s,
             QL_HIP(ql_gemm2_qkv(xhat, B, wq, wk, wv, h->q_dim, h->kv_dim, c.d, bq, bk, bv, f,
                                 true, 1, h->g2part, s)));
    da.q_in = static_cast<const bf16*>(h->q);
    da.out_hilo = static_cast<bf16*>(h->attn);  // [B, 2q]: hi | lo
    da.lo_off = h->q_dim;
    da.ldo = 2 * h->q_dim;
    QL_STAGE(h, QL_STAGE_ATTENTION, s, QL_HIP(ql_attn_decode_bf16(da, s)));
    h->attn_hilo = true;
    QL_STAGE(h, QL_STAGE_O_PROJ, s,
             QL_HIP(ql_gemm2_resid_f32(static_cast<const bf16*>(h->attn), B, wo, c.d, h->q_dim,
                                       x, h->r, true, 1, h->g2part, s)));
    return ffn_dense_or_moe(h, B, true, y, s);
  }
  QL_STAGE(h, QL_STAGE_QKV, s,
           QL_HIP(ql_gemv_qkv_raw(x, g1, B, wq, wk, wv, h->q_dim, h->kv_dim, c.d, h->qkv,
                                  c.rms_eps, h->inv_rms, s)));
  da.k_cache_w = static_cast<bf16*>(kc);
  da.v_cache_w = static_cast<bf16*>(vc);
  da.qkv_raw = h->qkv;
  da.ld_raw = h->qkv_dim;
  da.x = x;
  da.d = c.d;
  da.bq = bq;
  da.bk = bk;
  da.bv = bv;
  if (c.qk_norm) {
    da.q_norm_g = static_cast<const bf16*>(w.q_norm_g);
    da.k_norm_g = static_cast<const bf16*>(w.k_norm_g);
  }
  da.eps = c.rms_eps;
  da.theta = c.rope_theta;
  da.pos_offset = pos_offset;
  da.q_out = static_cast<bf16*>(h->q);
  da.out = static_cast<float*>(h->attn);
  da.ldo = h->q_dim;
  da.rope_omega = h->rope_omega;
  da.inv_rms = h->inv_rms;
  QL_STAGE(h, QL_STAGE_ATTENTION, s, QL_HIP(ql_attn_decode_bf16(da, s)));
  h->attn_hilo = false;
  QL_STAGE(h, QL_STAGE_O_PROJ, s,
           QL_HIP(ql_gemv_resid_f32(static_cast<const float*>(h->attn), B, wo, c.d, h->q_dim, x,
                                    h->r, s)));
  return ffn_dense_or_moe(h, B, true, y, s);
}

// ---- fp32 layer (small shapes) ---------------------------------------------

ql_status layer_f32(ql_handle* h, const float* x, int N, bool decode, int B, int S,
                    const int* cache_len, int pos_offset, void* kc, void* vc, int T_max, float* y,
                    hipStream_t s) {
  h->attn_hilo = false;
  h->ffn_pair = false;
  const ql_config& c = h->cfg;
  const ql_weights& w = h->w;
  float* xhat = static_cast<float*>(h->xhat);
  QL_HIP(ql_rmsnorm_f32(x, static_cast<const float*>(w.ln1_g), xhat, N, c.d, c.rms_eps, s));
  const float* wq = static_cast<const float*>(w.wq);
  const float* wk = static_cast<const float*>(w.wk);
  const float* wv = static_cast<const float*>(w.wv);
  const float* bq = c.qkv_bias ? static_cast<const float*>(w.bq) : nullptr;
  const float* bk = c.qkv_bias ? static_cast<const float*>(w.bk) : nullptr;
  const float* bv = c.qkv_bias ? static_cast<const float*>(w.bv) : nullptr;
  QL_HIP(ql_gemm_f32_generic(0, xhat, wq, nullptr, N, h->q_dim, c.d, bq, h->qkv, h->qkv_dim, s));
  QL_HIP(ql_gemm_f32_generic(0, xhat, wk, nullptr, N, h->kv_dim, c.d, bk, h->qkv + h->q_dim,
                             h->qkv_dim, s));
  QL_HIP(ql_gemm_f32_generic(0, xhat, wv, nullptr, N, h->kv_dim, c.d, bv,
                             h->qkv + h->q_dim + h->kv_dim, h->qkv_dim, s));
  QkvPostArgs qa{};
  qa.qkv = h->qkv;
  qa.ld_qkv = h->qkv_dim;
  qa.rows = N;
  qa.seq = S;
  qa.cache_len = decode ? cache_len : nullptr;
  qa.T_max = T_max;
  qa.pos_offset = pos_offset;
  qa.n_q_heads = c.n_q_heads;
  qa.n_kv_heads = c.n_kv_heads;
  qa.head_dim = c.head_dim;
  qa.eps = c.rms_eps;
  qa.theta = c.rope_theta;
  qa.q_norm_g = c.qk_norm ? w.q_norm_g : nullptr;
  qa.k_norm_g = c.qk_norm ? w.k_norm_g : nullptr;
  qa.q_out = h->q;
  qa.k_cache = kc;
  qa.v_cache = vc;
  QL_HIP(ql_qkv_post_f32(qa, s));
  float* attn = static_cast<float*>(h->attn);
  if (decode) {
    AttnDecodeArgs da{};
    da.qf = static_cast<const float*>(h->q);
    da.kf = static_cast<const float*>(kc);
    da.vf = static_cast<const float*>(vc);
    da.outf = attn;
    da.cache_len = cache_len;
    da.ldq = h->q_dim;
    da.ldo = h->q_dim;
    da.B = B;
    da.T_max = T_max;
    da.n_q_heads = c.n_q_heads;
    da.n_kv_heads = c.n_kv_heads;
    da.head_dim = c.head_dim;
    QL_HIP(ql_attn_decode_f32(da, s));
  } else {
    AttnPrefillArgs pa{};
    pa.qf = static_cast<const float*>(h->q);
    pa.kf = static_cast<const float*>(kc);
    pa.vf = static_cast<const float*>(vc);
    pa.outf = attn;
    pa.ldq = h->q_dim;
    pa.ldo = h->q_dim;
    pa.B = B;
    pa.S = S;
    pa.T_max = T_max;
    pa.n_q_heads = c.n_q_heads;
    pa.n_kv_heads = c.n_kv_heads;
    pa.head_dim = c.head_dim;
    QL_HIP(ql_attn_prefill_f32(pa, s));
  }
  QL_HIP(ql_gemm_f32_generic(1, attn, static_cast<const float*>(w.wo), nullptr, N, c.d, h->q_dim,
                             x, h->r, c.d, s));
  float* z = static_cast<float*>(h->z);
  QL_HIP(ql_rmsnorm_f32(h->r, static_cast<const float*>(w.ln2_g), z, N, c.d, c.rms_eps, s));
  float* hh = static_cast<float*>(h->h);
  QL_HIP(ql_gemm_f32_generic(2, z, static_cast<const float*>(w.w_gate),
                             static_cast<const float*>(w.w_up), N, c.ffn_dim, c.d, nullptr, hh,
                             c.ffn_dim, s));
  QL_HIP(ql_gemm_f32_generic(1, hh, static_cast<const float*>(w.w_down), nullptr, N, c.d,
                             c.ffn_dim, h->r, y, c.d, s));
  return QL_OK;
}

void init_dims(ql_handle* h, const ql_config* cfg, const ql_weights* w) {
  h->cfg = *cfg;
  h->w = *w;
  h->es = cfg->dtype == QL_BF16 ? 2 : 4;
  h->q_dim = cfg->n_q_heads * cfg->head_dim;
  h->kv_dim = cfg->n_kv_heads * cfg->head_dim;
  h->qkv_dim = h->q_dim + 2 * h->kv_dim;
  h->G = cfg->n_q_heads / cfg->n_kv_heads;
  h->rows = std::max(std::max(cfg->max_tokens, cfg->max_batch), 1);
}

// omega_i = theta^(-2i/dh), i < dh/2 ("推理系统 03" §6), in fp64 on the host
std::vector<double> rope_table(const ql_config& c) {
  std::vector<double> om(c.head_dim / 2);
  for (int i = 0; i < c.head_dim / 2; ++i)
    om[i] = std::pow((double)c.rope_theta, -2.0 * i / (double)c.head_dim);
  return om;
}

ql_status check_decode_args(const void* x, int B, const int* cache_len, const int* cache_len_host,
                            const void* k_cache, const void* v_cache, int T_max, const void* y) {
  if (!x || !cache_len || !k_cache || !v_cache || !y)
    return fail(QL_EINVAL, "decode: NULL argument");
  if (B <= 0) return fail(QL_EINVAL, "decode: B must be positive");
  if (T_max <= 0) return fail(QL_EINVAL, "decode: T_max must be positive");
  if (x == y) return fail(QL_EINVAL, "decode: y must not alias x");
  if (cache_len_host)
    for (int b = 0; b < B; ++b)
      if (cache_len_host[b] < 0 || cache_len_host[b] + 1 > T_max)
        return fail(QL_ECACHE_FULL, "decode: cache_len[%d] = %d does not fit T_max = %d", b,
                    cache_len_host[b], T_max);
  return QL_OK;
}

ql_status run_decode(ql_handle* h, const void* x, int B, const int* cache_len, int pos_offset,
                     void* k_cache, void* v_cache, int T_max, void* y, hipStream_t s) {
  ql_status st;
  if (h->cfg.dtype == QL_F32) {
    st = layer_f32(h, static_cast<const float*>(x), B, true, B, 1, cache_len, pos_offset, k_cache,
                   v_cache, T_max, static_cast<float*>(y), s);
  } else {
    st = decode_bf16(h, static_cast<const bf16*>(x), B, cache_len, pos_offset, k_cache, v_cache,
                     T_max, static_cast<bf16*>(y), s);
  }
  if (st == QL_OK) st = copy_taps(h, B, s);
  return st;
}

}  // namespace

extern "C" {

const char* qlayer_last_error(void) { return g_last_error.c_str(); }

int qlayer_abi_version(void) { return QLAYER_ABI_VERSION; }

ql_status qlayer_create(const ql_config* cfg, const ql_weights* w, ql_handle** out) {
  if (!out) return fail(QL_EINVAL, "out must not be NULL");
  *out = nullptr;
  ql_status st = validate(cfg, w);
  if (st != QL_OK) return st;
  ql_handle* h = new ql_handle();
  init_dims(h, cfg, w);
  hipError_t e = hipGetDevice(&h->device);
  if (e != hipSuccess) {
    delete h;
    return fail(QL_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  }
  h->ws_bytes = layout(h, nullptr);
  e = hipMalloc(reinterpret_cast<void**>(&h->ws), h->ws_bytes);
  if (e != hipSuccess) {
    delete h;
    return fail(QL_ENOMEM, "workspace of %zu bytes: %s", h->ws_bytes, hipGetErrorString(e));
  }
  layout(h, h->ws);
  if (cfg->dtype == QL_BF16) {
    const std::vector<double> om = rope_table(*cfg);
    e = hipMemcpy(h->rope_omega, om.data(), om.size() * sizeof(double), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      (void)hipFree(h->ws);  // the upload's error is the one reported
      delete h;
      return fail(QL_EHIP, "RoPE table upload: %s", hipGetErrorString(e));
    }
  }
  *out = h;
  return QL_OK;
}

ql_status qlayer_destroy(ql_handle* h) {
  if (!h) return QL_OK;
  hipError_t e = hipDeviceSynchronize();
  hipError_t f = hipFree(h->ws);
  delete h;
  if (e != hipSuccess) return fail(QL_EHIP, "hipDeviceSynchronize: %s", hipGetErrorString(e));
  if (f != hipSuccess) return fail(QL_EHIP, "hipFree: %s", hipGetErrorString(f));
  return QL_OK;
}

size_t qlayer_workspace_bytes(const ql_handle* h) { return h ? h->ws_bytes : 0; }

ql_status qlayer_set_taps(ql_handle* h, const ql_taps* taps) {
  if (!h) return fail(QL_EINVAL, "handle must not be NULL");
  if (taps) h->taps = *taps;
  else std::memset(&h->taps, 0, sizeof(h->taps));
  return QL_OK;
}

ql_status qlayer_set_stage_events(ql_handle* h, int stage, void* start_event, void* stop_event) {
  if (!h) return fail(QL_EINVAL, "handle must not be NULL");
  if (stage < QL_STAGE_NONE || stage > QL_STAGE_SHARED_DOWN)
    return fail(QL_EINVAL, "unknown stage %d", stage);
  if (stage == QL_STAGE_NONE || !start_event || !stop_event) {
    h->ev_stage = QL_STAGE_NONE;
    h->ev_start = h->ev_stop = nullptr;
    return QL_OK;
  }
  h->ev_stage = stage;
  h->ev_start = static_cast<hipEvent_t>(start_event);
  h->ev_stop = static_cast<hipEvent_t>(stop_event);
  return QL_OK;
}

ql_status qlayer_prefill(ql_handle* h, const void* x, int B, int S, int pos_offset, void* k_cache,
                         void* v_cache, int T_max, void* y, void* stream) {
  if (!h || !x || !k_cache || !v_cache || !y)
    return fail(QL_EINVAL, "prefill: NULL argument");
  if (B <= 0 || S <= 0) return fail(QL_EINVAL, "prefill: B and S must be positive");
  if ((long long)B * S > h->cfg.max_tokens)
    return fail(QL_EINVAL, "prefill: B*S = %lld exceeds max_tokens %d", (long long)B * S,
                h->cfg.max_tokens);
  if (S > T_max) return fail(QL_EINVAL, "prefill: S (%d) > T_max (%d)", S, T_max);
  if (x == y) return fail(QL_EINVAL, "prefill: y must not alias x");
  if (h->cfg.dtype == QL_BF16 && !prefill_cache_fits(h->cfg, T_max))
    return fail(QL_EUNSUPPORTED, "prefill: T_max = %d: one sequence's cache must stay below 4 GiB",
                T_max);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int N = B * S;
  ql_status st;
  if (h->cfg.dtype == QL_F32) {
    st = layer_f32(h, static_cast<const float*>(x), N, false, B, S, nullptr, pos_offset, k_cache,
                   v_cache, T_max, static_cast<float*>(y), s);
  } else {
    st = prefill_bf16(h, static_cast<const bf16*>(x), B, S, pos_offset, k_cache, v_cache, T_max,
                      static_cast<bf16*>(y), s);
  }
  if (st == QL_OK) st = copy_taps(h, N, s);
  return st;
}

ql_status qlayer_prefill_varlen(ql_handle* h, const void* x, int B, const int* seq_start,
                                const int* cache_len, const int* seq_start_host,
                                const int* cache_len_host, int pos_offset, void* k_cache,
                                void* v_cache, int T_max, void* y, void* stream) {
  if (!h || !x || !seq_start || !cache_len || !seq_start_host || !cache_len_host || !k_cache ||
      !v_cache || !y)
    return fail(QL_EINVAL, "prefill_varlen: NULL argument");
  if (B <= 0) return fail(QL_EINVAL, "prefill_varlen: B must be positive");
  if (x == y) return fail(QL_EINVAL, "prefill_varlen: y must not alias x");
  if (h->cfg.dtype != QL_BF16)
    return fail(QL_EUNSUPPORTED, "prefill_varlen: needs dtype QL_BF16");
  if (!prefill_cache_fits(h->cfg, T_max))
    return fail(QL_EUNSUPPORTED,
                "prefill_varlen: T_max = %d: one sequence's cache must stay below 4 GiB", T_max);
  if (seq_start_host[0] != 0) return fail(QL_EINVAL, "prefill_varlen: seq_start[0] must be 0");
  int S_max = 0;
  for (int b = 0; b < B; ++b) {
    const int n = seq_start_host[b + 1] - seq_start_host[b];
    if (n < 0) return fail(QL_EINVAL, "prefill_varlen: seq_start must not decrease (at %d)", b);
    S_max = std::max(S_max, n);
    if (cache_len_host[b] < 0 || (long long)cache_len_host[b] + n > T_max)
      return fail(QL_ECACHE_FULL, "prefill_varlen: sequence %d: %d cached + %d new rows exceed "
                  "T_max = %d", b, cache_len_host[b], n, T_max);
  }
  const int N = seq_start_host[B];
  if (N <= 0) return fail(QL_EINVAL, "prefill_varlen: no new rows");
  if (N > h->cfg.max_tokens)
    return fail(QL_EINVAL, "prefill_varlen: %d rows exceed max_tokens %d", N, h->cfg.max_tokens);
  hipStream_t s = static_cast<hipStream_t>(stream);
  Varlen vl{seq_start, cache_len, N};
  ql_status st = prefill_bf16(h, static_cast<const bf16*>(x), B, S_max, pos_offset, k_cache,
                              v_cache, T_max, static_cast<bf16*>(y), s, vl);
  if (st == QL_OK) st = copy_taps(h, N, s);
  return st;
}

ql_status qlayer_decode(ql_handle* h, const void* x, int B, const int* cache_len,
                        const int* cache_len_host, int pos_offset, void* k_cache, void* v_cache,
                        int T_max, void* y, void* stream) {
  if (!h) return fail(QL_EINVAL, "decode: NULL argument");
  ql_status st = check_decode_args(x, B, cache_len, cache_len_host, k_cache, v_cache, T_max, y);
  if (st != QL_OK) return st;
  if (B > h->cfg.max_batch)
    return fail(QL_EINVAL, "decode: B = %d exceeds max_batch %d", B, h->cfg.max_batch);
  return run_decode(h, x, B, cache_len, pos_offset, k_cache, v_cache, T_max, y,
                    static_cast<hipStream_t>(stream));
}

ql_status qlayer_decode_stack(ql_handle* const* layers, int L, const void* x, int B,
                              const int* cache_len, const int* cache_len_host, int pos_offset,
                              void* const* k_caches, void* const* v_caches, int T_max, void* y,
                              void* tmp, void* stream) {
  if (!layers || !k_caches || !v_caches || !tmp || L <= 0)
    return fail(QL_EINVAL, "decode_stack: NULL argument or L <= 0");
  ql_status st = check_decode_args(x, B, cache_len, cache_len_host, k_caches[0], v_caches[0],
                                   T_max, y);
  if (st != QL_OK) return st;
  if (tmp == x || tmp == y) return fail(QL_EINVAL, "decode_stack: tmp must not alias x or y");
  const ql_config& c0 = layers[0] ? layers[0]->cfg : ql_config{};
  for (int l = 0; l < L; ++l) {
    const ql_handle* h = layers[l];
    if (!h || !k_caches[l] || !v_caches[l])
      return fail(QL_EINVAL, "decode_stack: layer %d: NULL handle or cache", l);
    if (h->cfg.d != c0.d || h->cfg.dtype != c0.dtype)
      return fail(QL_EINVAL, "decode_stack: layer %d: d or dtype differs from layer 0", l);
    if (B > h->cfg.max_batch)
      return fail(QL_EINVAL, "decode_stack: layer %d: B = %d exceeds max_batch %d", l, B,
                  h->cfg.max_batch);
  }
  // layer l writes y when L - 1 - l is even, else tmp, so the last lands in y
  hipStream_t s = static_cast<hipStream_t>(stream);
  const void* in = x;
  for (int l = 0; l < L; ++l) {
    void* out = ((L - 1 - l) % 2 == 0) ? y : tmp;
    st = run_decode(layers[l], in, B, cache_len, pos_offset, k_caches[l], v_caches[l], T_max, out,
                    s);
    if (st != QL_OK) return st;
    in = out;
  }
  return QL_OK;
}

ql_status qlayer_decode_noalloc(const ql_config* cfg, const ql_weights* w, const void* x, int B,
                                const int* cache_len, const int* cache_len_host, int pos_offset,
                                void* k_cache, void* v_cache, int T_max, void* y, void* stream) {
  if (!cfg || !w) return fail(QL_EINVAL, "decode_noalloc: config and weights must not be NULL");
  ql_status st = check_decode_args(x, B, cache_len, cache_len_host, k_cache, v_cache, T_max, y);
  if (st != QL_OK) return st;
  ql_config c = *cfg;
  c.max_tokens = 0;
  c.max_batch = B;
  st = validate(&c, w);
  if (st != QL_OK) return st;
  ql_handle h{};  // a handle on the stack over the file-scope array: nothing is allocated
  init_dims(&h, &c, w);
  const size_t need = layout(&h, nullptr, B);
  if (need > (size_t)QLAYER_NOALLOC_MAX_WORKSPACE)
    return fail(QL_EUNSUPPORTED,
                "decode_noalloc: B = %d of this layer needs %zu bytes of workspace; the static "
                "array holds %zu",
                B, need, (size_t)QLAYER_NOALLOC_MAX_WORKSPACE);
  void* base = nullptr;
  QL_HIP(ql_noalloc_scratch(&base));
  QL_HIP(hipGetDevice(&h.device));
  h.ws = static_cast<char*>(base);
  h.ws_bytes = need;
  layout(&h, h.ws, B);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (c.dtype == QL_BF16) {
    const std::vector<double> om = rope_table(c);
    QL_HIP(ql_fill_rope_table(om.data(), (int)om.size(), h.rope_omega, s));
  }
  return run_decode(&h, x, B, cache_len, pos_offset, k_cache, v_cache, T_max, y, s);
}

ql_status qlayer_moe_ffn(ql_handle* h, const void* r, int N, void* y, int* topk_idx,
                         float* topk_w, void* stream) {
  if (!h || !r || !y) return fail(QL_EINVAL, "moe_ffn: NULL argument");
  if (h->cfg.n_experts <= 0) return fail(QL_EUNSUPPORTED, "moe_ffn: the handle has a dense FFN");
  if (N <= 0) return fail(QL_EINVAL, "moe_ffn: N must be positive");
  if (N > h->rows) return fail(QL_EINVAL, "moe_ffn: N = %d exceeds %d rows", N, h->rows);
  if (r == y) return fail(QL_EINVAL, "moe_ffn: y must not alias r");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const ql_config& c = h->cfg;
  // RMSNorm2 as a [hi | lo] pair and in fp32; the N rows run as a prefill
  QL_HIP(ql_rmsnorm_bf16_to_hilo(static_cast<const bf16*>(r), static_cast<const bf16*>(h->w.ln2_g),
                                 static_cast<bf16*>(h->xhat), N, c.d, c.rms_eps, s, h->zf));
  ql_status st = moe_core(h, N, r, 0, static_cast<bf16*>(y), false, s);
  if (st != QL_OK) return st;
  const size_t nk = (size_t)N * c.top_k;
  if (topk_idx)
    QL_HIP(hipMemcpyAsync(topk_idx, h->idx, nk * 4, hipMemcpyDeviceToDevice, s));
  if (topk_w) QL_HIP(hipMemcpyAsync(topk_w, h->topw, nk * 4, hipMemcpyDeviceToDevice, s));
  if (h->taps.logits) {
    st = copy_logits(h, N, h->taps.logits, s);
    if (st != QL_OK) return st;
  }
  if (h->taps.z)
    QL_HIP(hipMemcpyAsync(h->taps.z, h->zf, (size_t)N * c.d * 4, hipMemcpyDeviceToDevice, s));
  return QL_OK;
}

}  // extern "C"

// Host-side launchers of the layer's kernels (internal to the library).
// Every launcher enqueues on `s`, returns the launch status and never
// synchronises. Shapes are validated by the caller (qlayer.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

typedef __bf16 bf16;

constexpr int kMaxTopK = 32;
constexpr int kMaxExperts = 256;

// ---- RMSNorm (rows x d) ----
hipError_t ql_rmsnorm_bf16(const bf16* x, const bf16* gamma, bf16* out, float* out_f32, int rows,
                           int d, float eps, hipStream_t s);
// bf16 rows -> normalised rows as a bf16 pair per row: [hi (d) | lo (d)]
hipError_t ql_rmsnorm_bf16_to_hilo(const bf16* x, const bf16* gamma, bf16* out, int rows, int d,
                                   float eps, hipStream_t s, float* out_f32 = nullptr);
// [rows][hi (cols) | lo (cols)] -> fp32 hi + lo
hipError_t ql_hilo_to_f32(const bf16* hl, int rows, int cols, float* out, hipStream_t s);
hipError_t ql_rmsnorm_f32in_bf16(const float* x, const bf16* gamma, bf16* out, float* out_f32,
                                 int rows, int d, float eps, hipStream_t s);
// fp32 rows -> normalised rows as a bf16 pair per row: [hi (d) | lo (d)]
hipError_t ql_rmsnorm_f32_to_hilo(const float* x, const bf16* gamma, bf16* out, int rows, int d,
                                  float eps, hipStream_t s, float* out_f32 = nullptr);
// bf16 -> fp32, n elements
hipError_t ql_bf16_to_f32(const bf16* x, size_t n, float* out, hipStream_t s);
hipError_t ql_rmsnorm_f32(const float* x, const float* gamma, float* out, int rows, int d,
                          float eps, hipStream_t s);

// ---- MoE expert GEMMs over routed 32-row tiles (decode-sized batches;
// mf % 64 == 0, d % 128 == 0). fp32 activations, each staged as a bf16
// hi + lo pair (two MFMAs per weight fragment): Zf [N, d] gathered by
// slot_token, H [N*k, mf] fp32, out [N*k, d] fp32 in slot order ----
hipError_t ql_gemm_moe_gu(const float* Zf, const int* slot_token, const bf16* Wg, const bf16* Wu,
                          int mf, int d, const int* tile_expert, const int* tile_row0,
                          const int* tile_rows, const int* num_tiles, int max_tiles, float* H,
                          hipStream_t s);
hipError_t ql_gemm_moe_down(const float* H, const bf16* Wd, int mf, int d, const int* tile_expert,
                            const int* tile_row0, const int* tile_rows, const int* num_tiles,
                            int max_tiles, float* out, hipStream_t s);

// ---- GEMMs on 256-column tiles (N % 256 == 0, or F % 128 for SwiGLU; K % 64) ----
// A2 = [hi | lo] bf16 pair of an fp32 activation, [M, 2K].
// rows128 = false: prefill tiles; splits > 1 runs split-K through `part`
// (ql_gemm2_part_bytes(M, weight rows read per call, splits) bytes); the
// split count is clamped to the k steps. The pair-input forms (QKV, O) pick
// their own tile shape and split count (ql_gemm2_pair_part_bytes bytes of
// `part`) and ignore `splits`.
// rows128 = true: the 4-wave decode tiles (three-stage ring), 64 token rows
// for a pair A, whose hi and lo rows share each weight tile, 128 for a plain
// A; the (tile, k step) units are cut evenly over up to 256 blocks (stream-K)
// whose partials go through `part` (ql_gemm2_decode_part_bytes bytes);
// `splits` is ignored.
size_t ql_gemm2_part_bytes(int M, int b_rows, int splits);
size_t ql_gemm2_pair_part_bytes(int M, int N, int K);
size_t ql_gemm2_decode_part_bytes(int M, int b_rows, int K, bool pair);
bool ql_gemm2_ok(int N, int Kb, bool dual);
// QKV projection with bias, per-head QK-norm, RoPE and the cache write. Prefill
// (cache_len NULL): row = b * S + t, position t + pos_offset, cache row t.
// Decode (cache_len set): row = b, position cache_len[b] + pos_offset, cache
// row cache_len[b] (skipped when outside [0, T_max)). q goes to q_out [M, q].
// (q, kv multiples of 256; head_dim 128)
struct QkvFinish {
  int S, pos_offset, T_max;
  const int* cache_len;  // decode: [M] device, or NULL
  const int* seq_start;  // varlen prefill: [nseq + 1] device (row -> sequence), or NULL
  const int* prefix;     // varlen prefill: [nseq] cache rows before the new ones
  int nseq;
  float eps;
  const double* omega;   // [64]
  const bf16* q_norm_g;  // or NULL
  const bf16* k_norm_g;
  bf16* q_out;
  bf16* k_cache;
  bf16* v_cache;
};
hipError_t ql_gemm2_qkv(const bf16* A2, int M, const bf16* Wq, const bf16* Wk, const bf16* Wv,
                        int q, int kv, int K, const bf16* bq, const bf16* bk, const bf16* bv,
                        const QkvFinish& f, bool rows128, int splits, void* part, hipStream_t s);
hipError_t ql_gemm2_resid_f32(const bf16* A2, int M, const bf16* W, int N, int K,
                              const bf16* resid, float* out, bool rows128, int splits, void* part,
                              hipStream_t s);
// pair_in / pair: A is a [hi | lo] pair [M, 2K] (read over a doubled K on
// the prefill tiles, hi and lo rows sharing each weight tile on the decode
// tiles); SwiGLU also stores h as a pair [M, 2F] (hi | lo).
hipError_t ql_gemm2_resid_out(const bf16* A, int M, const bf16* W, int N, int K,
                              const float* resid, bf16* out, bool rows128, int splits, void* part,
                              hipStream_t s, bool pair_in = false);
hipError_t ql_gemm2_swiglu(const bf16* A, int M, const bf16* Wg, const bf16* Wu, int F, int K,
                           bf16* out, bool rows128, int splits, void* part, hipStream_t s,
                           bool pair = false);
// out[M, N] fp32 = resid + sigmoid(gate_logit[m * gate_ld]) * (A W^T)[m]:
// a shared expert's down projection scaled by its gate (resid_f32, else
// resid_bf16, else nothing is added); pair_in as above
hipError_t ql_gemm2_gated_out(const bf16* A, int M, const bf16* W, int N, int K,
                              const float* gate_logit, int gate_ld, const float* resid_f32,
                              const bf16* resid_bf16, float* out, bool rows128, int splits,
                              void* part, hipStream_t s, bool pair_in);
// MoE expert GEMMs on expert tiles of bm = 128 or 256 token rows (the
// permute's tile table built with the same bm; max_tiles bounds *num_tiles;
// mf % 128 == 0, d % 256 == 0). Z2 [N, 2d] and H2 [N*k, 2mf] are [hi | lo]
// pairs; out [N*k, d] fp32 in slot order.
hipError_t ql_gemm2_moe_gu(const bf16* Z2, const int* slot_token, const bf16* Wg, const bf16* Wu,
                           int mf, int d, const int* tile_expert, const int* tile_row0,
                           const int* tile_rows, const int* num_tiles, int max_tiles, int bm,
                           bf16* H2, hipStream_t s);
hipError_t ql_gemm2_moe_down(const bf16* H2, const bf16* Wd, int mf, int d,
                             const int* tile_expert, const int* tile_row0, const int* tile_rows,
                             const int* num_tiles, int max_tiles, int bm, float* out,
                             hipStream_t s);

// ---- decode GEMVs for M <= kGemvMaxRows rows (N % 2 == 0, K % 8 == 0) ----
// qkv_raw: out[M, q+2kv] fp32 = raw sums of (x * gamma) [Wq; Wk; Wv]^T (x,
// gamma bf16; RMSNorm's 1/rms and the QKV bias are applied by the consumer).
// resid_f32: out[M, N] fp32 = resid + X W^T (X fp32). resid_out: out[M, N]
// bf16 = resid + X W^T. rmsnorm_swiglu: out[M, F] = SiLU(z Wg^T) * (z Wu^T)
// with z = RMSNorm(R) formed on the fly.
constexpr int kGemvMaxRows = 4;
bool ql_gemv_ok(int M, int N, int K);
// (the QKV form also writes RMSNorm's 1/rms of each x row to inv_rms[M] if non-NULL)
hipError_t ql_gemv_qkv_raw(const bf16* x, const bf16* gamma, int M, const bf16* Wq,
                           const bf16* Wk, const bf16* Wv, int q, int kv, int K, float* out,
                           float eps, float* inv_rms, hipStream_t s);
hipError_t ql_gemv_resid_f32(const float* X, int M, const bf16* W, int N, int K,
                             const bf16* resid, float* out, hipStream_t s);
hipError_t ql_gemv_resid_out(const bf16* X, int M, const bf16* W, int N, int K,
                             const float* resid, bf16* out, hipStream_t s);
// out[M, F] = SiLU(Z Wg^T) * (Z Wu^T), Z = RMSNorm(R) * gamma computed on the fly
// (R fp32 [M, K])
hipError_t ql_gemv_rmsnorm_swiglu(const float* R, const bf16* gamma, float eps, int M,
                                  const bf16* Wg, const bf16* Wu, int F, int K, bf16* out,
                                  hipStream_t s);

// ---- QK-norm + RoPE + cache write (fp32 layer) ----
struct QkvPostArgs {
  const float* qkv;      // [rows, ld_qkv] fp32 projections (bias added)
  int ld_qkv;
  int rows;              // prefill: B*S; decode: B
  int seq;               // prefill: S (row n -> sequence n / S, cache row n % S)
  const int* cache_len;  // decode: [B] cache row of the new token; NULL for prefill
  int T_max;
  int pos_offset;
  int n_q_heads, n_kv_heads, head_dim;
  float eps, theta;
  const void* q_norm_g;  // NULL -> no QK-norm
  const void* k_norm_g;
  void* q_out;           // [rows, Hq*dh]
  void* k_cache;         // [B, T_max, Hkv, dh]
  void* v_cache;
};
hipError_t ql_qkv_post_f32(const QkvPostArgs& a, hipStream_t s);

// ---- attention ----
struct AttnPrefillArgs {
  const bf16* q;         // [B*S, ldq]
  const bf16* k_cache;   // [B, T_max, Hkv, dh]
  const bf16* v_cache;
  bf16* out;             // [B*S, ldo] fp32 output as bf16 hi (column c) + lo (c + lo_off)
  int lo_off;
  const float* qf;       // fp32 variants of the same buffers (QL_F32)
  const float* kf;
  const float* vf;
  float* outf;
  int ldq, ldo;
  int B, S, T_max;       // S: new rows per sequence (varlen: the most of any sequence)
  int n_q_heads, n_kv_heads, head_dim;
  float scale_log2;      // log2(e) / sqrt(dh)
  int pair;              // set by the launcher: a block takes query tiles nqt-1-x and x
  int gx, gy, gtotal;    // set by the launcher: the (tile, head, sequence) work grid
  const int* seq_start;  // varlen [B + 1] device: sequence b's q rows, or NULL (b S)
  const int* prefix;     // [B] device: cache rows before the new ones, or NULL (0)
};
hipError_t ql_attn_prefill_bf16(const AttnPrefillArgs& a, hipStream_t s);
hipError_t ql_attn_prefill_f32(const AttnPrefillArgs& a, hipStream_t s);

struct AttnDecodeArgs {
  const bf16* q;         // unused by the fused bf16 kernel
  const bf16* k_cache;   // [B, T_max, Hkv, dh]
  const bf16* v_cache;
  bf16* k_cache_w;       // same caches, written at row cache_len[b]
  bf16* v_cache_w;
  const float* qkv_raw;  // [B, ld_raw] raw sums of (x * gamma1) [Wq; Wk; Wv]^T
  int ld_raw;
  const bf16* x;         // [B, d] layer input (for RMSNorm1's 1/rms)
  int d;
  const bf16* bq;        // QKV bias or NULL
  const bf16* bk;
  const bf16* bv;
  const bf16* q_norm_g;  // QK-norm gammas or NULL
  const bf16* k_norm_g;
  float eps, theta;
  int pos_offset;
  bf16* q_out;           // [B, Hq*dh] rotated queries (optional copy)
  const bf16* q_in;      // [B, Hq*dh] finished queries, row cache_len[b] already in
                         // the cache: no prologue (or NULL)
  float* out;            // [B, ldo] fp32
  bf16* out_hilo;        // or [B, ldo] bf16 hi at col, lo at col + lo_off
  int lo_off;
  const float* qf;
  const float* kf;
  const float* vf;
  float* outf;
  const int* cache_len;  // [B] device
  int ldq, ldo;
  int B, T_max;
  int n_q_heads, n_kv_heads, head_dim;
  int chunk, nsplit;     // keys per split, number of splits
  float* part_o;         // [B, Hq, nsplit, dh]
  float* part_ml;        // [B, Hq, nsplit, 2]
  const float* inv_rms;  // [B] RMSNorm1 1/rms of x, or NULL (computed from x)
  const double* rope_omega;  // [head_dim / 2] RoPE frequencies theta^(-2i/dh)
  float scale_log2;
};
constexpr int kMaxDecodeSplits = 1024;  // nsplit <= this
hipError_t ql_attn_decode_bf16(const AttnDecodeArgs& a, hipStream_t s);
hipError_t ql_attn_decode_f32(const AttnDecodeArgs& a, hipStream_t s);

// ---- fp32 GEMM for small layers: mode 0 bias, 1 residual, 2 SwiGLU ----
// out[m * ldo + n]; mode 1 reads add[m * ldo + n], mode 0 add[n] (may be NULL)
hipError_t ql_gemm_f32_generic(int mode, const float* A, const float* B, const float* B2, int M,
                               int N, int K, const float* add, float* out, int ldo, hipStream_t s);

// ---- MoE routing ----
struct RouterArgs {
  const float* zf;   // [N, d] fp32 RMSNorm2 output
  const bf16* wr;    // [E, d]
  const bf16* w_extra;  // [n_extra, d] rows computed after the E experts (a shared
  int n_extra;          // expert's gate) and left out of the top-k; or NULL, 0
  int N, d, E, k;
  int norm_topk;
  float* logits;     // [N, E + n_extra]
  int* idx;          // [N, k]
  float* w;          // [N, k]
};
hipError_t ql_router_topk(const RouterArgs& a, hipStream_t s);

struct PermuteArgs {
  const int* idx;    // [N, k]
  int N, k, E, bm;
  int* hist;         // [ceil(N/256), E]
  int* blkoff;       // [ceil(N/256), E]
  int* offsets;      // [E + 1]
  int* tile_expert;  // [max_tiles]
  int* tile_row0;
  int* tile_rows;
  int* num_tiles;    // [1]
  int* slot_token;   // [N*k]
  int* pos_of;       // [N, k]
};
hipError_t ql_moe_permute(const PermuteArgs& a, hipStream_t s);

struct CombineArgs {
  const float* out_slot;  // [N*k, d] expert outputs in slot order (fp32)
  const int* pos_of;      // [N, k]
  const float* w;         // [N, k]
  int N, k, d;
  bf16* y;                // [N, d]
};
hipError_t ql_moe_combine(const CombineArgs& a, const void* resid, int resid_is_f32,
                          hipStream_t s);

// ---- allocation-free decode (noalloc.hip) ----
// Device address of this device's file-scope workspace array
// (QLAYER_NOALLOC_MAX_WORKSPACE bytes), looked up once per device.
hipError_t ql_noalloc_scratch(void** ptr);
// dst[0..n) = w[0..n) (n <= 64) by a kernel on `s`
hipError_t ql_fill_rope_table(const double* w, int n, double* dst, hipStream_t s);

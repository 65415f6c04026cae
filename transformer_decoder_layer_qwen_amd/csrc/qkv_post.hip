// Per-head QK-RMSNorm, rotate_half RoPE and the KV-cache write, fp32 layer.
// (The bf16 prefill does the same in the QKV GEMM's epilogue; bf16 decode in
// the attention prologue.)
//
// Input: the projected rows qkv[n, Hq*dh + 2*Hkv*dh] in fp32 (bias already
// added by the projection). For each token row and each head:
//   * q, k heads: optional RMSNorm over the head's dh values with one gamma
//     shared by all Q heads (one by all K heads) ("推理系统 03：逐项算清一个真实
//     Qwen3 Transformer 层" §5), then rotation of each pair (x_i, x_{i+dh/2})
//     by pos * omega_i, omega_i = theta^(-2i/dh) (same page, §6);
//   * the rotated q goes to the query buffer, the rotated k and the plain v
//     to their cache row ("Qwen2.5-7B 结构拆解" §09.1: K and V are appended
//     once and reused; "推理系统 03" §12: cached keys are post-norm, post-RoPE).
//
// One group of dh/2 lanes serves one token row; lane i owns pair i for every
// head, so its angle is computed once (in fp64, reduced to [-pi, pi] before
// the fp32 sin/cos) and reused across heads.
#include "common.h"
#include "kernels.h"

namespace {

template <class T>
__global__ __launch_bounds__(256) void qkv_post_kernel(QkvPostArgs p) {
  const int half = p.head_dim / 2;
  const int rows_per_block = 256 / half;
  const int i = threadIdx.x % half;
  const int n = blockIdx.x * rows_per_block + threadIdx.x / half;
  if (n >= p.rows) return;  // whole lane groups leave together

  int b, crow;
  if (p.cache_len) {  // decode: one row per sequence, written at cache_len[b]
    b = n;
    crow = p.cache_len[b];
  } else {            // prefill: row n = b*S + s
    b = n / p.seq;
    crow = n % p.seq;
  }
  const bool in_range = crow >= 0 && crow < p.T_max;
  const double pos = (double)crow + (double)p.pos_offset;
  const double omega = exp2(-2.0 * (double)i / (double)p.head_dim * log2((double)p.theta));
  double ang = pos * omega;
  const double two_pi = 6.283185307179586476925286766559;
  ang -= two_pi * rint(ang * (1.0 / two_pi));
  float sn, cs;
  sincosf((float)ang, &sn, &cs);

  const float* src = p.qkv + (size_t)n * p.ld_qkv;
  const int qd = p.n_q_heads * p.head_dim;
  const int kvd = p.n_kv_heads * p.head_dim;
  const float nanv = __builtin_nanf("");
  const T* qg = static_cast<const T*>(p.q_norm_g);
  const T* kg = static_cast<const T*>(p.k_norm_g);

  // queries
  for (int h = 0; h < p.n_q_heads; ++h) {
    float x0 = src[h * p.head_dim + i];
    float x1 = src[h * p.head_dim + i + half];
    if (qg) {
      const float ss = group_sum(x0 * x0 + x1 * x1, half);
      const float inv = 1.0f / sqrtf(ss / (float)p.head_dim + p.eps);
      x0 = to_f32(qg[i]) * (x0 * inv);
      x1 = to_f32(qg[i + half]) * (x1 * inv);
    }
    float r0 = x0 * cs - x1 * sn;
    float r1 = x0 * sn + x1 * cs;
    if (!in_range) r0 = r1 = nanv;
    T* dst = static_cast<T*>(p.q_out) + (size_t)n * qd + h * p.head_dim;
    dst[i] = from_f32<T>(r0);
    dst[i + half] = from_f32<T>(r1);
  }
  if (!in_range) return;  // never write outside the cache
  const size_t cache_row = ((size_t)b * p.T_max + crow) * (size_t)kvd;
  for (int h = 0; h < p.n_kv_heads; ++h) {
    float x0 = src[qd + h * p.head_dim + i];
    float x1 = src[qd + h * p.head_dim + i + half];
    if (kg) {
      const float ss = group_sum(x0 * x0 + x1 * x1, half);
      const float inv = 1.0f / sqrtf(ss / (float)p.head_dim + p.eps);
      x0 = to_f32(kg[i]) * (x0 * inv);
      x1 = to_f32(kg[i + half]) * (x1 * inv);
    }
    T* kd = static_cast<T*>(p.k_cache) + cache_row + h * p.head_dim;
    kd[i] = from_f32<T>(x0 * cs - x1 * sn);
    kd[i + half] = from_f32<T>(x0 * sn + x1 * cs);
    const float* vs = src + qd + kvd + h * p.head_dim;
    T* vd = static_cast<T*>(p.v_cache) + cache_row + h * p.head_dim;
    vd[i] = from_f32<T>(vs[i]);
    vd[i + half] = from_f32<T>(vs[i + half]);
  }
}

template <class T>
hipError_t launch(const QkvPostArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  const int half = a.head_dim / 2;
  const int rpb = 256 / half;
  const int blocks = (a.rows + rpb - 1) / rpb;
  hipLaunchKernelGGL((qkv_post_kernel<T>), dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t ql_qkv_post_f32(const QkvPostArgs& a, hipStream_t s) { return launch<float>(a, s); }

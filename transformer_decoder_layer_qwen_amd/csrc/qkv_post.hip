// Per-head QK-RMSNorm, rotate_half RoPE and the KV-cache write.
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
  ang -= two_pi * rint(ang / two_pi);
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

// head_dim 128: one wave per (token row, head); lane i owns the pair
// (i, i + 64). Q heads come first, then one wave per KV head writes both the
// rotated K row and the V row.
__global__ __launch_bounds__(256) void qkv_post_head_kernel(QkvPostArgs p) {
  constexpr int kDh = 128;
  const int lane = threadIdx.x & 63;
  const int slots = p.n_q_heads + p.n_kv_heads;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= p.rows * slots) return;
  const int n = item / slots;
  const int slot = item % slots;
  int b, crow;
  if (p.cache_len) {
    b = n;
    crow = p.cache_len[b];
  } else {
    b = n / p.seq;
    crow = n % p.seq;
  }
  const bool in_range = crow >= 0 && crow < p.T_max;
  const int qd = p.n_q_heads * kDh;
  const int kvd = p.n_kv_heads * kDh;
  const bool is_q = slot < p.n_q_heads;
  const int h = is_q ? slot : slot - p.n_q_heads;
  if (!is_q && !in_range) return;  // never write outside the cache
  const float* src = p.qkv + (size_t)n * p.ld_qkv;
  const float* hs = src + (is_q ? h * kDh : qd + h * kDh);
  float x0 = hs[lane];
  float x1 = hs[lane + 64];
  float vv0 = 0.f, vv1 = 0.f;
  if (!is_q) {
    vv0 = src[qd + kvd + h * kDh + lane];
    vv1 = src[qd + kvd + h * kDh + lane + 64];
  }
  const double pos = (double)crow + (double)p.pos_offset;
  const double omega = exp2(-2.0 * (double)lane / (double)kDh * log2((double)p.theta));
  double ang = pos * omega;
  const double two_pi = 6.283185307179586476925286766559;
  ang -= two_pi * rint(ang / two_pi);
  float sn, cs;
  sincosf((float)ang, &sn, &cs);
  const bf16* gam = static_cast<const bf16*>(is_q ? p.q_norm_g : p.k_norm_g);
  if (gam) {
    const float ss = wave_sum(x0 * x0 + x1 * x1);
    const float inv = 1.0f / sqrtf(ss / (float)kDh + p.eps);
    x0 = to_f32(gam[lane]) * (x0 * inv);
    x1 = to_f32(gam[lane + 64]) * (x1 * inv);
  }
  float r0 = x0 * cs - x1 * sn;
  float r1 = x0 * sn + x1 * cs;
  if (is_q) {
    if (!in_range) r0 = r1 = __builtin_nanf("");
    bf16* dst = static_cast<bf16*>(p.q_out) + (size_t)n * qd + h * kDh;
    dst[lane] = (bf16)r0;
    dst[lane + 64] = (bf16)r1;
  } else {
    const size_t cache_row = ((size_t)b * p.T_max + crow) * (size_t)kvd + h * kDh;
    bf16* kd = static_cast<bf16*>(p.k_cache) + cache_row;
    bf16* vd = static_cast<bf16*>(p.v_cache) + cache_row;
    kd[lane] = (bf16)r0;
    kd[lane + 64] = (bf16)r1;
    vd[lane] = (bf16)vv0;
    vd[lane + 64] = (bf16)vv1;
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

hipError_t ql_qkv_post_bf16(const QkvPostArgs& a, hipStream_t s) {
  if (a.head_dim != 128) return launch<bf16>(a, s);
  const long long items = (long long)a.rows * (a.n_q_heads + a.n_kv_heads);
  if (items <= 0) return hipSuccess;
  hipLaunchKernelGGL(qkv_post_head_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}
hipError_t ql_qkv_post_f32(const QkvPostArgs& a, hipStream_t s) { return launch<float>(a, s); }

// fp32 kernels for small layers (QL_F32), any shape within the documented
// limits. They compute the same steps as the bf16 path in fp32 storage and
// arithmetic, one thread per output value or per (query, head), which suits
// the latency-bound toy layer of "推理系统 03：逐项算清一个真实 Qwen3 Transformer
// 层" §1 (3 positions, d = 4, 2 query heads, 1 KV head, dh = 2, MLP width 6).
//
//   gemm: C = A B^T with the bias / residual / SwiGLU epilogues
//   attention (prefill and decode): scores q.k/sqrt(dh), causal mask, stable
//   softmax (max, exp, sum), weighted sum of V (same page, §7-§9).
#include "common.h"
#include "kernels.h"

namespace {

enum : int { GF_BIAS = 0, GF_RESID, GF_SWIGLU };

template <int MODE>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A,
                                                       const float* __restrict__ B,
                                                       const float* __restrict__ B2, int M,
                                                       int N, int K, const float* __restrict__ add,
                                                       float* __restrict__ out, int ldo) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= M * N) return;
  const int m = i / N, n = i % N;
  float acc = 0.f, acc2 = 0.f;
  for (int k = 0; k < K; ++k) {
    const float a = A[(size_t)m * K + k];
    acc += a * B[(size_t)n * K + k];
    if (MODE == GF_SWIGLU) acc2 += a * B2[(size_t)n * K + k];
  }
  float v;
  if (MODE == GF_BIAS) v = acc + (add ? add[n] : 0.f);
  else if (MODE == GF_RESID) v = add[(size_t)m * ldo + n] + acc;
  else v = silu_f32(acc) * acc2;
  out[(size_t)m * ldo + n] = v;
}

constexpr int kMaxDh = 128;

__global__ __launch_bounds__(64) void attn_prefill_f32_kernel(const AttnPrefillArgs p) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  const int total = p.B * p.S * p.n_q_heads;
  if (i >= total) return;
  const int h = i % p.n_q_heads;
  const int row = i / p.n_q_heads;  // b*S + t
  const int b = row / p.S, t = row % p.S;
  const int dh = p.head_dim;
  const int g = h / (p.n_q_heads / p.n_kv_heads);
  const float* q = p.qf + (size_t)row * p.ldq + h * dh;
  const size_t rs = (size_t)p.n_kv_heads * dh;
  const float* kb = p.kf + (size_t)b * p.T_max * rs + g * dh;
  const float* vb = p.vf + (size_t)b * p.T_max * rs + g * dh;
  const float scale = 1.0f / sqrtf((float)dh);
  float m = -INFINITY;
  for (int u = 0; u <= t; ++u) {
    float s = 0.f;
    for (int e = 0; e < dh; ++e) s += q[e] * kb[u * rs + e];
    m = fmaxf(m, s * scale);
  }
  float o[kMaxDh];
  for (int e = 0; e < dh; ++e) o[e] = 0.f;
  float l = 0.f;
  for (int u = 0; u <= t; ++u) {
    float s = 0.f;
    for (int e = 0; e < dh; ++e) s += q[e] * kb[u * rs + e];
    const float pw = expf(s * scale - m);
    l += pw;
    for (int e = 0; e < dh; ++e) o[e] += pw * vb[u * rs + e];
  }
  float* out = p.outf + (size_t)row * p.ldo + h * dh;
  for (int e = 0; e < dh; ++e) out[e] = o[e] / l;
}

__global__ __launch_bounds__(64) void attn_decode_f32_kernel(const AttnDecodeArgs p) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i >= p.B * p.n_q_heads) return;
  const int b = i / p.n_q_heads, h = i % p.n_q_heads;
  const int dh = p.head_dim;
  const int g = h / (p.n_q_heads / p.n_kv_heads);
  const int L = p.cache_len[b];
  float* out = p.outf + (size_t)b * p.ldo + h * dh;
  if (L < 0 || L >= p.T_max) {
    for (int e = 0; e < dh; ++e) out[e] = __builtin_nanf("");
    return;
  }
  const float* q = p.qf + (size_t)b * p.ldq + h * dh;
  const size_t rs = (size_t)p.n_kv_heads * dh;
  const float* kb = p.kf + (size_t)b * p.T_max * rs + g * dh;
  const float* vb = p.vf + (size_t)b * p.T_max * rs + g * dh;
  const float scale = 1.0f / sqrtf((float)dh);
  float m = -INFINITY;
  for (int u = 0; u <= L; ++u) {
    float s = 0.f;
    for (int e = 0; e < dh; ++e) s += q[e] * kb[u * rs + e];
    m = fmaxf(m, s * scale);
  }
  float o[kMaxDh];
  for (int e = 0; e < dh; ++e) o[e] = 0.f;
  float l = 0.f;
  for (int u = 0; u <= L; ++u) {
    float s = 0.f;
    for (int e = 0; e < dh; ++e) s += q[e] * kb[u * rs + e];
    const float pw = expf(s * scale - m);
    l += pw;
    for (int e = 0; e < dh; ++e) o[e] += pw * vb[u * rs + e];
  }
  for (int e = 0; e < dh; ++e) out[e] = o[e] / l;
}

template <int MODE>
hipError_t launch_gemm(const float* A, const float* B, const float* B2, int M, int N, int K,
                       const float* add, float* out, int ldo, hipStream_t s) {
  const long long total = (long long)M * N;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_f32_kernel<MODE>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     s, A, B, B2, M, N, K, add, out, ldo);
  return hipGetLastError();
}

}  // namespace

hipError_t ql_gemm_f32_generic(int mode, const float* A, const float* B, const float* B2, int M,
                               int N, int K, const float* add, float* out, int ldo, hipStream_t s) {
  switch (mode) {
    case 0: return launch_gemm<GF_BIAS>(A, B, B2, M, N, K, add, out, ldo, s);
    case 1: return launch_gemm<GF_RESID>(A, B, B2, M, N, K, add, out, ldo, s);
    case 2: return launch_gemm<GF_SWIGLU>(A, B, B2, M, N, K, add, out, ldo, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t ql_attn_prefill_f32(const AttnPrefillArgs& a, hipStream_t s) {
  const int total = a.B * a.S * a.n_q_heads;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_prefill_f32_kernel, dim3((total + 63) / 64), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t ql_attn_decode_f32(const AttnDecodeArgs& a, hipStream_t s) {
  const int total = a.B * a.n_q_heads;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_decode_f32_kernel, dim3((total + 63) / 64), dim3(64), 0, s, a);
  return hipGetLastError();
}

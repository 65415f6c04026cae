// RMSNorm over the feature axis, one wave64 per row.
//
// out_j = gamma_j * x_j / sqrt(mean_k x_k^2 + eps), the mean of squares taken
// in fp32 ("推理系统 03：逐项算清一个真实 Qwen3 Transformer 层", §3). Rows are
// independent. The output is bf16 or fp32; an optional second output keeps
// the fp32 value next to a bf16 one (the MoE router takes its top-k decision
// from fp32 inputs).
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kRowsPerBlock = 4;

template <class TIn, class TG, class TOut>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const TIn* __restrict__ x,
                                                      const TG* __restrict__ gamma,
                                                      TOut* __restrict__ out,
                                                      float* __restrict__ out_f32, int rows,
                                                      int d, float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const TIn* xr = x + (size_t)row * d;
  TOut* orow = out + (size_t)row * d;
  float ss = 0.f;
  constexpr bool kVec = sizeof(TIn) == 2 && sizeof(TG) == 2;
  if (kVec && (d % 512) == 0) {
    // 16-byte loads: lane covers 8 consecutive features per 512-wide stripe.
    const int nv = d / 512;
    float v[8];
    for (int i = 0; i < nv; ++i) {
      unpack8(load_bf16x8(reinterpret_cast<const bf16*>(xr) + i * 512 + lane * 8), v);
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += v[j] * v[j];
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)d + eps);
    for (int i = 0; i < nv; ++i) {
      const int c = i * 512 + lane * 8;
      float g[8], o[8];
      unpack8(load_bf16x8(reinterpret_cast<const bf16*>(xr) + c), v);
      unpack8(load_bf16x8(reinterpret_cast<const bf16*>(gamma) + c), g);
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = g[j] * (v[j] * inv);
      if constexpr (sizeof(TOut) == 2) {
        store_bf16x8(reinterpret_cast<bf16*>(orow) + c, pack8(o));
      } else {
        float* of = reinterpret_cast<float*>(orow) + c;
        *reinterpret_cast<f32x4*>(of) = f32x4{o[0], o[1], o[2], o[3]};
        *reinterpret_cast<f32x4*>(of + 4) = f32x4{o[4], o[5], o[6], o[7]};
      }
      if (out_f32) {
        float* of = out_f32 + (size_t)row * d + c;
        *reinterpret_cast<f32x4*>(of) = f32x4{o[0], o[1], o[2], o[3]};
        *reinterpret_cast<f32x4*>(of + 4) = f32x4{o[4], o[5], o[6], o[7]};
      }
    }
    return;
  }
  for (int c = lane; c < d; c += 64) {
    const float v = to_f32(xr[c]);
    ss += v * v;
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)d + eps);
  for (int c = lane; c < d; c += 64) {
    const float o = to_f32(gamma[c]) * (to_f32(xr[c]) * inv);
    orow[c] = from_f32<TOut>(o);
    if (out_f32) out_f32[(size_t)row * d + c] = o;
  }
}

template <class TIn, class TG, class TOut>
hipError_t launch(const TIn* x, const TG* gamma, TOut* out, float* out_f32, int rows, int d,
                  float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL((rmsnorm_kernel<TIn, TG, TOut>), dim3(blocks), dim3(256), 0, s, x, gamma,
                     out, out_f32, rows, d, eps);
  return hipGetLastError();
}

}  // namespace

hipError_t ql_rmsnorm_bf16(const bf16* x, const bf16* gamma, bf16* out, float* out_f32, int rows,
                           int d, float eps, hipStream_t s) {
  return launch<bf16, bf16, bf16>(x, gamma, out, out_f32, rows, d, eps, s);
}
hipError_t ql_rmsnorm_bf16_to_f32(const bf16* x, const bf16* gamma, float* out, int rows, int d,
                                  float eps, hipStream_t s) {
  return launch<bf16, bf16, float>(x, gamma, out, nullptr, rows, d, eps, s);
}
hipError_t ql_rmsnorm_f32in_bf16(const float* x, const bf16* gamma, bf16* out, float* out_f32,
                                 int rows, int d, float eps, hipStream_t s) {
  return launch<float, bf16, bf16>(x, gamma, out, out_f32, rows, d, eps, s);
}
hipError_t ql_rmsnorm_f32(const float* x, const float* gamma, float* out, int rows, int d,
                          float eps, hipStream_t s) {
  return launch<float, float, float>(x, gamma, out, nullptr, rows, d, eps, s);
}

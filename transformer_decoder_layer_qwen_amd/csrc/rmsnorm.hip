// RMSNorm over the feature axis.
//
// out_j = gamma_j * x_j / sqrt(mean_k x_k^2 + eps), the mean of squares taken
// in fp32 ("推理系统 03：逐项算清一个真实 Qwen3 Transformer 层", §3). Rows are
// independent. The output is bf16 or fp32; an optional second output keeps
// the fp32 value next to a bf16 one (the MoE router takes its top-k decision
// from fp32 inputs). HILO stores the fp32 result as a bf16 pair per row,
// [hi | lo] with hi = RNE(o), lo = RNE(o - hi), the form in which the QKV
// projection reads it.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kRowsPerBlock = 4;

// V consecutive elements of T <-> float[V] with one vector memory access.
template <class T, int V> QL_DEV void loadv(const T* p, float* f) {
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int i = 0; i < V; i += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(p + i);
      f[i] = v[0]; f[i + 1] = v[1]; f[i + 2] = v[2]; f[i + 3] = v[3];
    }
  } else if constexpr (V == 8) {
    unpack8(*reinterpret_cast<const bf16x8*>(p), f);
  } else {
    const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = (float)v[i];
  }
}
template <class T, int V> QL_DEV void storev(T* p, const float* f) {
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int i = 0; i < V; i += 4)
      *reinterpret_cast<f32x4*>(p + i) = f32x4{f[i], f[i + 1], f[i + 2], f[i + 3]};
  } else if constexpr (V == 8) {
    *reinterpret_cast<bf16x8*>(p) = pack8(f);
  } else {
    const bf16x4 v = {(bf16)f[0], (bf16)f[1], (bf16)f[2], (bf16)f[3]};
    *reinterpret_cast<bf16x4*>(p) = v;
  }
}

// One block of 256 threads per row; thread t owns the V-wide pieces t, t+256,
// ... (PER of them), all loaded before the reduction so one row costs about
// one memory round trip.
template <class TIn, class TG, class TOut, int PER, bool HILO>
__global__ __launch_bounds__(256) void rmsnorm_row_kernel(const TIn* __restrict__ x,
                                                          const TG* __restrict__ gamma,
                                                          TOut* __restrict__ out,
                                                          float* __restrict__ out_f32, int d,
                                                          float eps) {
  constexpr int V = 16 / sizeof(TIn);
  __shared__ float wsum[4];
  const int tid = threadIdx.x;
  const size_t row = blockIdx.x;
  const TIn* xr = x + row * d;
  float v[PER][V], g[PER][V];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = (tid + 256 * i) * V;
    if (c < d) {
      loadv<TIn, V>(xr + c, v[i]);
      loadv<TG, V>(gamma + c, g[i]);
#pragma unroll
      for (int j = 0; j < V; ++j) ss += v[i][j] * v[i][j];
    }
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) wsum[tid >> 6] = ss;
  __syncthreads();
  const float tot = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  const float inv = 1.0f / sqrtf(tot / (float)d + eps);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = (tid + 256 * i) * V;
    if (c < d) {
      float o[V];
#pragma unroll
      for (int j = 0; j < V; ++j) o[j] = g[i][j] * (v[i][j] * inv);
      if constexpr (HILO) {
        float lo[V];
        TOut* orow = out + row * 2 * d;
#pragma unroll
        for (int j = 0; j < V; ++j) lo[j] = o[j] - (float)(bf16)o[j];
        storev<TOut, V>(orow + c, o);
        storev<TOut, V>(orow + d + c, lo);
        if (out_f32) storev<float, V>(out_f32 + row * d + c, o);
      } else {
        storev<TOut, V>(out + row * d + c, o);
        if (out_f32) storev<float, V>(out_f32 + row * d + c, o);
      }
    }
  }
}

// Any d: one wave per row, strided scalar accesses.
template <class TIn, class TG, class TOut, bool HILO>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const TIn* __restrict__ x,
                                                      const TG* __restrict__ gamma,
                                                      TOut* __restrict__ out,
                                                      float* __restrict__ out_f32, int rows,
                                                      int d, float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const TIn* xr = x + (size_t)row * d;
  TOut* orow = out + (size_t)row * (HILO ? 2 * d : d);
  float ss = 0.f;
  for (int c = lane; c < d; c += 64) {
    const float v = to_f32(xr[c]);
    ss += v * v;
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)d + eps);
  for (int c = lane; c < d; c += 64) {
    const float o = to_f32(gamma[c]) * (to_f32(xr[c]) * inv);
    orow[c] = from_f32<TOut>(o);
    if constexpr (HILO) orow[d + c] = from_f32<TOut>(o - to_f32(from_f32<TOut>(o)));
    if (out_f32) out_f32[(size_t)row * d + c] = o;
  }
}

template <class TIn, class TG, class TOut, bool HILO = false>
hipError_t launch(const TIn* x, const TG* gamma, TOut* out, float* out_f32, int rows, int d,
                  float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  constexpr int V = 16 / sizeof(TIn);
  const int per = (d + 256 * V - 1) / (256 * V);
  if (d % V == 0 && per <= 8) {
#define QL_RMS_CASE(P)                                                                    \
  if (per <= P) {                                                                         \
    hipLaunchKernelGGL((rmsnorm_row_kernel<TIn, TG, TOut, P, HILO>), dim3(rows), dim3(256), 0, s, \
                       x, gamma, out, out_f32, d, eps);                                   \
    return hipGetLastError();                                                             \
  }
    QL_RMS_CASE(1)
    QL_RMS_CASE(2)
    QL_RMS_CASE(4)
    QL_RMS_CASE(8)
#undef QL_RMS_CASE
  }
  const int blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL((rmsnorm_kernel<TIn, TG, TOut, HILO>), dim3(blocks), dim3(256), 0, s, x, gamma,
                     out, out_f32, rows, d, eps);
  return hipGetLastError();
}

}  // namespace

hipError_t ql_rmsnorm_bf16(const bf16* x, const bf16* gamma, bf16* out, float* out_f32, int rows,
                           int d, float eps, hipStream_t s) {
  return launch<bf16, bf16, bf16>(x, gamma, out, out_f32, rows, d, eps, s);
}
hipError_t ql_rmsnorm_bf16_to_hilo(const bf16* x, const bf16* gamma, bf16* out, int rows, int d,
                                   float eps, hipStream_t s, float* out_f32) {
  return launch<bf16, bf16, bf16, true>(x, gamma, out, out_f32, rows, d, eps, s);
}

namespace {
__global__ __launch_bounds__(256) void hilo_to_f32_kernel(const bf16* __restrict__ hl, int rows,
                                                          int cols, float* __restrict__ out) {
  const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (i >= (size_t)rows * cols) return;
  const size_t r = i / cols, c = i % cols;
  out[i] = (float)hl[r * 2 * cols + c] + (float)hl[r * 2 * cols + cols + c];
}
}  // namespace

hipError_t ql_hilo_to_f32(const bf16* hl, int rows, int cols, float* out, hipStream_t s) {
  const size_t n = (size_t)rows * cols;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(hilo_to_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, hl,
                     rows, cols, out);
  return hipGetLastError();
}
hipError_t ql_rmsnorm_f32in_bf16(const float* x, const bf16* gamma, bf16* out, float* out_f32,
                                 int rows, int d, float eps, hipStream_t s) {
  return launch<float, bf16, bf16>(x, gamma, out, out_f32, rows, d, eps, s);
}
hipError_t ql_rmsnorm_f32_to_hilo(const float* x, const bf16* gamma, bf16* out, int rows, int d,
                                  float eps, hipStream_t s, float* out_f32) {
  return launch<float, bf16, bf16, true>(x, gamma, out, out_f32, rows, d, eps, s);
}

namespace {
__global__ __launch_bounds__(256) void bf16_to_f32_kernel(const bf16* __restrict__ x, size_t n,
                                                          float* __restrict__ out) {
  const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (i < n) out[i] = (float)x[i];
}
}  // namespace

hipError_t ql_bf16_to_f32(const bf16* x, size_t n, float* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(bf16_to_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, n,
                     out);
  return hipGetLastError();
}
hipError_t ql_rmsnorm_f32(const float* x, const float* gamma, float* out, int rows, int d,
                          float eps, hipStream_t s) {
  return launch<float, float, float>(x, gamma, out, nullptr, rows, d, eps, s);
}

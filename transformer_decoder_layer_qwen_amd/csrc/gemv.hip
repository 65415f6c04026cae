// Decode projections for one to four token rows: y = X W^T on the vector ALUs.
//
// With so few rows the layer reads each weight byte once and does a couple of
// FLOPs per byte ("Qwen2.5-7B 结构拆解" §03.6: one token costs 2 FLOPs per
// weight), so what matters is how the weights stream from HBM. Every load
// instruction of a wave reads 1 KiB of ONE weight row (lane l takes bytes
// [16 l, 16 l + 16) of a 512-element chunk): whole cache lines, in order.
// A block owns R output rows (2R weight rows for SwiGLU); its NW waves take the
// K chunks round-robin, each keeping U chunks x R rows of loads in flight, and
// meet in LDS at the end. Products and sums are fp32; fp32 inputs are used as
// they are, so no hi/lo split is needed on this path.
//
// X forms: bf16 rows; fp32 rows (the attention output); bf16 rows times a bf16
// gamma (RMSNorm1 folded into the QKV projection: the per-row 1/rms and the
// bias are applied by the consumer of the raw sums); fp32 rows times a bf16
// gamma with RMSNorm applied in the epilogue (RMSNorm2 folded into the gate/up
// projection: the block reads every element of its X rows anyway, so it sums
// their squares on the way and scales the dot products by 1/rms at the end).
// Epilogues: RAW out_f32 = acc; RESID_F32 out_f32 = resid_bf16 + acc;
// RESID_OUT out = bf16(resid_f32 + acc); SWIGLU out = bf16(SiLU(g) * u).
#include "common.h"
#include "kernels.h"

namespace {

enum : int { GV_RAW = 0, GV_RESID_F32, GV_RESID_OUT, GV_SWIGLU };
enum : int { GX_BF16 = 0, GX_F32, GX_GAMMA, GX_F32_NORM };

constexpr int kChunk = 512;  // elements of K per wave step (64 lanes x 8)

struct GemvArgs {
  const bf16* X;
  const float* Xf;
  const bf16* gam;
  int K;
  const bf16* W;   // [N, K]
  const bf16* W2;  // SWIGLU: up; RAW: rows [seg1, seg2)
  const bf16* W3;  // RAW: rows [seg2, N)
  int seg1, seg2;
  int N;
  float* out_f32;
  bf16* out_bf16;
  const bf16* resid_bf16;
  const float* resid_f32;
  float eps;       // GX_F32_NORM, GX_GAMMA
  float* inv_out;  // GX_GAMMA: [M] 1/rms of the raw X rows (written by block 0), or NULL
};

// Eight weights. Each weight byte is read once per call, so the loads carry
// the non-temporal hint: the stream does not displace the activations and
// other lines from the caches (Qwen2.5-7B batch-1 layer 102.6 -> 95.8 us).
QL_DEV bf16x8 load_w(const bf16* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p));
}

// Eight raw X values of row m at columns k + 8 lane .. +7 (zeros where !ok).
template <int XM>
QL_DEV void load_x(const GemvArgs& p, int m, int k, int lane, bool ok, float* xv) {
  const size_t off = (size_t)m * p.K + k + lane * 8;
  if (!ok) {
#pragma unroll
    for (int j = 0; j < 8; ++j) xv[j] = 0.f;
    return;
  }
  if constexpr (XM == GX_F32 || XM == GX_F32_NORM) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p.Xf + off);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p.Xf + off + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xv[j] = a[j];
      xv[j + 4] = b[j];
    }
  } else {
    unpack8(load_bf16x8(p.X + off), xv);
  }
}

template <int M, int MODE, int XM, int R, int NW, int U>
__global__ __launch_bounds__(NW * 64) void gemv_kernel(const GemvArgs p) {
  constexpr int NOUT = MODE == GV_SWIGLU ? 2 : 1;
  constexpr int NS = NOUT * R;  // weight-row streams of the block
  __shared__ float red[NW][NS][M];
  __shared__ float red_ss[NW][M];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n0 = blockIdx.x * R;

  // QKV: the block's rows lie inside one of the three weight matrices
  const bf16* Wm = p.W;
  int nb = n0;
  if constexpr (MODE == GV_RAW) {
    if (n0 >= p.seg2) {
      Wm = p.W3;
      nb = n0 - p.seg2;
    } else if (n0 >= p.seg1) {
      Wm = p.W2;
      nb = n0 - p.seg1;
    }
  }
  const bf16* rows[NS];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    rows[r] = Wm + (size_t)(nb + r) * p.K + lane * 8;
    if constexpr (NOUT == 2) rows[R + r] = p.W2 + (size_t)(n0 + r) * p.K + lane * 8;
  }

  float acc[NS][M];
#pragma unroll
  for (int i = 0; i < NS; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[i][m] = 0.f;
  float ss[M];  // GX_GAMMA, GX_F32_NORM: sum of squares of this wave's raw X elements
#pragma unroll
  for (int m = 0; m < M; ++m) ss[m] = 0.f;
  // X values of one chunk for every row, ready for the dot products
  auto get_x = [&](int k, bool ok, float (&xv)[M][8]) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      load_x<XM>(p, m, k, lane, ok, xv[m]);
      if constexpr (XM == GX_GAMMA || XM == GX_F32_NORM) {
        float g[8];
        if (ok) {
          unpack8(load_bf16x8(p.gam + k + lane * 8), g);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) g[j] = 0.f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          ss[m] += xv[m][j] * xv[m][j];
          xv[m][j] *= g[j];
        }
      }
    }
  };

  const int nfull = p.K / kChunk;
  int c = wave;
  for (; c + (U - 1) * NW < nfull; c += U * NW) {
    bf16x8 w[U][NS];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < NS; ++i) w[u][i] = load_w(rows[i] + (c + u * NW) * kChunk);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float xv[M][8];
      get_x((c + u * NW) * kChunk, true, xv);
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        float wf[8];
        unpack8(w[u][i], wf);
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[i][m] += wf[j] * xv[m][j];
      }
    }
  }
  // leftover full chunks, then the ragged tail chunk (K % 512 elements)
  const int tail = p.K - nfull * kChunk;
  const int last = tail > 0 ? nfull + 1 : nfull;
  for (; c < last; c += NW) {
    const int k = c * kChunk;
    const bool ok = c < nfull || lane * 8 < tail;
    bf16x8 w[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (ok) {
        w[i] = load_w(rows[i] + k);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) w[i][j] = (bf16)0.f;
      }
    }
    float xv[M][8];
    get_x(k, ok, xv);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      float wf[8];
      unpack8(w[i], wf);
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][m] += wf[j] * xv[m][j];
    }
  }

#pragma unroll
  for (int i = 0; i < NS; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float v = wave_sum(acc[i][m]);
      if (lane == 0) red[wave][i][m] = v;
    }
  if constexpr (XM == GX_F32_NORM || XM == GX_GAMMA) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float v = wave_sum(ss[m]);
      if (lane == 0) red_ss[wave][m] = v;
    }
  }
  __syncthreads();
  if constexpr (XM == GX_GAMMA) {
    if (p.inv_out && blockIdx.x == 0 && tid < M) {
      float t = 0.f;
#pragma unroll
      for (int q = 0; q < NW; ++q) t += red_ss[q][tid];
      p.inv_out[tid] = 1.0f / sqrtf(t / (float)p.K + p.eps);
    }
  }
  if (tid < R * M) {
    const int r = tid / M, m = tid % M;
    float v[NOUT];
#pragma unroll
    for (int o = 0; o < NOUT; ++o) {
      float t = 0.f;
#pragma unroll
      for (int q = 0; q < NW; ++q) t += red[q][o * R + r][m];
      v[o] = t;
    }
    if constexpr (XM == GX_F32_NORM) {
      float t = 0.f;
#pragma unroll
      for (int q = 0; q < NW; ++q) t += red_ss[q][m];
      const float inv = 1.0f / sqrtf(t / (float)p.K + p.eps);
#pragma unroll
      for (int o = 0; o < NOUT; ++o) v[o] *= inv;
    }
    const size_t oi = (size_t)m * p.N + n0 + r;
    if constexpr (MODE == GV_RAW) {
      p.out_f32[oi] = v[0];
    } else if constexpr (MODE == GV_RESID_F32) {
      p.out_f32[oi] = to_f32(p.resid_bf16[oi]) + v[0];
    } else if constexpr (MODE == GV_RESID_OUT) {
      p.out_bf16[oi] = (bf16)(p.resid_f32[oi] + v[0]);
    } else {
      p.out_bf16[oi] = (bf16)(silu_f32(v[0]) * v[1]);
    }
  }
}

template <int MODE, int XM, int R, int NW, int U>
hipError_t launch_cfg(const GemvArgs& a, int M, hipStream_t s) {
  const dim3 grid(a.N / R), block(NW * 64);
  switch (M) {
    case 1: hipLaunchKernelGGL((gemv_kernel<1, MODE, XM, R, NW, U>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((gemv_kernel<2, MODE, XM, R, NW, U>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((gemv_kernel<3, MODE, XM, R, NW, U>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((gemv_kernel<4, MODE, XM, R, NW, U>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Launch shapes, the best of sweeps over (rows per block, waves, chunks in
// flight per row stream) on the batch-1 projections of d = 3584 / ffn = 18944
// with non-temporal weight loads: gate/up takes four output rows (eight
// weight row streams) with one chunk in flight each, 38.9 us for 272 MB
// (two rows and two chunks: 43.4 us); Q/K/V, O and down take two rows, four
// waves and two chunks (6.5, 4.3 and 19.7 us; no other shape tried was
// faster on them).
template <int MODE, int XM>
hipError_t launch(const GemvArgs& a, int M, hipStream_t s) {
  if (a.N <= 0) return hipSuccess;
  if constexpr (MODE == GV_SWIGLU) {
    if (a.N % 4 == 0) return launch_cfg<MODE, XM, 4, 4, 1>(a, M, s);
  }
  return launch_cfg<MODE, XM, 2, 4, 2>(a, M, s);
}

GemvArgs base(const bf16* X, int K, const bf16* W, int N) {
  GemvArgs a{};
  a.X = X;
  a.K = K;
  a.W = W;
  a.N = N;
  a.seg1 = a.seg2 = 0x7fffffff;
  return a;
}

}  // namespace

bool ql_gemv_ok(int M, int N, int K) {
  return M >= 1 && M <= kGemvMaxRows && N % 2 == 0 && K % 8 == 0;
}

hipError_t ql_gemv_qkv_raw(const bf16* x, const bf16* gamma, int M, const bf16* Wq,
                           const bf16* Wk, const bf16* Wv, int q, int kv, int K, float* out,
                           float eps, float* inv_rms, hipStream_t s) {
  GemvArgs a = base(x, K, Wq, q + 2 * kv);
  a.gam = gamma;
  a.eps = eps;
  a.inv_out = inv_rms;
  a.W2 = Wk;
  a.W3 = Wv;
  a.seg1 = q;
  a.seg2 = q + kv;
  a.out_f32 = out;
  return launch<GV_RAW, GX_GAMMA>(a, M, s);
}

hipError_t ql_gemv_resid_f32(const float* X, int M, const bf16* W, int N, int K,
                             const bf16* resid, float* out, hipStream_t s) {
  GemvArgs a = base(nullptr, K, W, N);
  a.Xf = X;
  a.resid_bf16 = resid;
  a.out_f32 = out;
  return launch<GV_RESID_F32, GX_F32>(a, M, s);
}

hipError_t ql_gemv_resid_out(const bf16* X, int M, const bf16* W, int N, int K,
                             const float* resid, bf16* out, hipStream_t s) {
  GemvArgs a = base(X, K, W, N);
  a.resid_f32 = resid;
  a.out_bf16 = out;
  return launch<GV_RESID_OUT, GX_BF16>(a, M, s);
}

hipError_t ql_gemv_rmsnorm_swiglu(const float* R, const bf16* gamma, float eps, int M,
                                  const bf16* Wg, const bf16* Wu, int F, int K, bf16* out,
                                  hipStream_t s) {
  GemvArgs a = base(nullptr, K, Wg, F);
  a.Xf = R;
  a.gam = gamma;
  a.eps = eps;
  a.W2 = Wu;
  a.out_bf16 = out;
  return launch<GV_SWIGLU, GX_F32_NORM>(a, M, s);
}

// Decode projections with few token rows (M = batch <= 128): C = X * W^T.
//
// One decode step multiplies a handful of new-token rows by every weight
// matrix ("Qwen2.5-7B 结构拆解" §09.1: h[1,3584] @ W_q ...), so the weight
// bytes dominate and each weight byte should cross HBM exactly once.
//
// Design: a block owns 16 weight rows (16 output features; 16 gate + 16 up
// rows for SwiGLU) and splits K over its 8 waves. A wave streams its K-slice
// of the 16 rows straight from global memory as the MFMA "A" operand (one
// 16-byte load per lane per 32-wide k step), while the token rows X are the
// "B" operand (up to MT tiles of 16 tokens, read through L2). The 8 partial
// tiles are summed through LDS and the fused epilogue writes the output:
//   F32_BIAS (Q/K/V + bias), RESID_F32 (R = X + A), RESID_OUT (Y = R + F),
//   SWIGLU (H = SiLU(gate) * up) -- same epilogues as the prefill GEMM.
// As in the prefill GEMM, the RMSNorm1 output and the attention output enter
// the Q/K/V and O projections as fp32 rows split into a bf16 hi + lo pair (two
// MFMAs per weight fragment; the kernel stays bound by the weight stream).
#include "common.h"
#include "kernels.h"

namespace {

enum : int { SK_F32_BIAS = 0, SK_RESID_F32, SK_RESID_OUT, SK_SWIGLU };

constexpr int kWaves = 8;

struct SkinnyArgs {
  const bf16* X;   // [M, K]
  const float* Xf; // [M, K] fp32 rows, used as a bf16 hi + lo pair
  int M;
  int K;
  const bf16* W;   // [N, K]
  const bf16* W2;  // SwiGLU: up matrix; F32_BIAS: rows [seg1, seg2)
  const bf16* W3;  // F32_BIAS: rows [seg2, N)
  int seg1, seg2;
  float* out_f32;
  bf16* out_bf16;
  int ldo;
  const bf16* bias;
  const bf16* bias2;
  const bf16* bias3;
  const bf16* resid_bf16;
  const float* resid_f32;
  int ldr;
};

template <int MT, int MODE, bool XF32>
__global__ __launch_bounds__(512) void skinny_kernel(const SkinnyArgs p) {
  constexpr int NOUT = (MODE == SK_SWIGLU) ? 2 : 1;
  __shared__ __attribute__((aligned(16))) float red[kWaves * NOUT * MT * 256];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n0 = blockIdx.x * 16;
  const int g = lane >> 4;
  const int ksteps = p.K / 32;                    // K % 32 == 0
  const int per = (ksteps + kWaves - 1) / kWaves;
  const int nks = max(0, min(per, ksteps - wave * per));
  const int kbeg = wave * per * 32;

  // QKV: the 16 rows of a block lie inside one of the three weight matrices
  const bf16* Wm = p.W;
  const bf16* bias = p.bias;
  int nb = n0;
  if constexpr (MODE == SK_F32_BIAS) {
    if (n0 >= p.seg2) {
      Wm = p.W3;
      bias = p.bias3;
      nb = n0 - p.seg2;
    } else if (n0 >= p.seg1) {
      Wm = p.W2;
      bias = p.bias2;
      nb = n0 - p.seg1;
    }
  }
  const bf16* wrow = Wm + (size_t)(nb + (lane & 15)) * p.K + kbeg + g * 8;
  const bf16* wrow2 = nullptr;
  if constexpr (NOUT == 2) wrow2 = p.W2 + (size_t)(n0 + (lane & 15)) * p.K + kbeg + g * 8;
  size_t xoff[MT];
  bool xval[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + (lane & 15);
    xval[mt] = m < p.M;
    xoff[mt] = (size_t)(xval[mt] ? m : 0) * p.K + kbeg + g * 8;
  }
  // B operand for k step ks: bf16 row piece, or fp32 split into (hi, lo)
  auto xload = [&](int mt, int ks, bf16x8& hi, bf16x8& lo) {
    if constexpr (XF32) {
      if (!xval[mt]) {
        hi = bf16x8{};
        lo = bf16x8{};
        return;
      }
      const float* src = p.Xf + xoff[mt] + ks * 32;
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(src);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hi[i] = (bf16)v0[i];
        hi[i + 4] = (bf16)v1[i];
        lo[i] = (bf16)(v0[i] - (float)hi[i]);
        lo[i + 4] = (bf16)(v1[i] - (float)hi[i + 4]);
      }
    } else {
      hi = xval[mt] ? load_bf16x8(p.X + xoff[mt] + ks * 32) : bf16x8{};
    }
  };

  f32x4 acc[NOUT][MT];
#pragma unroll
  for (int o = 0; o < NOUT; ++o)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[o][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int XT = XF32 ? 2 : 1;
  constexpr int U = (MT * XT <= 2) ? 8 : (MT * XT <= 4 ? 4 : 2);
  int ks = 0;
  for (; ks + U <= nks; ks += U) {
    bf16x8 wa[U], wb[U], xa[U][MT][XT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      wa[u] = load_bf16x8(wrow + (ks + u) * 32);
      if constexpr (NOUT == 2) wb[u] = load_bf16x8(wrow2 + (ks + u) * 32);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) xload(mt, ks + u, xa[u][mt][0], xa[u][mt][XT - 1]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < XT; ++t) {
          acc[0][mt] = mfma_16x16x32(wa[u], xa[u][mt][t], acc[0][mt]);
          if constexpr (NOUT == 2)
            acc[1][mt] = mfma_16x16x32(wb[u], xa[u][mt][t], acc[1][mt]);
        }
  }
  for (; ks < nks; ++ks) {
    const bf16x8 wa = load_bf16x8(wrow + ks * 32);
    bf16x8 wb;
    if constexpr (NOUT == 2) wb = load_bf16x8(wrow2 + ks * 32);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      bf16x8 xa[XT];
      xload(mt, ks, xa[0], xa[XT - 1]);
#pragma unroll
      for (int t = 0; t < XT; ++t) {
        acc[0][mt] = mfma_16x16x32(wa, xa[t], acc[0][mt]);
        if constexpr (NOUT == 2) acc[1][mt] = mfma_16x16x32(wb, xa[t], acc[1][mt]);
      }
    }
  }

  // lane holds D[n = 4*(lane/16) + r][m = mt*16 + lane%16]
#pragma unroll
  for (int o = 0; o < NOUT; ++o)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        red[((wave * NOUT + o) * MT + mt) * 256 + r * 64 + lane] = acc[o][mt][r];
  __syncthreads();

  for (int e = tid; e < 16 * 16 * MT; e += 512) {
    const int nl = e & 15;
    const int m = e >> 4;
    if (m >= p.M) continue;
    const int mt = m >> 4;
    const int src = (nl & 3) * 64 + (m & 15) + 16 * (nl >> 2);
    float v[NOUT];
#pragma unroll
    for (int o = 0; o < NOUT; ++o) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) s += red[((w * NOUT + o) * MT + mt) * 256 + src];
      v[o] = s;
    }
    const int n = n0 + nl;
    const size_t oi = (size_t)m * p.ldo + n;
    if constexpr (MODE == SK_F32_BIAS) {
      p.out_f32[oi] = v[0] + (bias ? to_f32(bias[nb + nl]) : 0.f);
    } else if constexpr (MODE == SK_RESID_F32) {
      p.out_f32[oi] = to_f32(p.resid_bf16[(size_t)m * p.ldr + n]) + v[0];
    } else if constexpr (MODE == SK_RESID_OUT) {
      p.out_bf16[oi] = (bf16)(p.resid_f32[(size_t)m * p.ldr + n] + v[0]);
    } else {
      p.out_bf16[oi] = (bf16)(silu_f32(v[0]) * v[1]);
    }
  }
}

template <int MODE, bool XF32 = false>
hipError_t launch(const SkinnyArgs& a, int N, hipStream_t s) {
  const int blocks = N / 16;
  if (blocks <= 0 || a.M <= 0) return hipSuccess;
  const int mt = (a.M + 15) / 16;
#define QL_SK_CASE(V)                                                                      \
  case V:                                                                                  \
    hipLaunchKernelGGL((skinny_kernel<V, MODE, XF32>), dim3(blocks), dim3(512), 0, s, a); \
    break;
  switch (mt) {
    QL_SK_CASE(1)
    QL_SK_CASE(2)
    QL_SK_CASE(3)
    QL_SK_CASE(4)
    QL_SK_CASE(5)
    QL_SK_CASE(6)
    QL_SK_CASE(7)
    QL_SK_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef QL_SK_CASE
  return hipGetLastError();
}

SkinnyArgs args(const bf16* X, int M, int K, const bf16* W) {
  SkinnyArgs a{};
  a.X = X;
  a.seg1 = a.seg2 = 0x7fffffff;
  a.M = M;
  a.K = K;
  a.W = W;
  return a;
}

}  // namespace

hipError_t ql_skinny_qkv(const float* X, int M, const bf16* Wq, const bf16* Wk, const bf16* Wv,
                         int q, int kv, int K, const bf16* bq, const bf16* bk, const bf16* bv,
                         float* out, hipStream_t s) {
  const int N = q + 2 * kv;
  SkinnyArgs a = args(nullptr, M, K, Wq);
  a.Xf = X;
  a.W2 = Wk;
  a.W3 = Wv;
  a.seg1 = q;
  a.seg2 = q + kv;
  a.bias = bq;
  a.bias2 = bk;
  a.bias3 = bv;
  a.out_f32 = out;
  a.ldo = N;
  return launch<SK_F32_BIAS, true>(a, N, s);
}

hipError_t ql_skinny_resid_f32(const float* X, int M, const bf16* W, int N, int K,
                               const bf16* resid, float* out, hipStream_t s) {
  SkinnyArgs a = args(nullptr, M, K, W);
  a.Xf = X;
  a.resid_bf16 = resid;
  a.ldr = N;
  a.out_f32 = out;
  a.ldo = N;
  return launch<SK_RESID_F32, true>(a, N, s);
}

hipError_t ql_skinny_resid_out(const bf16* X, int M, const bf16* W, int N, int K,
                               const float* resid, bf16* out, hipStream_t s) {
  SkinnyArgs a = args(X, M, K, W);
  a.resid_f32 = resid;
  a.ldr = N;
  a.out_bf16 = out;
  a.ldo = N;
  return launch<SK_RESID_OUT>(a, N, s);
}

hipError_t ql_skinny_swiglu(const bf16* X, int M, const bf16* Wg, const bf16* Wu, int F, int K,
                            bf16* out, hipStream_t s) {
  SkinnyArgs a = args(X, M, K, Wg);
  a.W2 = Wu;
  a.out_bf16 = out;
  a.ldo = F;
  return launch<SK_SWIGLU>(a, F, s);
}

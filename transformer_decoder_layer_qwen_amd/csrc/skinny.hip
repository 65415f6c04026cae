// Decode projections with few token rows (M = batch <= 128): C = X * W^T.
//
// One decode step multiplies a handful of new-token rows by every weight
// matrix ("Qwen2.5-7B 结构拆解" §09.1: h[1,3584] @ W_q ...), so the weight
// bytes dominate and each weight byte should cross HBM exactly once, with
// enough loads in flight to keep HBM busy.
//
// Work unit: a tile of 16 weight rows (16 output features; 16 gate + 16 up
// rows for SwiGLU). The weight rows are the MFMA "A" operand, loaded straight
// from global memory (one 16-byte load per lane per 32-wide k step, issued in
// unrolled batches); the token rows X are the "B" operand (up to MT tiles of
// 16 tokens, served from L2). A block of NW waves (4, 8 or 16) splits K; the
// NW partial tiles are summed through LDS and the epilogue writes the output
// directly. Few tiles (QKV, O, down) get 16 waves per block so that every CU
// still has many weight bytes in flight; many tiles (gate/up) get 4.
//
// X operand forms:
//   X_BF16   bf16 rows
//   X_F32    fp32 rows carried as a bf16 hi + lo pair (two MFMAs per weight
//            fragment): the attention output entering the O projection
//   X_GAMMA  bf16 rows times a bf16 gamma: x*gamma is exact in fp32 (16
//            significant bits) and so is its hi + lo split. The QKV
//            projection takes RMSNorm1 in this form; the per-row 1/rms is
//            applied by the consumer of the raw sums.
// Epilogues:
//   RAW        out_f32 = acc                    (QKV; scaled and biased later)
//   RESID_F32  out_f32 = resid_bf16 + acc       (R = X + A)
//   RESID_OUT  out     = bf16(resid_f32 + acc)  (Y = R + F)
//   SWIGLU     out     = bf16(SiLU(g) * u)      (H)
#include "common.h"
#include "kernels.h"

namespace {

enum : int { SK_RAW = 0, SK_RESID_F32, SK_RESID_OUT, SK_SWIGLU };
enum : int { X_BF16 = 0, X_F32, X_GAMMA };

struct SkinnyArgs {
  const bf16* X;    // [M, K] (X_BF16, X_GAMMA)
  const float* Xf;  // [M, K] (X_F32)
  const bf16* gam;  // [K] (X_GAMMA)
  int M;
  int K;
  const bf16* W;    // [N, K]
  const bf16* W2;   // SWIGLU: up matrix; RAW: rows [seg1, seg2)
  const bf16* W3;   // RAW: rows [seg2, N)
  int seg1, seg2;
  int N;
  float* out_f32;
  bf16* out_bf16;
  const bf16* resid_bf16;
  const float* resid_f32;
};

template <int MT, int MODE, int XM, int NW>
__global__ __launch_bounds__(NW * 64) void skinny_kernel(const SkinnyArgs p) {
  constexpr int NOUT = (MODE == SK_SWIGLU) ? 2 : 1;
  constexpr int XT = (XM == X_BF16) ? 1 : 2;
  constexpr int U = (MT * XT <= 2) ? 8 : (MT * XT <= 4 ? 4 : 2);
  __shared__ __attribute__((aligned(16))) float red[NW * NOUT * MT * 256];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n0 = blockIdx.x * 16;
  const int g = lane >> 4;

  // this wave's share of K (in 32-wide steps)
  const int ksteps = p.K / 32;
  const int per_w = (ksteps + NW - 1) / NW;
  const int w0 = wave * per_w;
  const int nks = max(0, min(per_w, ksteps - w0));
  const int kbeg = w0 * 32;

  // QKV: the 16 rows of a tile lie inside one of the three weight matrices
  const bf16* Wm = p.W;
  int nb_row = n0;
  if constexpr (MODE == SK_RAW) {
    if (n0 >= p.seg2) {
      Wm = p.W3;
      nb_row = n0 - p.seg2;
    } else if (n0 >= p.seg1) {
      Wm = p.W2;
      nb_row = n0 - p.seg1;
    }
  }
  const bf16* wrow = Wm + (size_t)(nb_row + (lane & 15)) * p.K + kbeg + g * 8;
  const bf16* wrow2 = nullptr;
  if constexpr (NOUT == 2) wrow2 = p.W2 + (size_t)(n0 + (lane & 15)) * p.K + kbeg + g * 8;
  // token rows: lanes past M read row 0 and multiply by a zero mask, so every
  // load is unconditional and the loads of a batch stay in flight together
  size_t xoff[MT];
  float xmask[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + (lane & 15);
    xmask[mt] = m < p.M ? 1.f : 0.f;
    xoff[mt] = (size_t)(m < p.M ? m : 0) * p.K + kbeg + g * 8;
  }
  auto split = [&](const float* v, bf16x8* out) {
    bf16x8 hi, lo;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      hi[i] = (bf16)v[i];
      lo[i] = (bf16)(v[i] - (float)hi[i]);
    }
    out[0] = hi;
    out[XT - 1] = lo;
  };
  auto xload = [&](int mt, int ks, bf16x8* out) {
    float f[8];
    if constexpr (XM == X_F32) {
      const float* src = p.Xf + xoff[mt] + ks * 32;
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(src);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[i] = v0[i] * xmask[mt];
        f[i + 4] = v1[i] * xmask[mt];
      }
      split(f, out);
    } else if constexpr (XM == X_GAMMA) {
      float gm[8];
      unpack8(load_bf16x8(p.X + xoff[mt] + ks * 32), f);
      unpack8(load_bf16x8(p.gam + kbeg + g * 8 + ks * 32), gm);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] *= gm[i] * xmask[mt];
      split(f, out);
    } else {
      unpack8(load_bf16x8(p.X + xoff[mt] + ks * 32), f);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] *= xmask[mt];
      out[0] = pack8(f);
    }
  };

  f32x4 acc[NOUT][MT];
#pragma unroll
  for (int o = 0; o < NOUT; ++o)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[o][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  int ks = 0;
  for (; ks + U <= nks; ks += U) {
    bf16x8 wa[U], wb[U], xa[U][MT][XT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      wa[u] = load_bf16x8(wrow + (ks + u) * 32);
      if constexpr (NOUT == 2) wb[u] = load_bf16x8(wrow2 + (ks + u) * 32);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) xload(mt, ks + u, xa[u][mt]);
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
      xload(mt, ks, xa);
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

  for (int e = tid; e < 16 * 16 * MT; e += NW * 64) {
    const int nl = e & 15;
    const int m = e >> 4;
    if (m >= p.M) continue;
    const int src = (nl & 3) * 64 + (m & 15) + 16 * (nl >> 2);
    float v[NOUT];
#pragma unroll
    for (int o = 0; o < NOUT; ++o) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) s += red[((w * NOUT + o) * MT + (m >> 4)) * 256 + src];
      v[o] = s;
    }
    const int n = n0 + nl;
    const size_t oi = (size_t)m * p.N + n;
    if constexpr (MODE == SK_RAW) {
      p.out_f32[oi] = v[0];
    } else if constexpr (MODE == SK_RESID_F32) {
      p.out_f32[oi] = to_f32(p.resid_bf16[oi]) + v[0];
    } else if constexpr (MODE == SK_RESID_OUT) {
      p.out_bf16[oi] = (bf16)(p.resid_f32[oi] + v[0]);
    } else {
      p.out_bf16[oi] = (bf16)(silu_f32(v[0]) * v[1]);
    }
  }
}

// Waves per block: about 4096 waves over the whole launch (so every CU has
// many weight loads in flight), at least 4 k-steps per wave, and at most
// 64 KiB of LDS for the cross-wave reduction.
int choose_waves(int tiles, int K, int nout, int mt) {
  int nw = 4;
  while (nw < 16 && tiles * nw < 4096 && (K / 32) / (nw * 2) >= 4 &&
         nw * 2 * nout * mt <= 64)
    nw *= 2;
  return nw;
}

template <int MODE, int XM, int MT, int W>
hipError_t launch_one(const SkinnyArgs& a, int tiles, hipStream_t s) {
  constexpr int NOUT = MODE == SK_SWIGLU ? 2 : 1;
  if constexpr (W * NOUT * MT <= 64) {  // reduction buffer within 64 KiB of LDS
    hipLaunchKernelGGL((skinny_kernel<MT, MODE, XM, W>), dim3(tiles), dim3(W * 64), 0, s, a);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

template <int MODE, int XM>
hipError_t launch(SkinnyArgs a, int N, hipStream_t s) {
  const int tiles = N / 16;
  if (tiles <= 0 || a.M <= 0) return hipSuccess;
  const int mt = (a.M + 15) / 16;
  a.N = N;
  const int nw = choose_waves(tiles, a.K, MODE == SK_SWIGLU ? 2 : 1, mt);
#define QL_SK(V, W) \
  if (mt == V && nw == W) return launch_one<MODE, XM, V, W>(a, tiles, s);
#define QL_SK_MT(V) QL_SK(V, 4) QL_SK(V, 8) QL_SK(V, 16)
  QL_SK_MT(1)
  QL_SK_MT(2)
  QL_SK_MT(3)
  QL_SK_MT(4)
  QL_SK_MT(5)
  QL_SK_MT(6)
  QL_SK_MT(7)
  QL_SK_MT(8)
#undef QL_SK_MT
#undef QL_SK
  return hipErrorInvalidValue;
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

hipError_t ql_skinny_qkv_raw(const bf16* x, const bf16* gamma, int M, const bf16* Wq,
                             const bf16* Wk, const bf16* Wv, int q, int kv, int K, float* out,
                             hipStream_t s) {
  SkinnyArgs a = args(x, M, K, Wq);
  a.gam = gamma;
  a.W2 = Wk;
  a.W3 = Wv;
  a.seg1 = q;
  a.seg2 = q + kv;
  a.out_f32 = out;
  return launch<SK_RAW, X_GAMMA>(a, q + 2 * kv, s);
}

hipError_t ql_skinny_resid_f32(const float* X, int M, const bf16* W, int N, int K,
                               const bf16* resid, float* out, hipStream_t s) {
  SkinnyArgs a = args(nullptr, M, K, W);
  a.Xf = X;
  a.resid_bf16 = resid;
  a.out_f32 = out;
  return launch<SK_RESID_F32, X_F32>(a, N, s);
}

hipError_t ql_skinny_resid_out(const bf16* X, int M, const bf16* W, int N, int K,
                               const float* resid, bf16* out, hipStream_t s) {
  SkinnyArgs a = args(X, M, K, W);
  a.resid_f32 = resid;
  a.out_bf16 = out;
  return launch<SK_RESID_OUT, X_BF16>(a, N, s);
}

hipError_t ql_skinny_swiglu(const bf16* X, int M, const bf16* Wg, const bf16* Wu, int F, int K,
                            bf16* out, hipStream_t s) {
  SkinnyArgs a = args(X, M, K, Wg);
  a.W2 = Wu;
  a.out_bf16 = out;
  return launch<SK_SWIGLU, X_BF16>(a, F, s);
}

// Tiled bf16 GEMM on MFMA for the layer's projections, C = A * B^T.
//
// A is [M, K] (token rows), B is [N, K] (a weight in the [out, in] storage
// convention of "Qwen2.5-7B 结构拆解" §03.1), both K-contiguous. Token rows
// never interact in a projection (§03.2 of the same page), so M = B*S rows
// form one GEMM.
//
// Design (gfx950, wave64):
// * block = 256 threads = 4 waves; block tile BM x BN x 64; each wave owns a
//   WM x WN sub-tile built from 16x16x32 bf16 MFMAs with fp32 accumulators.
// * global -> registers -> LDS, double-buffered: the loads of k-tile t+1 are
//   in flight while the MFMAs of tile t run; one barrier per k-tile.
// * LDS rows are 64 bf16 (8 chunks of 16 B); chunk c of row r lives at slot
//   c ^ (r & 7), so the 8 lanes served together by a 16-byte LDS read hit 8
//   distinct bank groups.
// * the epilogue goes through LDS: the fp32 tile is written once, then every
//   thread handles 8 consecutive columns of one row, which makes the global
//   stores 16/32-byte contiguous and lets an epilogue combine columns that
//   different waves computed (gate with up for SwiGLU).
//
// A operand: bf16, or fp32 carried as an unevaluated sum hi + lo of two bf16
// values (hi = RNE(a), lo = RNE(a - hi)): two MFMAs against the same weight
// fragment give the product with the fp32 input kept to about 16 significant
// bits instead of 8. Used for the two GEMMs whose inputs are the RMSNorm1
// output and the attention output.
//
// Epilogues (fused, one rounding at the stored tensor):
//   F32_BIAS   out_f32 = acc (+ bias)            Q/K/V projection (+QKV bias)
//   RESID_F32  out_f32 = resid_bf16 + acc        R = X + O W_O^T
//   RESID_OUT  out     = bf16(resid_f32 + acc)   Y = R + H W_down^T
//   SWIGLU     out     = bf16(SiLU(g) * u)       B tile = [W_gate rows | W_up rows]
//   MOE_GU     SWIGLU on gathered token rows with one expert's weights
//              (fp32 A gathered by token, fp32 h)
//   MOE_DOWN   out     = acc for one expert's slot rows (fp32 A and out)
// ("推理系统 03：逐项算清一个真实 Qwen3 Transformer 层" §4, §9, §10; "MoE 初步"
// Expert 的 FFN 结构.)
#include "common.h"
#include "kernels.h"

namespace {

// Expert weights: the 32-row tiles run at decode-sized routings, where each
// expert's weights are read about once per call, so their loads carry the
// non-temporal hint (Qwen3-30B-A3B batch-128 expert gate/up 149 -> 127 us).
QL_DEV u32x4 load_w(const bf16* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

enum : int { GM_F32_BIAS = 0, GM_RESID_F32, GM_RESID_OUT, GM_SWIGLU, GM_MOE_GU, GM_MOE_DOWN };

struct GemmArgs {
  const bf16* A;
  const float* Af;  // fp32 A (split into a bf16 hi + lo pair while staging)
  int lda;
  int M;
  const bf16* B;
  const bf16* B2;
  const bf16* B3;   // F32_BIAS: rows [seg1, seg2) of the output come from B2, [seg2, N) from B3
  int seg1, seg2;
  int ldb;
  int K;
  size_t b_expert_stride;
  float* out_f32;
  bf16* out_bf16;
  int ldo;
  const bf16* bias;
  const bf16* bias2;
  const bf16* bias3;
  const bf16* resid_bf16;
  const float* resid_f32;
  int ldr;
  const int* row_index;
  const int* tile_expert;
  const int* tile_row0;
  const int* tile_rows;
  const int* num_tiles;
  int tiles_n;
};

constexpr int kBK = 64;

template <int BM, int BN, int WM, int WN, int MODE, bool AF32>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmArgs p) {
  constexpr int WAVES_N = BN / WN;
  static_assert((BM / WM) * WAVES_N == 4, "four waves per block");
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int A_CH = BM * 8 / 256, B_CH = BN * 8 / 256;
  static_assert(A_CH >= 1 && B_CH >= 1, "tile too small for 256 threads");
  constexpr int AT = AF32 ? 2 : 1;        // A tiles per stage: hi (+ lo)
  constexpr int STAGE = (AT * BM + BN) * kBK;  // bf16 elements per pipeline stage
  constexpr int PITCH = BN + 4;           // fp32 epilogue tile pitch
  constexpr int LDS_BYTES =
      (2 * STAGE * 2) > (BM * PITCH * 4) ? (2 * STAGE * 2) : (BM * PITCH * 4);
  constexpr bool kDual = (MODE == GM_SWIGLU || MODE == GM_MOE_GU);
  constexpr bool kGrouped = (MODE == GM_MOE_GU || MODE == GM_MOE_DOWN);
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  bf16* lds = reinterpret_cast<bf16*>(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  const int tm = blockIdx.x / p.tiles_n;
  const int tn = blockIdx.x % p.tiles_n;

  int m0, rows_valid;
  size_t expert_off = 0;
  if constexpr (kGrouped) {
    if (tm >= *p.num_tiles) return;
    m0 = p.tile_row0[tm];
    rows_valid = p.tile_rows[tm];
    expert_off = (size_t)p.tile_expert[tm] * p.b_expert_stride;
  } else {
    m0 = tm * BM;
    rows_valid = min(BM, p.M - m0);
  }
  const int n0 = tn * (kDual ? BN / 2 : BN);  // first output column of the tile
  // QKV: each 128-column tile lies inside one of the three weight matrices
  const bf16* Bw = p.B;
  const bf16* bias = p.bias;
  int nb = n0;
  if constexpr (MODE == GM_F32_BIAS) {
    if (n0 >= p.seg2) {
      Bw = p.B3;
      bias = p.bias3;
      nb = n0 - p.seg2;
    } else if (n0 >= p.seg1) {
      Bw = p.B2;
      bias = p.bias2;
      nb = n0 - p.seg1;
    }
  }

  // Per-thread global sources and LDS destinations of the tile loads.
  size_t a_off[A_CH];  // element offset of the thread's 8-wide A piece
  int a_dst[A_CH];
#pragma unroll
  for (int c = 0; c < A_CH; ++c) {
    const int ch = tid + c * 256;
    const int r = ch >> 3, kc = ch & 7;
    const int rr = min(r, rows_valid - 1);  // rows past the end re-read a valid row
    size_t row;
    if constexpr (MODE == GM_MOE_GU) row = (size_t)p.row_index[m0 + rr];
    else row = (size_t)(m0 + rr);
    a_off[c] = row * p.lda + kc * 8;
    a_dst[c] = r * kBK + ((kc ^ (r & 7)) * 8);
  }
  const bf16* b_src[B_CH];
  int b_dst[B_CH];
#pragma unroll
  for (int c = 0; c < B_CH; ++c) {
    const int ch = tid + c * 256;
    const int r = ch >> 3, kc = ch & 7;
    const bf16* base;
    if constexpr (kDual) {
      base = (r < BN / 2) ? p.B + expert_off + (size_t)(n0 + r) * p.ldb
                          : p.B2 + expert_off + (size_t)(n0 + r - BN / 2) * p.ldb;
    } else {
      base = Bw + expert_off + (size_t)(nb + r) * p.ldb;
    }
    b_src[c] = base + kc * 8;
    b_dst[c] = AT * BM * kBK + r * kBK + ((kc ^ (r & 7)) * 8);
  }

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[A_CH][AT], rb[B_CH];
  const int nk = p.K / kBK;

  // A piece -> registers (bf16, or fp32 split into bf16 hi/lo)
  auto aload = [&](int ko) {
#pragma unroll
    for (int c = 0; c < A_CH; ++c) {
      if constexpr (AF32) {
        const float* src = p.Af + a_off[c] + ko;
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(src);
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(src + 4);
        bf16x8 hi, lo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          hi[i] = (bf16)v0[i];
          hi[i + 4] = (bf16)v1[i];
          lo[i] = (bf16)(v0[i] - (float)hi[i]);
          lo[i + 4] = (bf16)(v1[i] - (float)hi[i + 4]);
        }
        ra[c][0] = *reinterpret_cast<const u32x4*>(&hi);
        ra[c][AT - 1] = *reinterpret_cast<const u32x4*>(&lo);
      } else {
        ra[c][0] = *reinterpret_cast<const u32x4*>(p.A + a_off[c] + ko);
      }
    }
  };
  auto astore = [&](bf16* base) {
#pragma unroll
    for (int c = 0; c < A_CH; ++c)
#pragma unroll
      for (int t = 0; t < AT; ++t)
        *reinterpret_cast<u32x4*>(base + t * BM * kBK + a_dst[c]) = ra[c][t];
  };

  aload(0);
#pragma unroll
  for (int c = 0; c < B_CH; ++c) rb[c] = load_w(b_src[c]);
  astore(lds);
#pragma unroll
  for (int c = 0; c < B_CH; ++c) *reinterpret_cast<u32x4*>(lds + b_dst[c]) = rb[c];
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    const bool more = (kt + 1) < nk;
    if (more) {
      const int ko = (kt + 1) * kBK;
      aload(ko);
#pragma unroll
      for (int c = 0; c < B_CH; ++c) rb[c] = load_w(b_src[c] + ko);
    }
    const bf16* As = lds + st * STAGE;
    const bf16* Bs = As + AT * BM * kBK;
#pragma unroll
    for (int ks = 0; ks < kBK / 32; ++ks) {
      const int kc = ks * 4 + (lane >> 4);
      bf16x8 af[AT][TM], bfr[TN];
#pragma unroll
      for (int t = 0; t < AT; ++t)
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int r = wm * WM + i * 16 + (lane & 15);
          af[t][i] = *reinterpret_cast<const bf16x8*>(As + t * BM * kBK + r * kBK +
                                                      ((kc ^ (r & 7)) * 8));
        }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * WN + j * 16 + (lane & 15);
        bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + r * kBK + ((kc ^ (r & 7)) * 8));
      }
#pragma unroll
      for (int t = 0; t < AT; ++t)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = mfma_16x16x32(af[t][i], bfr[j], acc[i][j]);
    }
    if (more) {
      bf16* Ad = lds + (st ^ 1) * STAGE;
      astore(Ad);
#pragma unroll
      for (int c = 0; c < B_CH; ++c) *reinterpret_cast<u32x4*>(Ad + b_dst[c]) = rb[c];
    }
    __syncthreads();
  }

  // fp32 tile -> LDS
  float* C = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        C[(wm * WM + i * 16 + 4 * (lane >> 4) + r) * PITCH + wn * WN + j * 16 + (lane & 15)] =
            acc[i][j][r];
  __syncthreads();

  if constexpr (kDual) {
    constexpr int SEGS = BN / 2 / 8;   // 8-column segments of the output per row
    constexpr int RPP = 256 / SEGS;    // rows per pass
    const int seg = tid % SEGS;
    for (int r = tid / SEGS; r < rows_valid; r += RPP) {
      const float* g = C + r * PITCH + seg * 8;
      const float* u = g + BN / 2;
      float h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = silu_f32(g[i]) * u[i];
      if (p.out_f32) {
        float* o = p.out_f32 + (size_t)(m0 + r) * p.ldo + n0 + seg * 8;
        *reinterpret_cast<f32x4*>(o) = f32x4{h[0], h[1], h[2], h[3]};
        *reinterpret_cast<f32x4*>(o + 4) = f32x4{h[4], h[5], h[6], h[7]};
      } else {
        store_bf16x8(p.out_bf16 + (size_t)(m0 + r) * p.ldo + n0 + seg * 8, pack8(h));
      }
    }
  } else {
    constexpr int SEGS = BN / 8;
    constexpr int RPP = 256 / SEGS;
    const int seg = tid % SEGS;
    const int col = n0 + seg * 8;
    float badd[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) badd[i] = 0.f;
    if constexpr (MODE == GM_F32_BIAS) {
      if (bias) unpack8(load_bf16x8(bias + nb + seg * 8), badd);
    }
    for (int r = tid / SEGS; r < rows_valid; r += RPP) {
      const float* c = C + r * PITCH + seg * 8;
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = c[i] + badd[i];
      const size_t row = (size_t)(m0 + r);
      if constexpr (MODE == GM_RESID_F32) {
        float x[8];
        unpack8(load_bf16x8(p.resid_bf16 + row * p.ldr + col), x);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] += x[i];
      }
      if constexpr (MODE == GM_RESID_OUT) {
        const float* rr = p.resid_f32 + row * p.ldr + col;
        const f32x4 r0 = *reinterpret_cast<const f32x4*>(rr);
        const f32x4 r1 = *reinterpret_cast<const f32x4*>(rr + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] += r0[i];
          v[i + 4] += r1[i];
        }
        store_bf16x8(p.out_bf16 + row * p.ldo + col, pack8(v));
      } else if constexpr (MODE == GM_MOE_DOWN) {
        if (p.out_f32) {
          float* o = p.out_f32 + row * p.ldo + col;
          *reinterpret_cast<f32x4*>(o) = f32x4{v[0], v[1], v[2], v[3]};
          *reinterpret_cast<f32x4*>(o + 4) = f32x4{v[4], v[5], v[6], v[7]};
        } else {
          store_bf16x8(p.out_bf16 + row * p.ldo + col, pack8(v));
        }
      } else {
        float* o = p.out_f32 + row * p.ldo + col;
        *reinterpret_cast<f32x4*>(o) = f32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4*>(o + 4) = f32x4{v[4], v[5], v[6], v[7]};
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int MODE, bool AF32 = false>
hipError_t launch(const GemmArgs& a, int tiles_m, hipStream_t s) {
  const int blocks = tiles_m * a.tiles_n;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, MODE, AF32>), dim3(blocks), dim3(256), 0, s,
                     a);
  return hipGetLastError();
}

GemmArgs base_args(const bf16* A, int lda, int M, const bf16* B, int ldb, int K) {
  GemmArgs a{};
  a.A = A;
  a.seg1 = a.seg2 = 0x7fffffff;
  a.lda = lda;
  a.M = M;
  a.B = B;
  a.ldb = ldb;
  a.K = K;
  return a;
}

}  // namespace

hipError_t ql_gemm_moe_gu(const float* Zf, const int* slot_token, const bf16* Wg, const bf16* Wu,
                          int mf, int d, const int* tile_expert, const int* tile_row0,
                          const int* tile_rows, const int* num_tiles, int max_tiles, float* H,
                          hipStream_t s) {
  GemmArgs a = base_args(nullptr, d, 0, Wg, d, d);
  a.Af = Zf;
  a.B2 = Wu;
  a.b_expert_stride = (size_t)mf * d;
  a.row_index = slot_token;
  a.tile_expert = tile_expert;
  a.tile_row0 = tile_row0;
  a.tile_rows = tile_rows;
  a.num_tiles = num_tiles;
  a.out_f32 = H;
  a.ldo = mf;
  a.tiles_n = mf / 64;
  return launch<32, 128, 32, 32, GM_MOE_GU, true>(a, max_tiles, s);
}

hipError_t ql_gemm_moe_down(const float* H, const bf16* Wd, int mf, int d, const int* tile_expert,
                            const int* tile_row0, const int* tile_rows, const int* num_tiles,
                            int max_tiles, float* out, hipStream_t s) {
  GemmArgs a = base_args(nullptr, mf, 0, Wd, mf, mf);
  a.Af = H;
  a.b_expert_stride = (size_t)d * mf;
  a.tile_expert = tile_expert;
  a.tile_row0 = tile_row0;
  a.tile_rows = tile_rows;
  a.num_tiles = num_tiles;
  a.out_f32 = out;
  a.ldo = d;
  a.tiles_n = d / 128;
  return launch<32, 128, 32, 32, GM_MOE_DOWN, true>(a, max_tiles, s);
}

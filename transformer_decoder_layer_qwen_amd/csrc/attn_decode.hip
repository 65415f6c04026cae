// Decode attention: one new query per sequence over its cached rows
// 0..cache_len[b] (the new row was appended just before), head_dim 128.
//
// ("Qwen2.5-7B 结构拆解" §09.1: q attends to all t+1 cache rows; §05.5: no
// causal halving for the single query; §05.2: the Hq/Hkv query heads of a
// group read the same K/V bytes, so the group pays for them once.)
//
// Split-K: grid (splits, Hkv, B). A block reads one key range of one KV head
// once and serves all G = Hq/Hkv query heads of the group:
//   * scores: S^T[key][head] = K Q^T with 16x16x32 MFMAs, K rows loaded
//     straight from the cache with 16-byte loads (A operand), the G queries
//     padded to 16 columns (B operand, held in registers);
//   * online softmax per head (column): max over 16 keys = 4 registers and
//     two lane exchanges;
//   * P V on the vector ALUs: lane (dh piece of 8, key sub-group) loads its
//     V rows with 16-byte loads and accumulates G x 8 fp32 outputs; P and the
//     per-head rescale factors go through a per-wave LDS scratch.
// Each block writes an unnormalised partial (m, l, o[128]) per head; the
// combine kernel merges the splits (with a single split the block writes the
// normalised output itself).
//
// Prologue (fused QK-norm / RoPE / cache append): the Q/K/V projection hands
// over raw sums of (x * gamma1) W^T. Each block computes RMSNorm1's 1/rms for
// its row, forms q for its G heads (scale, bias, QK-norm, rotate_half RoPE at
// position cache_len + pos_offset) and keeps them in LDS; the block whose key
// range contains the new row also forms that row's k and v, appends them to
// the cache and uses them from LDS ("Qwen2.5-7B 结构拆解" §09.1; "推理系统 03：
// 逐项算清一个真实 Qwen3 Transformer 层" §5, §6, §12).
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kDh = 128;

template <int G>
__global__ __launch_bounds__(256) void attn_decode_kernel(const AttnDecodeArgs p) {
  __shared__ float p_lds[4][16 * 16];  // per wave: P[key 16][head 16]
  __shared__ float a_lds[4][16];       // per wave: rescale per head
  __shared__ float w_o[4][G * kDh];    // cross-wave partial outputs
  __shared__ float w_m[4][16];
  __shared__ float w_l[4][16];
  __shared__ __attribute__((aligned(16))) bf16 q_lds[16][kDh];    // rows >= G stay zero
  __shared__ __attribute__((aligned(16))) bf16 kv_new[2][kDh];    // appended K and V row
  __shared__ float red4[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;

  const int L = p.cache_len[b];
  const bool valid = L >= 0 && L < p.T_max;
  const int nkeys = valid ? L + 1 : 0;
  const int kbeg = split * p.chunk;
  const int kend = min(kbeg + p.chunk, nkeys);

  // ---- prologue: RMSNorm1 scale, q heads, the appended K/V row ----
  {
    const bf16* xr = p.x + (size_t)b * p.d;
    float ss = 0.f;
    for (int c = tid * 8; c < p.d; c += 256 * 8) {
      float f[8];
      unpack8(load_bf16x8(xr + c), f);
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += f[j] * f[j];
    }
    ss = wave_sum(ss);
    if (lane == 0) red4[wave] = ss;
  }
  __syncthreads();
  const float inv = 1.0f / sqrtf((red4[0] + red4[1] + red4[2] + red4[3]) / (float)p.d + p.eps);
  float sn, cs;
  {
    const double pos = (double)L + (double)p.pos_offset;
    const double omega = exp2(-2.0 * (double)lane / (double)kDh * log2((double)p.theta));
    double ang = pos * omega;
    const double two_pi = 6.283185307179586476925286766559;
    ang -= two_pi * rint(ang / two_pi);
    sincosf((float)ang, &sn, &cs);
  }
  const int qd = p.n_q_heads * kDh;
  const int kvd = p.n_kv_heads * kDh;
  const float* raw = p.qkv_raw + (size_t)b * p.ld_raw;
  // one head's 128 values: lane owns (lane, lane + 64); scale, bias, norm, rotate
  auto head_vec = [&](int col0, const bf16* bias, const bf16* gam, bool rotate, float& o0,
                      float& o1) {
    float x0 = inv * raw[col0 + lane];
    float x1 = inv * raw[col0 + lane + 64];
    if (bias) {
      x0 += to_f32(bias[lane]);
      x1 += to_f32(bias[lane + 64]);
    }
    if (gam) {
      const float hs = wave_sum(x0 * x0 + x1 * x1);
      const float hinv = 1.0f / sqrtf(hs / (float)kDh + p.eps);
      x0 = to_f32(gam[lane]) * (x0 * hinv);
      x1 = to_f32(gam[lane + 64]) * (x1 * hinv);
    }
    if (rotate) {
      o0 = x0 * cs - x1 * sn;
      o1 = x0 * sn + x1 * cs;
    } else {
      o0 = x0;
      o1 = x1;
    }
  };
  for (int hh = wave; hh < 16; hh += 4) {
    float r0 = 0.f, r1 = 0.f;
    if (hh < G) {
      const int hq = g * G + hh;
      head_vec(hq * kDh, p.bq ? p.bq + hq * kDh : nullptr, p.q_norm_g, true, r0, r1);
      if (split == 0 && p.q_out) {
        const float nv = valid ? 0.f : __builtin_nanf("");
        p.q_out[(size_t)b * qd + hq * kDh + lane] = (bf16)(r0 + nv);
        p.q_out[(size_t)b * qd + hq * kDh + lane + 64] = (bf16)(r1 + nv);
      }
    }
    q_lds[hh][lane] = (bf16)r0;
    q_lds[hh][lane + 64] = (bf16)r1;
  }
  const bool has_new = valid && kbeg <= L && L < kend;
  if (has_new && wave == 0) {
    float k0, k1, v0, v1;
    head_vec(qd + g * kDh, p.bk ? p.bk + g * kDh : nullptr, p.k_norm_g, true, k0, k1);
    head_vec(qd + kvd + g * kDh, p.bv ? p.bv + g * kDh : nullptr, nullptr, false, v0, v1);
    const size_t crow = ((size_t)b * p.T_max + L) * kvd + g * kDh;
    const bf16 bk0 = (bf16)k0, bk1 = (bf16)k1, bv0 = (bf16)v0, bv1 = (bf16)v1;
    p.k_cache_w[crow + lane] = bk0;
    p.k_cache_w[crow + lane + 64] = bk1;
    p.v_cache_w[crow + lane] = bv0;
    p.v_cache_w[crow + lane + 64] = bv1;
    kv_new[0][lane] = bk0;
    kv_new[0][lane + 64] = bk1;
    kv_new[1][lane] = bv0;
    kv_new[1][lane + 64] = bv1;
  }
  __syncthreads();

  // Q^T fragments: lane (head col, group grp) holds dh [32s + 8grp, +8)
  bf16x8 qf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(&q_lds[col][32 * s + 8 * grp]);
  const size_t row_stride = (size_t)p.n_kv_heads * kDh;
  const bf16* kb_ = p.k_cache + (size_t)b * p.T_max * row_stride + g * kDh;
  const bf16* vb_ = p.v_cache + (size_t)b * p.T_max * row_stride + g * kDh;

  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  float m_run = -INFINITY;  // for head `col`
  float l_run = 0.f;

  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  for (int k0 = kbeg + 16 * wave; k0 < kend; k0 += 64) {
    // scores for keys k0 .. k0+15
    const int krow = k0 + col;
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
    {
      const bool kv = krow < kend;
      const bool knew = has_new && krow == L;
      const bf16* kr = knew ? kv_new[0] : kb_ + (size_t)(kv ? krow : kbeg) * row_stride;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 kraw = kv ? *reinterpret_cast<const u32x4*>(kr + 32 * s + 8 * grp) : zero4;
        sc = mfma_16x16x32(*reinterpret_cast<const bf16x8*>(&kraw), qf[s], sc);
      }
    }
    // V rows this lane accumulates: keys k0 + 4*grp + j, dh piece col
    u32x4 vraw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = k0 + 4 * grp + j;
      const bf16* vr = (has_new && key == L) ? kv_new[1] : vb_ + (size_t)key * row_stride;
      vraw[j] = key < kend ? *reinterpret_cast<const u32x4*>(vr + col * 8) : zero4;
    }
    // lane holds S^T[key 4*grp + r][head col]
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = sc[r] * p.scale_log2;
      if (k0 + 4 * grp + r >= kend) x = -INFINITY;
      sc[r] = x;
      mt = fmaxf(mt, x);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16, kWave));
    mt = fmaxf(mt, __shfl_xor(mt, 32, kWave));
    const float m_new = fmaxf(m_run, mt);  // finite: key k0 < kend is valid
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pv = exp2f(sc[r] - m_new);
      ps += pv;
      p_lds[wave][(4 * grp + r) * 16 + col] = pv;
    }
    ps += __shfl_xor(ps, 16, kWave);
    ps += __shfl_xor(ps, 32, kWave);
    l_run = l_run * alpha + ps;
    if (grp == 0) a_lds[wave][col] = alpha;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float al = a_lds[wave][h];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= al;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v[8];
      unpack8(*reinterpret_cast<const bf16x8*>(&vraw[j]), v);
      const float* pr = &p_lds[wave][(4 * grp + j) * 16];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pw = pr[h];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] += pw * v[e];
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  }

  // reduce the 4 key sub-groups of the wave (lanes col, col+16, col+32, col+48)
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = acc[h][e];
        v += __shfl_xor(v, 16, kWave);
        v += __shfl_xor(v, 32, kWave);
        acc[h][e] = v;
      }
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) w_o[wave][h * kDh + col * 8 + e] = acc[h][e];
    w_m[wave][col] = m_run;
    w_l[wave][col] = l_run;
  }
  __syncthreads();

  // merge the 4 waves; write this split's partial for each head of the group
  for (int i = tid; i < G * kDh; i += 256) {
    const int h = i / kDh;
    const int d = i % kDh;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, w_m[w][h]);
    float o = 0.f, l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if (w_m[w][h] == -INFINITY) continue;
        const float f = exp2f(w_m[w][h] - M);
        o += w_o[w][h * kDh + d] * f;
        l += w_l[w][h] * f;
      }
    }
    if (p.nsplit == 1) {  // the only split: normalise here
      p.out[(size_t)b * p.ldo + (size_t)(g * G + h) * kDh + d] =
          valid ? o / l : __builtin_nanf("");
      continue;
    }
    const size_t slot = ((size_t)b * p.n_q_heads + g * G + h) * p.nsplit + split;
    p.part_o[slot * kDh + d] = o;
    if (d == 0) {
      p.part_ml[slot * 2 + 0] = M;
      p.part_ml[slot * 2 + 1] = l;
    }
  }
}

__global__ __launch_bounds__(128) void attn_decode_combine_kernel(const AttnDecodeArgs p) {
  const int bh = blockIdx.x;  // b * Hq + head
  const int b = bh / p.n_q_heads;
  const int d = threadIdx.x;
  const int L = p.cache_len[b];
  const bool valid = L >= 0 && L < p.T_max;
  const size_t base = (size_t)bh * p.nsplit;
  float M = -INFINITY;
  for (int s = 0; s < p.nsplit; ++s) M = fmaxf(M, p.part_ml[(base + s) * 2]);
  float o = 0.f, l = 0.f;
  for (int s = 0; s < p.nsplit; ++s) {
    const float m = p.part_ml[(base + s) * 2];
    if (m == -INFINITY) continue;
    const float f = exp2f(m - M);
    o += p.part_o[(base + s) * kDh + d] * f;
    l += p.part_ml[(base + s) * 2 + 1] * f;
  }
  const float out = valid ? o / l : __builtin_nanf("");
  p.out[(size_t)b * p.ldo + (size_t)(bh % p.n_q_heads) * kDh + d] = out;
}

}  // namespace

hipError_t ql_attn_decode_bf16(const AttnDecodeArgs& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  const dim3 grid(a.nsplit, a.n_kv_heads, a.B);
  switch (a.n_q_heads / a.n_kv_heads) {
#define QL_G(V)                                                                     \
  case V:                                                                           \
    hipLaunchKernelGGL(attn_decode_kernel<V>, grid, dim3(256), 0, s, a);           \
    break;
    QL_G(1) QL_G(2) QL_G(3) QL_G(4) QL_G(5) QL_G(6) QL_G(7) QL_G(8)
    QL_G(9) QL_G(10) QL_G(11) QL_G(12) QL_G(13) QL_G(14) QL_G(15) QL_G(16)
#undef QL_G
    default:
      return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  hipLaunchKernelGGL(attn_decode_combine_kernel, dim3(a.B * a.n_q_heads), dim3(128), 0, s, a);
  return hipGetLastError();
}

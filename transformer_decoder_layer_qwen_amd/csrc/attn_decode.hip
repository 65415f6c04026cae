// Decode attention: one new query per sequence over its cached rows
// 0..cache_len[b] (the new row was appended just before), head_dim 128.
//
// ("Qwen2.5-7B 结构拆解" §09.1: q attends to all t+1 cache rows; §05.5: no
// causal halving for the single query; §05.2: the Hq/Hkv query heads of a
// group read the same K/V bytes, so the group pays for them once.)
//
// Split-K: grid (splits, Hkv, B), 4 or 8 waves per block. A block reads
// one key range of one KV head once and serves all G = Hq/Hkv query heads of
// the group; its waves take 16-key tiles round-robin, each keeping the next
// tile's loads in flight while it works on the current one:
//   * scores: S^T[key][head] = K Q^T with 16x16x32 MFMAs, K rows loaded
//     straight from the cache with 16-byte loads (A operand), the G queries
//     padded to 16 columns (B operand, held in registers);
//   * online softmax per head (column): max over 16 keys = 4 registers and
//     two lane exchanges;
//   * P V on the vector ALUs: lane (dh piece of 8, key sub-group) loads its
//     V rows with 16-byte loads and accumulates G x 8 fp32 outputs; P and the
//     per-head rescale factors go through a per-wave LDS scratch.
// The waves merge in LDS. With one split the block writes the normalised
// output; otherwise it writes an unnormalised partial (m, l, o[128]) per head
// and a small combine kernel merges the splits (a cross-block merge inside
// the kernel would need device-scope fences, which write back and invalidate
// the whole L2 of the XCD on this GPU and cost far more than a launch).
//
// Prologue (fused QK-norm / RoPE / cache append): the Q/K/V projection hands
// over raw sums of (x * gamma1) W^T, and 1/rms of x (or the block computes it
// from x). Each block forms q for its G heads (scale, bias, QK-norm,
// rotate_half RoPE at position cache_len + pos_offset) and keeps them in LDS;
// the block whose key range contains the new row also forms that row's k and
// v, appends them to the cache and uses them from LDS ("Qwen2.5-7B 结构拆解"
// §09.1; "推理系统 03：逐项算清一个真实 Qwen3 Transformer 层" §5, §6, §12).
// The cache, K/V tile, projection and bias loads are all issued before the
// prologue's arithmetic.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kDh = 128;

// NW waves per block (4 or 8); wave w takes keys kbeg + 16 w + 16 NW i.
template <int G, int NW>
__global__ __launch_bounds__(NW * 64) void attn_decode_kernel(const AttnDecodeArgs p) {
  constexpr int kQS = 16 / NW;            // query-head slots per wave in the prologue
  __shared__ float p_lds[NW][16 * 16];    // per wave: P[key 16][head 16]
  __shared__ float a_lds[NW][16];         // per wave: rescale per head
  __shared__ float w_o[NW][G * kDh];      // cross-wave partial outputs
  __shared__ float w_m[NW][16];
  __shared__ float w_l[NW][16];
  __shared__ __attribute__((aligned(16))) bf16 q_lds[16][kDh];    // rows >= G stay zero
  __shared__ __attribute__((aligned(16))) bf16 kv_new[2][kDh];    // appended K and V row
  __shared__ float red[NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;

  // ---- every load goes out before any of them is waited on ----
  // Nothing here depends on cache_len[b]: the first tile is loaded up to the
  // split's end within T_max and masked once the length is known, the
  // projection / bias / norm loads are unconditional (absent biases and norms
  // read a harmless valid address and are masked to 0 / 1).
  const int L = p.cache_len[b];
  const int kbeg = split * p.chunk;
  const int kcap = min(kbeg + p.chunk, p.T_max);
  const size_t row_stride = (size_t)p.n_kv_heads * kDh;
  const bf16* kb_ = p.k_cache + (size_t)b * p.T_max * row_stride + g * kDh;
  const bf16* vb_ = p.v_cache + (size_t)b * p.T_max * row_stride + g * kDh;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  // A wave's tile: keys k0 .. k0+15. K: lane (key col, k-group grp) loads dh
  // [32 s + 8 grp, +8) of key k0 + col; V: keys k0 + 4 grp + j, dh piece col.
  auto load_tile = [&](int k0, int lim, u32x4 (&kt)[4], u32x4 (&vt)[4]) {
    const int krow = k0 + col;
    const bool kv = krow < lim;
    const bf16* kr = kb_ + (size_t)(kv ? krow : kbeg) * row_stride;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      kt[s] = kv ? *reinterpret_cast<const u32x4*>(kr + 32 * s + 8 * grp) : zero4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = k0 + 4 * grp + j;
      vt[j] = key < lim ? *reinterpret_cast<const u32x4*>(vb_ + (size_t)key * row_stride + col * 8)
                        : zero4;
    }
  };
  u32x4 kcur[4], vcur[4];
  load_tile(kbeg + 16 * wave, kcap, kcur, vcur);

  const int qd = p.n_q_heads * kDh;
  const int kvd = p.n_kv_heads * kDh;
  const float* raw = p.qkv_raw + (size_t)b * p.ld_raw;
  // slots 0 .. kQS-1: query heads wave + NW i of the group; kQS, kQS+1: the new K and V row
  constexpr int kSlots = kQS + 2;
  float hv[kSlots][2], hb[kSlots][2];
#pragma unroll
  for (int i = 0; i < kSlots; ++i) {
    const int hq = g * G + wave + NW * i;
    const int c0 = i < kQS ? (wave + NW * i < G ? hq * kDh : 0)
                           : (i == kQS ? qd + g * kDh : qd + kvd + g * kDh);
    hv[i][0] = raw[c0 + lane];
    hv[i][1] = raw[c0 + lane + 64];
    const bf16* bias = i < kQS ? p.bq : (i == kQS ? p.bk : p.bv);
    const int bc = i < kQS ? c0 : g * kDh;
    const bf16* bsrc = bias ? bias + bc : p.x;
    const float b0 = to_f32(bsrc[lane]), b1 = to_f32(bsrc[lane + 64]);
    hb[i][0] = bias ? b0 : 0.f;
    hb[i][1] = bias ? b1 : 0.f;
  }
  const float inv_given = p.inv_rms ? p.inv_rms[b] : 0.f;
  const bool qkn = p.q_norm_g != nullptr;
  const bf16* qgs = qkn ? p.q_norm_g : p.x;
  const bf16* kgs = qkn ? p.k_norm_g : p.x;
  const float qg0r = to_f32(qgs[lane]), qg1r = to_f32(qgs[lane + 64]);
  const float kg0r = to_f32(kgs[lane]), kg1r = to_f32(kgs[lane + 64]);
  const float qg0 = qkn ? qg0r : 1.f, qg1 = qkn ? qg1r : 1.f;
  const float kg0 = qkn ? kg0r : 1.f, kg1 = qkn ? kg1r : 1.f;

  const bool valid = L >= 0 && L < p.T_max;
  const int nkeys = valid ? L + 1 : 0;
  const int kend = min(kbeg + p.chunk, nkeys);
  const bool has_new = valid && kbeg <= L && L < kend;
  // rows of the first tile past the live keys may hold anything (a NaN would
  // survive a zero softmax weight in P V): zero their V
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (kbeg + 16 * wave + 4 * grp + j >= kend) vcur[j] = zero4;

  // ---- prologue: RMSNorm1 scale, q heads, the appended K/V row ----
  float inv = inv_given;
  if (!p.inv_rms) {
    const bf16* xr = p.x + (size_t)b * p.d;
    float ss = 0.f;
    for (int c = tid * 8; c < p.d; c += NW * 64 * 8) {
      float f[8];
      unpack8(load_bf16x8(xr + c), f);
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += f[j] * f[j];
    }
    ss = wave_sum(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += red[w];
    inv = 1.0f / sqrtf(t / (float)p.d + p.eps);
  }
  float sn, cs;
  {
    const double pos = (double)L + (double)p.pos_offset;
    const double omega = exp2(-2.0 * (double)lane / (double)kDh * log2((double)p.theta));
    double ang = pos * omega;
    const double two_pi = 6.283185307179586476925286766559;
    ang -= two_pi * rint(ang / two_pi);
    sincosf((float)ang, &sn, &cs);
  }
  // one head's 128 values: lane owns (lane, lane + 64); scale, bias, norm, rotate
  auto head_vec = [&](int i, bool norm, float g0, float g1, bool rotate, float& o0, float& o1) {
    float x0 = inv * hv[i][0] + hb[i][0];
    float x1 = inv * hv[i][1] + hb[i][1];
    if (norm) {
      const float hs = wave_sum(x0 * x0 + x1 * x1);
      const float hinv = 1.0f / sqrtf(hs / (float)kDh + p.eps);
      x0 = g0 * (x0 * hinv);
      x1 = g1 * (x1 * hinv);
    }
    if (rotate) {
      o0 = x0 * cs - x1 * sn;
      o1 = x0 * sn + x1 * cs;
    } else {
      o0 = x0;
      o1 = x1;
    }
  };
#pragma unroll
  for (int i = 0; i < kQS; ++i) {
    const int hh = wave + NW * i;
    float r0 = 0.f, r1 = 0.f;
    if (hh < G) {
      head_vec(i, qkn, qg0, qg1, true, r0, r1);
      if (split == 0 && p.q_out) {
        const int hq = g * G + hh;
        const float nv = valid ? 0.f : __builtin_nanf("");
        p.q_out[(size_t)b * qd + hq * kDh + lane] = (bf16)(r0 + nv);
        p.q_out[(size_t)b * qd + hq * kDh + lane + 64] = (bf16)(r1 + nv);
      }
    }
    q_lds[hh][lane] = (bf16)r0;
    q_lds[hh][lane + 64] = (bf16)r1;
  }
  if (has_new && wave == 0) {
    float k0, k1, v0, v1;
    head_vec(kQS, qkn, kg0, kg1, true, k0, k1);
    head_vec(kQS + 1, false, 1.f, 1.f, false, v0, v1);
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

  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  float m_run = -INFINITY;  // for head `col`
  float l_run = 0.f;

  for (int k0 = kbeg + 16 * wave; k0 < kend; k0 += 16 * NW) {
    // the next tile's loads overlap this tile's arithmetic
    u32x4 knext[4], vnext[4];
    load_tile(k0 + 16 * NW, kend, knext, vnext);
    // the appended row comes from LDS (its cache write may still be in flight)
    if (has_new) {
      if (k0 + col == L) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          kcur[s] = *reinterpret_cast<const u32x4*>(&kv_new[0][32 * s + 8 * grp]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (k0 + 4 * grp + j == L) vcur[j] = *reinterpret_cast<const u32x4*>(&kv_new[1][col * 8]);
    }
    // scores for keys k0 .. k0+15
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) sc = mfma_16x16x32(*reinterpret_cast<const bf16x8*>(&kcur[s]), qf[s], sc);
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
      unpack8(*reinterpret_cast<const bf16x8*>(&vcur[j]), v);
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
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      kcur[s] = knext[s];
      vcur[s] = vnext[s];
    }
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
  // merge the waves; write this split's partial for each head of the group
  for (int i = tid; i < G * kDh; i += NW * 64) {
    const int h = i / kDh;
    const int d = i % kDh;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, w_m[w][h]);
    float o = 0.f, l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
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

// Merge the splits of one (sequence, head): every partial is loaded at once
// (the loads are independent), the maxima and sums go through LDS.
__global__ __launch_bounds__(128) void attn_decode_combine_kernel(const AttnDecodeArgs p) {
  __shared__ float s_m[kMaxDecodeSplits], s_l[kMaxDecodeSplits];
  const int bh = blockIdx.x;  // b * Hq + head
  const int b = bh / p.n_q_heads;
  const int d = threadIdx.x;
  const size_t base = (size_t)bh * p.nsplit;
  float ov[kMaxDecodeSplits];
#pragma unroll
  for (int s = 0; s < kMaxDecodeSplits; ++s)
    ov[s] = s < p.nsplit ? p.part_o[(base + s) * kDh + d] : 0.f;
  if (d < p.nsplit) {
    s_m[d] = p.part_ml[(base + d) * 2];
    s_l[d] = p.part_ml[(base + d) * 2 + 1];
  }
  const int L = p.cache_len[b];
  const bool valid = L >= 0 && L < p.T_max;
  __syncthreads();
  float M = -INFINITY;
  for (int s = 0; s < p.nsplit; ++s) M = fmaxf(M, s_m[s]);
  float o = 0.f, l = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxDecodeSplits; ++s) {
    if (s >= p.nsplit) break;
    const float m = s_m[s];
    if (m == -INFINITY) continue;
    const float f = exp2f(m - M);
    o += ov[s] * f;
    l += s_l[s] * f;
  }
  const float out = valid ? o / l : __builtin_nanf("");
  p.out[(size_t)b * p.ldo + (size_t)(bh % p.n_q_heads) * kDh + d] = out;
}

template <int G>
hipError_t launch_g(const AttnDecodeArgs& a, hipStream_t s) {
  const dim3 grid(a.nsplit, a.n_kv_heads, a.B);
  switch (a.waves) {
    case 4: hipLaunchKernelGGL((attn_decode_kernel<G, 4>), grid, dim3(256), 0, s, a); break;
    case 8:
      if constexpr (G <= 8) {
        hipLaunchKernelGGL((attn_decode_kernel<G, 8>), grid, dim3(512), 0, s, a);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t ql_attn_decode_bf16(const AttnDecodeArgs& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  hipError_t e;
  switch (a.n_q_heads / a.n_kv_heads) {
#define QL_G(V) \
  case V: e = launch_g<V>(a, s); break;
    QL_G(1) QL_G(2) QL_G(3) QL_G(4) QL_G(5) QL_G(6) QL_G(7) QL_G(8)
    QL_G(9) QL_G(10) QL_G(11) QL_G(12) QL_G(13) QL_G(14) QL_G(15) QL_G(16)
#undef QL_G
    default:
      return hipErrorInvalidValue;
  }
  if (e != hipSuccess || a.nsplit == 1) return e;
  hipLaunchKernelGGL(attn_decode_combine_kernel, dim3(a.B * a.n_q_heads), dim3(128), 0, s, a);
  return hipGetLastError();
}

// Decode attention: one new query per sequence over its cached rows
// 0..cache_len[b] (the new row was appended just before), head_dim 128.
//
// ("Qwen2.5-7B 结构拆解" §09.1: q attends to all t+1 cache rows; §05.5: no
// causal halving for the single query; §05.2: the Hq/Hkv query heads of a
// group read the same K/V bytes, so the group pays for them once.)
//
// One wave per (key split, KV head, sequence). The wave reads its key range of
// one KV head once and serves all G = Hq/Hkv query heads of the group, 16 keys
// (a tile) at a time, with the next tile's loads in flight during the current
// tile's arithmetic:
//   * scores: S^T[key][head] = K Q^T with 16x16x32 MFMAs, K rows loaded
//     straight from the cache with 16-byte loads (A operand), the G queries
//     padded to 16 columns (B operand, held in registers);
//   * online softmax per head (column): max over 16 keys = 4 registers and
//     two lane exchanges; P goes through LDS;
//   * P V on the vector ALUs: lane (dh piece col of 8 values, head group grp)
//     owns heads grp, grp + 4, ... and sums over all 16 keys of the tile, so
//     no cross-lane reduction is needed at the end.
// With one split the wave writes the normalised output; otherwise it writes an
// unnormalised partial (m, l, o[128]) per head and the combine kernel merges
// the splits. (Merging across blocks would need device-scope fences, which
// write back and invalidate the whole L2 of the XCD on this GPU and cost far
// more than a second launch; the batched kernel below merges splits that
// share a block.) Short caches get one tile per wave, so every K/V byte a
// wave needs is requested when the wave starts.
//
// Prologue (fused QK-norm / RoPE / cache append): the Q/K/V projection hands
// over raw sums of (x * gamma1) W^T, and 1/rms of x (or the wave computes it
// from x). The wave forms q for its G heads (scale, bias, QK-norm,
// rotate_half RoPE at position cache_len + pos_offset) into LDS; the wave
// whose key range contains the new row also forms that row's k and v, appends
// them to the cache and uses them from LDS ("Qwen2.5-7B 结构拆解" §09.1;
// "推理系统 03：逐项算清一个真实 Qwen3 Transformer 层" §5, §6, §12). All cache,
// projection, bias and norm loads are issued before any is waited on.
// Larger batches, where the projection runs on MFMA tiles and already
// finished q and appended the new row, use attn_decode_mfma_kernel below.
//
// Output: fp32, or (out_hilo) the bf16 pair hi = RNE(o), lo = RNE(o - hi)
// that the O projection takes as its A operand.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace {

// Whole-wave sum / max through LDS permutes. In this file's latency-bound
// prologue and split combine they measure faster than the DPP-and-swap chain
// of wave_sum / wave_max (Qwen2.5-7B batch-1 attention stage 11.0 -> 9.3 us,
// batch 32 25.2 -> 23.1 us).
QL_DEV float wave_sum_perm(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
QL_DEV float wave_max_perm(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

constexpr int kDh = 128;

// 8 output values of one head -> fp32 or the bf16 hi/lo pair
QL_DEV void store_out8(const AttnDecodeArgs& p, size_t idx, const float (&v)[8]) {
  if (p.out_hilo) {
    float lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) lo[e] = v[e] - (float)(bf16)v[e];
    store_bf16x8(p.out_hilo + idx, pack8(v));
    store_bf16x8(p.out_hilo + idx + p.lo_off, pack8(lo));
  } else {
    *reinterpret_cast<f32x4*>(p.out + idx) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p.out + idx + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
}

template <int G>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3))) void attn_decode_kernel(const AttnDecodeArgs p) {
  constexpr int HPL = (G + 3) / 4;  // heads per lane in P V
  __shared__ float p_lds[16 * 16];  // P[key 16][head 16]
  __shared__ float a_lds[16];       // per-head rescale, then per-head l
  __shared__ __attribute__((aligned(16))) bf16 q_lds[16][kDh];  // rows >= G stay zero
  __shared__ __attribute__((aligned(16))) bf16 kv_new[2][kDh];  // appended K and V row
  __shared__ __attribute__((aligned(16))) bf16 v_lds[16][kDh];  // the tile's V rows

  const int lane = threadIdx.x;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;

  // ---- every load goes out before any of them is waited on ----
  // Nothing here depends on cache_len[b]: the first tile is loaded up to the
  // split's end within T_max and masked once the length is known; the
  // projection / bias / norm loads are unconditional (absent biases and norms
  // read a harmless valid address and are masked to 0 / 1).
  const int L = p.cache_len[b];
  // splits of `chunk` keys; the last one also takes the remainder
  const int kbeg = split * p.chunk;
  const int kcap = split == p.nsplit - 1 ? p.T_max : min(kbeg + p.chunk, p.T_max);
  const size_t row_stride = (size_t)p.n_kv_heads * kDh;
  const bf16* kb_ = p.k_cache + (size_t)b * p.T_max * row_stride + g * kDh;
  const bf16* vb_ = p.v_cache + (size_t)b * p.T_max * row_stride + g * kDh;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  // tile at key k0: K lane (key col, k-group grp) holds dh [32 s + 8 grp, +8)
  // of key k0 + col; V lane holds dh piece col of keys k0 + 4 grp + j
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
  load_tile(kbeg, kcap, kcur, vcur);

  const int qd = p.n_q_heads * kDh;
  const int kvd = p.n_kv_heads * kDh;
  // Q^T fragments: lane (head col, group grp) holds dh [32s + 8grp, +8)
  bf16x8 qf[4];
  const bool valid = L >= 0 && L < p.T_max;
  const int nkeys = valid ? L + 1 : 0;
  const int kend = min(kcap, nkeys);
  const bool has_new = valid && kbeg <= L && L < kend;
  // first-tile rows past the live keys may hold anything (a NaN would survive
  // a zero softmax weight in P V): zero their V, once every load is out
  auto zero_dead_v = [&]() {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (kbeg + 4 * grp + j >= kend) vcur[j] = zero4;
  };
  {
    const float* raw = p.qkv_raw + (size_t)b * p.ld_raw;
    // slots 0 .. G-1: the group's query heads; G, G+1: the new K and V row
    float hv[G + 2][2], hb[G + 2][2];
#pragma unroll
    for (int i = 0; i < G + 2; ++i) {
      const int c0 = i < G ? (g * G + i) * kDh : (i == G ? qd + g * kDh : qd + kvd + g * kDh);
      hv[i][0] = raw[c0 + lane];
      hv[i][1] = raw[c0 + lane + 64];
      const bf16* bias = i < G ? p.bq : (i == G ? p.bk : p.bv);
      const bf16* bsrc = bias ? bias + (i < G ? c0 : g * kDh) : p.x;
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
    const double omega = p.rope_omega[lane];
    zero_dead_v();

    // ---- prologue: RMSNorm1 scale, q heads, the appended K/V row ----
    float inv = inv_given;
    if (!p.inv_rms) {
      const bf16* xr = p.x + (size_t)b * p.d;
      float ss = 0.f;
      for (int c = lane * 8; c < p.d; c += 64 * 8) {
        float f[8];
        unpack8(load_bf16x8(xr + c), f);
#pragma unroll
        for (int j = 0; j < 8; ++j) ss += f[j] * f[j];
      }
      inv = 1.0f / sqrtf(wave_sum_perm(ss) / (float)p.d + p.eps);
    }
    float sn, cs;
    {
      double ang = ((double)L + (double)p.pos_offset) * omega;
      const double two_pi = 6.283185307179586476925286766559;
      ang -= two_pi * rint(ang * (1.0 / two_pi));
      sincosf((float)ang, &sn, &cs);
    }
    // one head's 128 values: lane owns (lane, lane + 64); scale, bias, norm, rotate
    auto head_vec = [&](int i, bool norm, float g0, float g1, bool rotate, float& o0, float& o1) {
      float x0 = inv * hv[i][0] + hb[i][0];
      float x1 = inv * hv[i][1] + hb[i][1];
      if (norm) {
        const float hs = wave_sum_perm(x0 * x0 + x1 * x1);
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
    for (int hh = 0; hh < 16; ++hh) {
      float r0 = 0.f, r1 = 0.f;
      if (hh < G) {
        head_vec(hh, qkn, qg0r, qg1r, true, r0, r1);
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
    if (has_new) {
      float k0, k1, v0, v1;
      head_vec(G, qkn, kg0r, kg1r, true, k0, k1);
      head_vec(G + 1, false, 1.f, 1.f, false, v0, v1);
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
    // LDS traffic of one wave is processed in order; the barrier only keeps the
    // compiler from moving LDS accesses across it
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(&q_lds[col][32 * s + 8 * grp]);
  }

  float acc[HPL][8];
#pragma unroll
  for (int i = 0; i < HPL; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
  float m_run = -INFINITY;  // for head `col`
  float l_run = 0.f;

  for (int k0 = kbeg; k0 < kend; k0 += 16) {
    // the next tile's loads overlap this tile's arithmetic
    u32x4 knext[4], vnext[4];
    load_tile(k0 + 16, kend, knext, vnext);
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
    // V rows to LDS: row 4 grp + j, dh piece col
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4*>(&v_lds[4 * grp + j][col * 8]) = vcur[j];
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
    mt = xor32_max(xor16_max(mt));
    const float m_new = fmaxf(m_run, mt);  // finite: key k0 < kend is valid
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pv = exp2f(sc[r] - m_new);
      ps += pv;
      p_lds[(4 * grp + r) * 16 + col] = pv;
    }
    ps = xor32_sum(xor16_sum(ps));
    l_run = l_run * alpha + ps;
    if (grp == 0) a_lds[col] = alpha;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
    for (int i = 0; i < HPL; ++i) {
      // heads >= G (padding columns) are computed but never stored; reading
      // them unconditionally keeps the loop free of divergent loads
      const int h = grp + 4 * i;
      const float al = a_lds[h];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i][e] *= al;
    }
    // four keys at a time (the scheduling barrier bounds how many LDS reads
    // the compiler hoists, and with them the register count)
#pragma unroll
    for (int kq = 0; kq < 16; kq += 4) {
#pragma unroll
      for (int key = kq; key < kq + 4; ++key) {
        float v[8];
        unpack8(*reinterpret_cast<const bf16x8*>(&v_lds[key][col * 8]), v);
#pragma unroll
        for (int i = 0; i < HPL; ++i) {
          const int h = grp + 4 * i;
          const float pw = p_lds[key * 16 + h];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[i][e] += pw * v[e];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      kcur[s] = knext[s];
      vcur[s] = vnext[s];
    }
  }

  // per-head m and l (held by lanes grp 0, col = head) to every lane via LDS
  if (grp == 0) {
    a_lds[col] = l_run;
    p_lds[col] = m_run;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
  for (int i = 0; i < HPL; ++i) {
    const int h = grp + 4 * i;
    if (h >= G) continue;
    const int hq = g * G + h;
    if (p.nsplit == 1) {  // the only split: normalise here
      const float rl = valid ? 1.0f / a_lds[h] : __builtin_nanf("");
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = acc[i][e] * rl;
      store_out8(p, (size_t)b * p.ldo + (size_t)hq * kDh + col * 8, o);
    } else {
      const size_t slot = ((size_t)b * p.n_q_heads + hq) * p.nsplit + split;
      float* o = p.part_o + slot * kDh + col * 8;
      f32x4 o0, o1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o0[e] = acc[i][e];
        o1[e] = acc[i][e + 4];
      }
      *reinterpret_cast<f32x4*>(o) = o0;
      *reinterpret_cast<f32x4*>(o + 4) = o1;
      if (col == 0) {
        p.part_ml[slot * 2 + 0] = p_lds[h];
        p.part_ml[slot * 2 + 1] = a_lds[h];
      }
    }
  }
}

// Batched decode: the Q/K/V projection already finished the queries (scale,
// bias, QK-norm, RoPE) and appended the new row to the cache, so the wave only
// attends ("Qwen2.5-7B 结构拆解" §09.1; §05.2 for the shared K/V bytes of a
// group). One wave per (key split, KV head, sequence), 32 keys per step, both
// products on 16x16x32 MFMAs with the group's G <= 16 heads padded to 16:
//   * S^T = K Q^T: K rows straight from the cache as the A operand (two
//     16-key halves), Q^T fragments in registers;
//   * online softmax per head: lane (col, grp) holds keys 4 grp + r and
//     16 + 4 grp + r of head col, so the eight P values a lane owns are exactly
//     its B-operand slots of O^T += V^T P^T (k slot j < 4: key 4 grp + j,
//     j >= 4: key 16 + 4 grp + j - 4); P never leaves the registers;
//   * V^T: the tile's V rows are written transposed to LDS (four keys of one
//     dh value per 8-byte store) and read back as A fragments in that slot
//     order; the running output O^T (128 x 16) lives in eight accumulators,
//     rescaled only when some head's running maximum moved.
// Two register sets of 16 KB each are refilled with the tile after next as
// soon as they are consumed, so about two tiles stay in flight.
constexpr int kVtP = 36;  // bf16 per transposed-V row: 32 keys + 4 (bank spread)

QL_DEV void store_out4(const AttnDecodeArgs& p, size_t idx, const f32x4& v) {
  if (p.out_hilo) {
    bf16x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[e] = (bf16)v[e];
      l[e] = (bf16)(v[e] - (float)h[e]);
    }
    *reinterpret_cast<bf16x4*>(p.out_hilo + idx) = h;
    *reinterpret_cast<bf16x4*>(p.out_hilo + idx + p.lo_off) = l;
  } else {
    *reinterpret_cast<f32x4*>(p.out + idx) = v;
  }
}

// W > 1: the block's W waves are the splits of one (KV head, sequence) and
// merge in LDS at the end (waves past nsplit have no keys), so no combine
// kernel runs; W = 1: one wave per split, merged by the combine kernel.
// HM (head-major): the block's waves are the Hkv <= HMW KV heads of one
// (split, sequence), so the block's loads of a key cover the key's whole
// cache row across heads (Hkv x 256 contiguous bytes) at once; the splits
// merge in the combine kernel. (A load-only probe of the Qwen3-8B B = 64
// cache: 6.7 TB/s head-major against 5.9 TB/s split-major.)
constexpr int kHmMaxHeads = 8;
template <int G, int W, bool HM = false>
__global__ __launch_bounds__(HM ? 64 * kHmMaxHeads : 64 * W) __attribute__((amdgpu_waves_per_eu(2))) void attn_decode_mfma_kernel(const AttnDecodeArgs p) {
  static_assert(G >= 1 && G <= 16, "query heads per KV head");
  static_assert(16 * kDh * sizeof(float) <= kDh * kVtP * sizeof(bf16), "merge rows fit a V^T slot");
  static_assert(!HM || W == 1, "head-major blocks merge through the combine kernel");
  constexpr int NWV = HM ? kHmMaxHeads : W;  // waves of the block
  __shared__ __attribute__((aligned(16))) bf16 vt_all[NWV][kDh * kVtP];

  const int wave = NWV == 1 ? 0 : (int)(threadIdx.x >> 6);
  bf16* vt_lds = vt_all[wave];
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  // KV heads fastest: the Hkv waves of one key range read neighbouring bytes
  const int g = HM ? wave : (int)blockIdx.x;
  const int split = HM ? (int)blockIdx.x : (W == 1 ? (int)blockIdx.y : wave);
  const int b = HM ? (int)blockIdx.y : (int)blockIdx.z;
  const bool idle = split >= p.nsplit;  // W > 1 only

  // splits of `chunk` keys; the last one also takes the remainder
  const int kbeg = idle ? 0 : split * p.chunk;
  const int kcap = idle ? min(p.chunk, p.T_max)
                        : (split == p.nsplit - 1 ? p.T_max : min(kbeg + p.chunk, p.T_max));
  const size_t rs = (size_t)p.n_kv_heads * kDh;
  const bf16* kb_ = p.k_cache + (size_t)b * p.T_max * rs + g * kDh;
  const bf16* vb_ = p.v_cache + (size_t)b * p.T_max * rs + g * kDh;
  // K lane (key col of half h, k-group grp): dh [32 s + 8 grp, +8) of key
  // k0 + 16 h + col. V lane: keys k0 + vkey + j (j < 4), dh pieces vpc + 8 i.
  // Loads are unconditional (a guarded load becomes a branch whose join waits
  // for it): rows at or past `lim` read row lim - 1 instead; such K rows are
  // masked in the scores and such V rows meet a zero weight. The cache is
  // read once per call, so its loads carry the non-temporal hint (3-7 %
  // faster on the 1 GB caches of batch 64-128 at 4096 rows).
  const int vkey = 4 * (lane & 7);
  const int vpc = lane >> 3;
  auto load_k = [&](int k0, int lim, u32x4 (&kt)[2][4]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16* kr = kb_ + (size_t)min(k0 + 16 * h + col, lim - 1) * rs + 8 * grp;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        kt[h][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kr + 32 * s));
    }
  };
  auto load_v = [&](int k0, int lim, u32x4 (&vv)[2][4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16* vr = vb_ + (size_t)min(k0 + vkey + j, lim - 1) * rs + 8 * vpc;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        vv[i][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vr + 64 * i));
    }
  };

  const int qd = p.n_q_heads * kDh;
  bf16x8 qf[4];  // Q^T fragments: lane (head col, grp) holds dh [32 s + 8 grp, +8)
  {
    const bf16* qrow = p.q_in + (size_t)b * qd + (size_t)(g * G + min(col, G - 1)) * kDh + 8 * grp;
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[s] = load_bf16x8(qrow + 32 * s);
  }
  // Two tiles in registers (A, B). The first two do not wait for cache_len:
  // they are read up to the split's end within T_max; their rows past the
  // live keys may hold anything (a NaN would survive a zero softmax weight),
  // so the first two steps zero those V rows.
  u32x4 kA[2][4], vA[2][4], kB[2][4], vB[2][4];
  load_k(kbeg, kcap, kA);
  load_v(kbeg, kcap, vA);
  load_k(kbeg + 32, kcap, kB);
  load_v(kbeg + 32, kcap, vB);
  if (col >= G) {
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[s] = bf16x8{};
  }
  const int L = p.cache_len[b];
  const bool valid = L >= 0 && L < p.T_max;
  const int kend = idle ? 0 : min(kcap, valid ? L + 1 : 0);

  f32x4 acc[8];  // lane: O^T[dh 16 blk + 4 grp + r][head col]
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // head col
  float l_run = 0.f;        // head col, this lane's keys only

  // One 32-key step on the tile held in (kt, vv); the other buffer holds the
  // next tile. Each register set is refilled with the tile after next as soon
  // as it is consumed (V after its LDS transpose, K after the scores), so
  // about two tiles stay in flight during the arithmetic.
  auto step = [&](int k0, u32x4 (&kt)[2][4], u32x4 (&vv)[2][4], auto first) {
    // V^T rows: dh 8 (vpc + 8 i) + e, keys vkey .. vkey + 3
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      bf16x8 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] = *reinterpret_cast<const bf16x8*>(&vv[i][j]);
        if constexpr (decltype(first)::value)
          if (k0 + vkey + j >= kend) v[j] = bf16x8{};
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bf16x4 t = {v[0][e], v[1][e], v[2][e], v[3][e]};
        *reinterpret_cast<bf16x4*>(&vt_lds[(8 * (vpc + 8 * i) + e) * kVtP + vkey]) = t;
      }
    }
    load_v(k0 + 64, kend, vv);  // the tile after next
    f32x4 sc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        sc[h] = mfma_16x16x32(*reinterpret_cast<const bf16x8*>(&kt[h][s]), qf[s], sc[h]);
    }
    load_k(k0 + 64, kend, kt);
    // sc[h][r]: S^T[key k0 + 16 h + 4 grp + r][head col]
    float mt = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = sc[h][r] * p.scale_log2;
        if (k0 + 16 * h + 4 * grp + r >= kend) x = -INFINITY;
        sc[h][r] = x;
        mt = fmaxf(mt, x);
      }
    mt = xor32_max(xor16_max(mt));
    const float m_new = fmaxf(m_run, mt);  // finite: key k0 < kend is live
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    bf16x8 pf;
    float ps = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // the sum takes the rounded weights P*V is formed with, so the
        // normalised weights sum to one
        const bf16 pb = (bf16)exp2f(sc[h][r] - m_new);
        ps += (float)pb;
        pf[4 * h + r] = pb;
      }
    l_run = l_run * alpha + ps;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][r] *= alpha;
    }
    // LDS traffic of one wave is processed in order; the barrier only keeps
    // the compiler from moving LDS accesses across it
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bf16* vr = &vt_lds[(16 * i + col) * kVtP + 4 * grp];
      const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vr);
      const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vr + 16);
      const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      acc[i] = mfma_16x16x32(vf, pf, acc[i]);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  };
  using First = std::integral_constant<bool, true>;
  using Rest = std::integral_constant<bool, false>;
  // steps go in pairs; a second step past kend has every key masked and
  // changes nothing (its refill loads stay inside the live rows)
  if (kbeg < kend) {
    step(kbeg, kA, vA, First{});
    step(kbeg + 32, kB, vB, First{});
    for (int k0 = kbeg + 64; k0 < kend; k0 += 64) {
      step(k0, kA, vA, Rest{});
      step(k0 + 32, kB, vB, Rest{});
    }
  }

  l_run = xor32_sum(xor16_sum(l_run));
  if constexpr (W > 1) {
    // each wave's partial (m, l, O) to LDS (O in its own V^T slot, which only
    // this wave has used), then the block merges: thread t takes elements
    // t, t + 64 W, ... of the G x 128 outputs
    __shared__ float mb[W][16], lb[W][16];
    float* ob = reinterpret_cast<float*>(vt_lds);  // [16][128]
    if (col < G) {
#pragma unroll
      for (int i = 0; i < 8; ++i) *reinterpret_cast<f32x4*>(ob + col * kDh + 16 * i + 4 * grp) = acc[i];
      if (grp == 0) {
        mb[wave][col] = m_run;
        lb[wave][col] = l_run;
      }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < G * kDh; e += 64 * W) {
      const int h = e / kDh, d = e % kDh;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < W; ++w) M = fmaxf(M, mb[w][h]);
      float l = 0.f, o = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float m = mb[w][h];
        const float wt = m == -INFINITY ? 0.f : exp2f(m - M);
        l += wt * lb[w][h];
        o += wt * reinterpret_cast<const float*>(vt_all[w])[h * kDh + d];
      }
      const float v = valid ? o / l : __builtin_nanf("");
      const size_t idx = (size_t)b * p.ldo + (size_t)(g * G + h) * kDh + d;
      if (p.out_hilo) {
        const bf16 hi = (bf16)v;
        p.out_hilo[idx] = hi;
        p.out_hilo[idx + p.lo_off] = (bf16)(v - (float)hi);
      } else {
        p.out[idx] = v;
      }
    }
    return;
  }
  if (col >= G) return;
  const int hq = g * G + col;
  if (p.nsplit == 1) {  // the only split: normalise here
    const float rl = valid ? 1.0f / l_run : __builtin_nanf("");
    const size_t base = (size_t)b * p.ldo + (size_t)hq * kDh + 4 * grp;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      f32x4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = acc[i][r] * rl;
      store_out4(p, base + 16 * i, o);
    }
  } else {
    const size_t slot = ((size_t)b * p.n_q_heads + hq) * p.nsplit + split;
    float* o = p.part_o + slot * kDh + 4 * grp;
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<f32x4*>(o + 16 * i) = acc[i];
    if (grp == 0) {
      p.part_ml[slot * 2 + 0] = m_run;
      p.part_ml[slot * 2 + 1] = l_run;
    }
  }
}

// Merge the splits of one (sequence, head): one wave per head, lane owns
// output elements 2 lane and 2 lane + 1; lane s holds split s's (m, l). Up
// to 64 splits take one round trip: every split's (m, l) and partial output
// are requested before any is used (the loads are unconditional, since a
// guarded load becomes a branch whose join waits for it: rows past the last
// split re-read it and get weight 0); the split weights w_s = 2^(m_s - max m)
// then reach every lane by lane reads. More splits take one such round per
// 64 after a first pass for the maximum.
template <int U>
QL_DEV void combine_round(const AttnDecodeArgs& p, size_t base, int s0, int n, int lane, float M_in,
                          bool have_max, float& M_out, float& o0, float& o1, float& l) {
  const int sl = s0 + min(lane, n - 1);
  const float m = p.part_ml[(base + sl) * 2];
  const float ls = p.part_ml[(base + sl) * 2 + 1];
  float2 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u)
    v[u] = *reinterpret_cast<const float2*>(p.part_o + (base + s0 + min(u, n - 1)) * kDh + 2 * lane);
  const float M = have_max ? M_in : wave_max_perm(lane < n ? m : -INFINITY);
  M_out = M;
  const float w = lane < n && m != -INFINITY ? exp2f(m - M) : 0.f;
  l += w * ls;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u));
    o0 += wu * v[u].x;
    o1 += wu * v[u].y;
  }
}

constexpr int kCombineWaves = 4;
__global__ __launch_bounds__(64 * kCombineWaves) void attn_decode_combine_kernel(const AttnDecodeArgs p) {
  const int lane = threadIdx.x & 63;
  const int bh = blockIdx.x * kCombineWaves + (threadIdx.x >> 6);  // b * Hq + head
  if (bh >= p.B * p.n_q_heads) return;
  const int b = bh / p.n_q_heads;
  const int ns = p.nsplit;
  const size_t base = (size_t)bh * ns;
  float M = -INFINITY, o0 = 0.f, o1 = 0.f, l = 0.f;
  if (ns <= 8) {
    combine_round<8>(p, base, 0, ns, lane, 0.f, false, M, o0, o1, l);
  } else if (ns <= 64) {
    combine_round<64>(p, base, 0, ns, lane, 0.f, false, M, o0, o1, l);
  } else {
    for (int s = lane; s < ns; s += 64) M = fmaxf(M, p.part_ml[(base + s) * 2]);
    M = wave_max_perm(M);
    for (int s0 = 0; s0 < ns; s0 += 64)
      combine_round<64>(p, base, s0, min(64, ns - s0), lane, M, true, M, o0, o1, l);
  }
  l = wave_sum_perm(l);
  const int L = p.cache_len[b];
  const bool valid = L >= 0 && L < p.T_max;
  const float rl = valid ? 1.0f / l : __builtin_nanf("");
  const float v0 = o0 * rl, v1 = o1 * rl;
  const size_t idx = (size_t)b * p.ldo + (size_t)(bh % p.n_q_heads) * kDh + 2 * lane;
  if (p.out_hilo) {
    const bf16 h0 = (bf16)v0, h1 = (bf16)v1;
    *reinterpret_cast<bf16x2*>(p.out_hilo + idx) = bf16x2{h0, h1};
    *reinterpret_cast<bf16x2*>(p.out_hilo + idx + p.lo_off) =
        bf16x2{(bf16)(v0 - (float)h0), (bf16)(v1 - (float)h1)};
  } else {
    *reinterpret_cast<float2*>(p.out + idx) = float2{v0, v1};
  }
}

}  // namespace

hipError_t ql_attn_decode_bf16(const AttnDecodeArgs& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  if (a.nsplit < 1 || a.nsplit > kMaxDecodeSplits) return hipErrorInvalidValue;
  const dim3 grid(a.nsplit, a.n_kv_heads, a.B);
  const dim3 grid_kv(a.n_kv_heads, a.nsplit, a.B);
  // finished queries with up to 8 splits: the splits are the waves of one
  // block and merge there
  // finished queries: head-major blocks (all KV heads of one split and
  // sequence) when the heads fit one block, else the splits of one head as
  // the waves of a block (<= 8 splits) or one wave per split
  const bool hm = a.q_in && a.n_kv_heads >= 2 && a.n_kv_heads <= kHmMaxHeads;
  const int wm = hm || !a.q_in || a.nsplit == 1 || a.nsplit > 8
                     ? 1 : (a.nsplit <= 2 ? 2 : a.nsplit <= 4 ? 4 : 8);
  const dim3 grid_wg(a.n_kv_heads, 1, a.B);
  const dim3 grid_hm(a.nsplit, a.B);
  switch (a.n_q_heads / a.n_kv_heads) {
#define QL_G(V)                                                                                 \
  case V:                                                                                       \
    if (!a.q_in)                                                                                \
      hipLaunchKernelGGL((attn_decode_kernel<V>), grid, dim3(64), 0, s, a);                     \
    else if (hm)                                                                                \
      hipLaunchKernelGGL((attn_decode_mfma_kernel<V, 1, true>), grid_hm, dim3(64 * a.n_kv_heads), \
                         0, s, a);                                                              \
    else if (wm == 1)                                                                           \
      hipLaunchKernelGGL((attn_decode_mfma_kernel<V, 1>), grid_kv, dim3(64), 0, s, a);          \
    else if (wm == 2)                                                                           \
      hipLaunchKernelGGL((attn_decode_mfma_kernel<V, 2>), grid_wg, dim3(128), 0, s, a);         \
    else if (wm == 4)                                                                           \
      hipLaunchKernelGGL((attn_decode_mfma_kernel<V, 4>), grid_wg, dim3(256), 0, s, a);         \
    else                                                                                        \
      hipLaunchKernelGGL((attn_decode_mfma_kernel<V, 8>), grid_wg, dim3(512), 0, s, a);         \
    break;
    QL_G(1) QL_G(2) QL_G(3) QL_G(4) QL_G(5) QL_G(6) QL_G(7) QL_G(8)
    QL_G(9) QL_G(10) QL_G(11) QL_G(12) QL_G(13) QL_G(14) QL_G(15) QL_G(16)
#undef QL_G
    default:
      return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1 || wm > 1) return e;
  const int heads = a.B * a.n_q_heads;
  hipLaunchKernelGGL(attn_decode_combine_kernel, dim3((heads + kCombineWaves - 1) / kCombineWaves),
                     dim3(64 * kCombineWaves), 0, s, a);
  return hipGetLastError();
}

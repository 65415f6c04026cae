// Causal GQA attention for prefill, head_dim 128, tiled online softmax on MFMA.
//
// For query head h of sequence b, rows t and keys u <= t:
//   o_t = sum_u softmax_u(q_t . k_u / sqrt(dh)) v_u,  KV head g = h / (Hq/Hkv)
// A sequence may start over a cache prefix of P rows (chunked prefill): its
// new row t is then key position P + t and sees the P prefix keys too
// ("Qwen2.5-7B 结构拆解" §09.1), and sequences of one call may differ in
// length (a varlen batch, rows concatenated).
// ("推理系统 03：逐项算清一个真实 Qwen3 Transformer 层" §7-§9; "Qwen2.5-7B 结构拆解"
// §05, §05.2: the KV head is indexed, never copied; §05.4: tiles above the
// diagonal are skipped in both products). The [S, S] probability matrix is
// never written to memory ("推理系统 03" §12).
//
// Block = 4 waves on 128 query rows of one (sequence, head); a wave owns 32
// rows. With KSPLIT the block has two such groups of 4 waves: group 0 takes
// the first half of the query tile's key tiles and group 1 the rest, and the
// two partial softmax states are merged through LDS at the end. That halves
// the longest tiles' time when the causal work would otherwise leave most
// CUs idle behind them (grids of at most one block per CU).
// Key tiles of 64 rows stream through LDS, double-buffered per group.
// Scores are formed transposed, S^T = K Q^T, with 32x32x16 MFMAs: the query
// is the MFMA column, so a lane owns one query and its running max / sum
// need only one cross-lane exchange per tile. P^T stays in registers and is
// the B operand of O^T += V^T P^T; V is stored transposed in LDS (pitch 68
// elements, which spreads the rows read together over distinct banks; the
// 16 lanes of a store cover 64 keys of one row). K rows are padded to 136
// elements, so the 16 lanes of a fragment read fall on distinct banks and a
// lane's fragments sit at fixed offsets from one base. The fp32 output is
// stored as a bf16 pair hi + lo, the form in which the O projection reads it.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kDh = 128;
constexpr int kBQ = 128;      // queries per block
constexpr int kBK = 64;       // keys per tile
constexpr int kVtPitch = 68;  // bf16 elements per transposed-V row
constexpr int kKPitch = kDh + 8;  // bf16 elements per K row
constexpr int kKElems = kBK * kKPitch;
constexpr int kVElems = kDh * kVtPitch;
constexpr int kStage = kKElems + kVElems;
constexpr float kSlack = 8.f;  // lazy-rescale threshold, log2 units
constexpr int kCUs = 256;

typedef float f32v2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16v2 __attribute__((ext_vector_type(2)));
constexpr bf16v2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

// Two 4-wave blocks per CU (one 68 KiB ring each), or one KSPLIT block with
// two rings: the register budget of two waves per SIMD keeps every
// accumulator in VGPRs, and one wave's MFMAs run while the other works
// through its softmax.
template <bool KSPLIT>
__global__ __launch_bounds__(KSPLIT ? 512 : 256, KSPLIT ? 1 : 2) void attn_prefill_kernel(
    const AttnPrefillArgs p) {
  constexpr int NG = KSPLIT ? 2 : 1;  // wave groups
  __shared__ __attribute__((aligned(16))) bf16 lds[NG * 2 * kStage];  // [group][stage]
  const int lane = threadIdx.x & 63;
  const int grp = KSPLIT ? (int)(threadIdx.x >> 8) : 0;  // key half
  const int tid = threadIdx.x & 255;                     // thread within the group
  const int wave = tid >> 6;          // query rows 32 wave .. +31 of the tile
  const int col = lane & 31;
  const int hi = lane >> 5;
  // XCD-aware order: the work items (tile slot x fastest, then query head,
  // then sequence) are cut into 8 contiguous stretches and block L runs item
  // (L mod 8) * stretch + L / 8; consecutive blocks go to the 8 XCDs in turn,
  // so each XCD walks whole heads and the query heads of one KV group find
  // its K/V tiles in that XCD's L2 (attention 2-5 % faster)
  const int wl = (int)blockIdx.x;
  const int wchunk = (p.gtotal + 7) / 8;
  const int wi = (wl % 8) * wchunk + wl / 8;
  if (wi >= p.gtotal) return;  // block-uniform, before any barrier
  const int bx = wi % p.gx;
  const int h = (wi / p.gx) % p.gy;
  const int b = wi / (p.gx * p.gy);
  const int g = h / (p.n_q_heads / p.n_kv_heads);
  // Sequence b: S new query rows from q row qbase, keys = its cache rows
  // 0 .. P + S - 1, the first P of them an earlier prefix; new row t is at
  // key position P + t and sees keys <= P + t. Uniform batches: qbase = b S,
  // P = 0.
  const int qbase = p.seq_start ? p.seq_start[b] : b * p.S;
  const int S = p.seq_start ? p.seq_start[b + 1] - qbase : p.S;
  const int P = p.prefix ? p.prefix[b] : 0;
  const int L = P + S;  // keys of the sequence
  // Causal work grows with the query tile, so with p.pair a block takes tile
  // nqt-1-x and then tile x: every block then does about the same work.
  // Otherwise a block takes one tile, the longest first. (Grids are sized
  // for the longest sequence; a shorter one's extra blocks have no tile.)
  const int nqt = (S + kBQ - 1) / kBQ;
  const int qt_first = p.pair ? nqt - 1 - bx : (p.gx - 1 - bx) - (p.gx - nqt);
  // block-uniform, before any barrier: no tile, or (pairs) a tile that a
  // lower block already takes as its second
  if (qt_first < 0 || (p.pair && bx > qt_first)) return;
  const int npass = (p.pair && bx < qt_first) ? 2 : 1;
  for (int pass = 0; pass < npass; ++pass) {
  if (pass > 0) __syncthreads();  // the LDS ring is reused
  const int qt = pass == 0 ? qt_first : bx;
  const int q0 = qt * kBQ;
  const int my_q = q0 + wave * 32 + col;         // new row of this lane's query
  const int my_pos = P + my_q;                   // its key position
  const int wave_qmax = P + q0 + wave * 32 + 31;

  // Q^T fragments (B operand): lane (query col, group hi) holds dh [16s+8hi, +8)
  bf16x8 qf[8];
  {
    const bf16* qrow = p.q + (size_t)(qbase + min(my_q, S - 1)) * p.ldq + h * kDh;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = load_bf16x8(qrow + 16 * s + 8 * hi);
  }

  const size_t kv_row_stride = (size_t)p.n_kv_heads * kDh;
  const bf16* kbase = p.k_cache + ((size_t)b * p.T_max) * kv_row_stride + g * kDh;
  const bf16* vbase = p.v_cache + ((size_t)b * p.T_max) * kv_row_stride + g * kDh;
  const int kend = min(P + q0 + kBQ, L);  // keys needed by this block
  const int ntiles = (kend + kBK - 1) / kBK;
  // this group's key tiles [kt_lo, kt_hi); both groups step niter times
  const int kt_lo = !KSPLIT ? 0 : grp == 0 ? 0 : ntiles / 2;
  const int kt_hi = !KSPLIT ? ntiles : grp == 0 ? ntiles / 2 : ntiles;
  const int niter = !KSPLIT ? ntiles : ntiles - ntiles / 2;
  bf16* ring = lds + grp * 2 * kStage;

  // tile-load assignment
  //   K: chunk = tid + 256*i, key = chunk >> 4, 16-byte piece c = chunk & 15
  //   V: keys 4*(tid & 15) .. +3, 8-wide dh piece c = tid >> 4
  const int vk = (tid & 15) * 4;
  const int vc = tid >> 4;
  u32x4 rk[4], rv[4];
  // piece idx of tile kt's prefetch (0-3: K, 4-7: V). Rows at or past the
  // sequence's end read its last row (an in-bounds address, so the load
  // needs no branch) and are zeroed at the LDS store: they may hold
  // anything, and a NaN would survive a zero softmax weight in P V.
  auto gload1 = [&](int kt, int idx) {
    const int k0 = kt * kBK;
    if (idx < 4) {
      const int ch = tid + 256 * idx;
      rk[idx] = *reinterpret_cast<const u32x4*>(
          kbase + (size_t)min(k0 + (ch >> 4), L - 1) * kv_row_stride + (ch & 15) * 8);
    } else {
      const int j = idx - 4;
      rv[j] = *reinterpret_cast<const u32x4*>(
          vbase + (size_t)min(k0 + vk + j, L - 1) * kv_row_stride + vc * 8);
    }
  };
  auto gload = [&](int kt) {
#pragma unroll
    for (int idx = 0; idx < 8; ++idx) gload1(kt, idx);
  };
  auto lstore = [&](int st, int kt) {
    const int k0 = kt * kBK;
    if (k0 + kBK > L) {  // ragged last tile (block-uniform)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (k0 + ((tid + 256 * i) >> 4) >= L) rk[i] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (k0 + vk + j >= L) rv[j] = u32x4{0u, 0u, 0u, 0u};
    }
    bf16* Ks = ring + st * kStage;
    bf16* Vt = Ks + kKElems;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = tid + 256 * i;
      const int key = ch >> 4, c = ch & 15;
      *reinterpret_cast<u32x4*>(Ks + key * kKPitch + c * 8) = rk[i];
    }
    const bf16x8 v0 = *reinterpret_cast<const bf16x8*>(&rv[0]);
    const bf16x8 v1 = *reinterpret_cast<const bf16x8*>(&rv[1]);
    const bf16x8 v2 = *reinterpret_cast<const bf16x8*>(&rv[2]);
    const bf16x8 v3 = *reinterpret_cast<const bf16x8*>(&rv[3]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bf16x4 t = {v0[e], v1[e], v2[e], v3[e]};
      *reinterpret_cast<bf16x4*>(Vt + (vc * 8 + e) * kVtPitch + vk) = t;
    }
  };

  f32x16 acc_o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[dt][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  if (kt_lo < kt_hi) {
    gload(kt_lo);
    lstore(0, kt_lo);
  }
  // Drain the Q-fragment loads on every path into the key loop. Left to
  // itself the compiler cannot tell, inside the loop, that they have landed,
  // and waits on the vector-memory counter before the first score MFMAs,
  // which then also waits for the next tile's prefetch issued just above
  // them: the tile load's latency is exposed in every iteration.
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // vmcnt(0) only
  __syncthreads();

  for (int it = 0; it < niter; ++it) {
    const int kt = kt_lo + it;
    const int st = it & 1;
    const bool more = kt + 1 < kt_hi;
    // the next tile's prefetch (the last step re-reads its own tile, unused,
    // so the loads need no branch and can sit among the score MFMAs)
    const int ktn = more ? kt + 1 : kt;
    const int k0 = kt * kBK;
    // skip tiles past the group's range (its last step when it has one tile
    // fewer) and tiles whose every key is in this wave's future (wave-uniform)
    if (__builtin_amdgcn_readfirstlane(kt < kt_hi && k0 <= wave_qmax)) {
      const bf16* Ks = ring + st * kStage;
      const bf16* Vt = Ks + kKElems;
      f32x16 sc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[t][r] = 0.f;
        const bf16* kr = Ks + (32 * t + col) * kKPitch + 8 * hi;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kr + 16 * s);
          sc[t] = mfma_32x32x16(kf, qf[s], sc[t]);
          if (s & 1) gload1(ktn, 4 * t + (s >> 1));
        }
      }
      // issue order: per pair of score MFMAs, their two K-fragment reads,
      // the MFMAs and one 16-byte global load of the next tile, so the
      // loads' issue overlaps the matrix work instead of stalling the wave
      // ahead of it
#pragma unroll
      for (int g8 = 0; g8 < 8; ++g8) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
      }
      // mask, tile max (raw scores; the scale is positive and applied in the
      // exponent). Register r of half t holds key 32t + 8(r/4) + 4hi + r%4.
      // The mask test is wave-uniform (readfirstlane), so the common unmasked
      // tile carries no per-element code.
      const bool need_mask = __builtin_amdgcn_readfirstlane(
          (k0 + kBK - 1 > P + q0 + wave * 32) || (k0 + kBK > L));
      if (need_mask) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * t + 8 * (r >> 2) + 4 * hi + (r & 3);
            sc[t][r] = (key > my_pos || key >= L) ? -INFINITY : sc[t][r];
          }
      }
      float mt = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sc[t][r]);
      mt = fmaxf(mt, __shfl_xor(mt, 32, kWave)) * p.scale_log2;
      // Lazy rescaling: the reference maximum only moves when a score exceeds
      // it by more than kSlack (log2 units), so p <= 2^kSlack and the output
      // is unchanged (numerator and denominator use the same reference); the
      // rescale of the accumulators runs only when some lane moved.
      const bool grow = mt > m_run + kSlack;  // first tile: m_run = -inf
      if (__any(grow)) {
        // lanes that do not grow keep their reference (alpha = 1; their
        // m_run may still be -inf, where m_run - m_run is not 0)
        const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mt) : 1.f;
        m_run = grow ? mt : m_run;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc_o[dt][r] *= alpha;
      }
      // A lane whose keys so far were all in its future still has m_run =
      // -inf, and then so is every score of this tile (a finite one would
      // have moved m_run): its weights are 0, not exp2(-inf + inf). This
      // happens with a cache prefix, whose length need not be a multiple of
      // the tile, in the second key group of a split tile, and in the
      // rescale above.
      const float m_ref = m_run == -INFINITY ? 0.f : m_run;
      // Weights are rounded to bf16 two at a time (one packed convert), and
      // the row sum is taken from those rounded pairs by a two-term dot
      // product with (1, 1), so it sums exactly the weights P*V is formed
      // with, at one instruction per pair.
      float lsum0 = 0.f, lsum1 = 0.f;
      u32x4 pfw[4];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const f32v2 e = {__builtin_amdgcn_exp2f(fmaf(sc[t][r], p.scale_log2, -m_ref)),
                           __builtin_amdgcn_exp2f(fmaf(sc[t][r + 1], p.scale_log2, -m_ref))};
          const bf16v2 pb = __builtin_convertvector(e, bf16v2);
          if (r & 2) lsum1 = __builtin_amdgcn_fdot2_f32_bf16(pb, kOnes2, lsum1, false);
          else lsum0 = __builtin_amdgcn_fdot2_f32_bf16(pb, kOnes2, lsum0, false);
          pfw[2 * t + (r >> 3)][(r & 7) >> 1] = __builtin_bit_cast(uint32_t, pb);
        }
      l_run += lsum0 + lsum1;
      bf16x8 pf[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) pf[u] = __builtin_bit_cast(bf16x8, pfw[u]);
      // O^T[d][q] += sum_key V^T[d][key] P^T[key][q]; k-step u covers keys
      // 32(u/2) + 16(u%2) + {4hi..4hi+3, 8+4hi..8+4hi+3} in slot order.
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kb = 32 * (u >> 1) + 16 * (u & 1) + 4 * hi;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const bf16* vr = Vt + (32 * dt + col) * kVtPitch + kb;
          const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vr);
          const bf16x4 hi4 = *reinterpret_cast<const bf16x4*>(vr + 8);
          const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi4[0], hi4[1], hi4[2], hi4[3]};
          acc_o[dt] = mfma_32x32x16(vf, pf[u], acc_o[dt]);
        }
      }
    } else {
      gload(ktn);
    }
    if (more) lstore(st ^ 1, kt + 1);
    __syncthreads();
  }

  // merge: group 1 hands its state to group 0 through LDS (the rings are
  // free: every tile read ended before the loop's last barrier). A lane's
  // state is relative to its own reference maximum m_run; a group that saw
  // no key of this query has m_run = -inf and contributes nothing.
  static_assert(4 * 66 * 64 * 4 <= 2 * kStage * 2, "merge state fits group 0's ring");
  float* mst = reinterpret_cast<float*>(lds) + wave * (66 * 64) + lane;
  if (KSPLIT && grp == 1) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mst[(16 * dt + r) * 64] = acc_o[dt][r];
    mst[64 * 64] = m_run;
    mst[65 * 64] = l_run;
  }
  if (KSPLIT) __syncthreads();
  if (grp == 1) continue;  // (the next pass starts with a barrier)
  if (KSPLIT) {
    const float m1 = mst[64 * 64], l1 = mst[65 * 64];
    const float m = fmaxf(m_run, m1);  // finite: every query sees key 0
    const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m);
    const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
    l_run = a0 * l_run + a1 * l1;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[dt][r] = a0 * acc_o[dt][r] + a1 * mst[(16 * dt + r) * 64];
  }
  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  const float inv = 1.0f / l_tot;
  // The fp32 output as a bf16 pair: hi = RNE(o) at column c, lo = RNE(o - hi)
  // at column c + lo_off (the O projection multiplies both). A lane holds 16
  // pieces of 4 values of one query row, so the rows are staged through LDS
  // as [query][dh] (in the ring of group 1, or of the only group: every tile
  // read ended before the loop's last barrier) and stored as whole 256-byte
  // rows, 16 lanes to a row, rather than as 8-byte pieces of 32 rows. Rows
  // past the sequence (a ragged last tile) are computed and not stored.
  constexpr int kOP = kDh + 8;  // staging pitch, bf16 elements
  static_assert(4 * 2 * 32 * kOP <= 2 * kStage, "output staging fits one ring");
  bf16* so = lds + (KSPLIT ? 2 * kStage : 0) + wave * (2 * 32 * kOP);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bf16x4 vh, vl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = acc_o[dt][4 * c + e] * inv;
        vh[e] = (bf16)v;
        vl[e] = (bf16)(v - (float)vh[e]);
      }
      *reinterpret_cast<bf16x4*>(so + col * kOP + 32 * dt + 8 * c + 4 * hi) = vh;
      *reinterpret_cast<bf16x4*>(so + (32 + col) * kOP + 32 * dt + 8 * c + 4 * hi) = vl;
    }
  // (the wave's own LDS writes and reads run in order; the fences keep the
  // compiler from moving the reads above the writes)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  bf16x8 h8[8], l8[8];  // query rows 4 i + lane / 16, columns 8 (lane % 16) ..
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 4 * i + (lane >> 4);
    h8[i] = *reinterpret_cast<const bf16x8*>(so + r * kOP + 8 * (lane & 15));
    l8[i] = *reinterpret_cast<const bf16x8*>(so + (32 + r) * kOP + 8 * (lane & 15));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int qr = q0 + wave * 32 + 4 * i + (lane >> 4);
    if (qr < S) {
      bf16* o = p.out + (size_t)(qbase + qr) * p.ldo + h * kDh + 8 * (lane & 15);
      *reinterpret_cast<bf16x8*>(o) = h8[i];
      *reinterpret_cast<bf16x8*>(o + p.lo_off) = l8[i];
    }
  }
  }  // pass
}

}  // namespace

hipError_t ql_attn_prefill_bf16(const AttnPrefillArgs& a, hipStream_t s) {
  if (a.B <= 0 || a.S <= 0) return hipSuccess;
  // (a.S: the longest sequence's new rows when seq_start is set)
  const int nqt = (a.S + kBQ - 1) / kBQ;
  const long pairs = (long)((nqt + 1) / 2) * a.n_q_heads * a.B;
  const long tiles = (long)nqt * a.n_q_heads * a.B;
  AttnPrefillArgs b = a;
  if (pairs >= 2L * kCUs) {
    // enough tile pairs (equal work each) for two 4-wave blocks per CU
    b.pair = true;
    b.gx = (nqt + 1) / 2;
    b.gy = a.n_q_heads;
    b.gtotal = b.gx * b.gy * a.B;
    hipLaunchKernelGGL(attn_prefill_kernel<false>, dim3(8 * ((b.gtotal + 7) / 8)), dim3(256), 0,
                       s, b);
  } else if (pairs >= kCUs || tiles <= kCUs) {
    // one 8-wave block per CU, each tile's keys split between its two groups:
    // tile pairs when they fill the CUs, else single tiles
    b.pair = pairs >= kCUs;
    b.gx = b.pair ? (nqt + 1) / 2 : nqt;
    b.gy = a.n_q_heads;
    b.gtotal = b.gx * b.gy * a.B;
    hipLaunchKernelGGL(attn_prefill_kernel<true>, dim3(8 * ((b.gtotal + 7) / 8)), dim3(512), 0,
                       s, b);
  } else {
    // single tiles, longest first, two 4-wave blocks per CU
    b.pair = false;
    b.gx = nqt;
    b.gy = a.n_q_heads;
    b.gtotal = b.gx * b.gy * a.B;
    hipLaunchKernelGGL(attn_prefill_kernel<false>, dim3(8 * ((b.gtotal + 7) / 8)), dim3(256), 0,
                       s, b);
  }
  return hipGetLastError();
}

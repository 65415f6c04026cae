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
// Key tiles of 64 rows stream through LDS, double-buffered per group, by
// direct global-to-LDS loads (no registers hold them on the way): K and V
// rows of 256 bytes as they sit in the cache, each 16-byte chunk c of row r
// at chunk position c ^ f(r) of the row, f(r) = r mod 16 for K and
// 4 (r mod 4) for V, which puts the lanes of every fragment read on
// distinct banks. Scores are formed transposed, S^T = K Q^T, with 32x32x16
// MFMAs: the query is the MFMA column, so a lane owns one query and its
// running max / sum need only one cross-lane exchange per tile. P^T stays
// in registers and is the B operand of O^T += V^T P^T; the V^T fragments
// come from the row-major V tile by gfx950's transposing LDS read
// (ds_read_b64_tr_b16: in each group of 16 lanes, lane i receives element
// i mod 4 of the 4-element pieces addressed by lanes 4 e + i / 4, e = 0..3),
// so no transpose is stored. The fp32 output is stored as a bf16 pair
// hi + lo, the form in which the O projection reads it.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kDh = 128;
constexpr int kBQ = 128;      // queries per block
constexpr int kBK = 64;       // keys per tile
constexpr int kTileBytes = kBK * kDh * 2;  // one K or V tile, 256-byte rows
constexpr int kStageBytes = 2 * kTileBytes;  // K then V
constexpr int kRingBytes = 2 * kStageBytes;  // two stages per wave group
// Block kinds: 4 waves on one head; 8 waves whose two groups split one
// head's key tiles (KSPLIT); 8 waves whose two groups are two query heads of
// one KV group sharing every K/V tile (HEADS2).
enum : int { kPlain = 0, kKsplit = 1, kHeads2 = 2 };
constexpr float kSlack = 8.f;  // lazy-rescale threshold, log2 units
constexpr int kCUs = 256;

typedef float f32v2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16v2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
constexpr bf16v2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
typedef const void __attribute__((address_space(1)))* gptr_t;
typedef void __attribute__((address_space(3)))* lptr_t;
typedef s16x4 __attribute__((address_space(3)))* lptr4_t;

QL_DEV int kswz(int r) { return r & 15; }        // K chunk position = c ^ kswz(row)
QL_DEV int vswz(int r) { return 4 * (r & 3); }   // V chunk position = c ^ vswz(row)

// 16 bytes from global memory straight into LDS: lane i of the wave writes
// lds_wave_base + 16 i (the base is wave-uniform)
QL_DEV void load_lds16(const bf16* g, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((gptr_t)g, (lptr_t)lds_wave_base, 16, 0, 0);
}

// Two 4-wave blocks per CU (one 64 KiB ring each), or one 8-wave block
// (KSPLIT: two rings; HEADS2: one shared ring of four stages): the register
// budget of two waves per SIMD keeps every accumulator in VGPRs, and one
// wave's MFMAs run while the other works through its softmax. HEADS2 halves
// the K/V bytes each CU moves per unit of work (the direct loads cost about
// a quarter of the kernel's time when two 4-wave blocks each fetch their own
// copy) and keeps three tiles in flight instead of one.
template <int VAR>
__global__ __launch_bounds__(VAR != kPlain ? 512 : 256, VAR != kPlain ? 1 : 2) void attn_prefill_kernel(
    const AttnPrefillArgs p) {
  constexpr bool KSPLIT = VAR == kKsplit;
  constexpr bool HEADS2 = VAR == kHeads2;
  constexpr int NG = KSPLIT ? 2 : 1;      // rings
  constexpr int NS = HEADS2 ? 4 : 2;      // stages per ring
  constexpr int kRing = NS * kStageBytes;
  constexpr int LW = HEADS2 ? 8 : 4;      // waves sharing a ring's loads
  constexpr int NLW = 16 / LW;            // 1 KiB loads per wave per K (or V) tile
  constexpr int kMpl = 16 / (2 * NLW);    // score MFMAs per interleaved load
  // [ring][stage][K | V], then (KSPLIT) group 1's running max and sum for
  // the merge, per wave and lane; the output staging (64 rows of 256 bytes
  // per storing wave) reuses the space. One LDS object: with a second one
  // the compiler no longer tells the tile reads from the in-flight direct
  // loads and waits for those loads before every fragment read.
  constexpr int kMlBytes = KSPLIT ? 4 * 2 * 64 * 4 : 0;
  constexpr int kStage = HEADS2 ? 8 * 64 * 256 : 0;
  constexpr int kLds = NG * kRing + kMlBytes > kStage ? NG * kRing + kMlBytes : kStage;
  static_assert(kLds <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) char lds[kLds];
  const int lane = threadIdx.x & 63;
  const int grp = VAR != kPlain ? (int)(threadIdx.x >> 8) : 0;  // key half, or head of the pair
  const int tid = threadIdx.x & 255;                     // thread within the group
  const int wave = tid >> 6;          // query rows 32 wave .. +31 of the tile
  const int lw = HEADS2 ? (int)(threadIdx.x >> 6) : wave;  // the wave's share of the loads
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
  const int h = HEADS2 ? 2 * ((wi / p.gx) % p.gy) + grp : (wi / p.gx) % p.gy;
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
  char* ring = lds + (KSPLIT ? grp * kRing : 0);

  // Load j (0 .. NLW-1) of load wave w fills LDS chunks 64 (LW j + w) + lane
  // of the K (then the V) tile: row 4 (LW j + w) + lane / 16, chunk position
  // lane % 16, which holds chunk (lane % 16) ^ f(row) of that key row. Rows
  // at or past the sequence's end read its last row instead (an in-bounds
  // address; K rows there are masked in the scores, V rows meet a zero
  // weight).
  // The lane's key row and byte position in the row are fixed per load j;
  // per tile a load adds the key row's offset (a 24-bit multiply, the cache
  // of one sequence being far below 4 GiB) to the block's K or V base, so the
  // load takes a scalar base and a 32-bit vector offset.
  const int lw_s = __builtin_amdgcn_readfirstlane(lw);
  const int lpos = lane & 15;
  const uint32_t row_bytes = (uint32_t)p.n_kv_heads * kDh * 2;
  int lrow_j[NLW];
  uint32_t kpos_j[NLW], vpos_j[NLW];
#pragma unroll
  for (int j = 0; j < NLW; ++j) {
    lrow_j[j] = 4 * (LW * j + lw) + (lane >> 4);
    kpos_j[j] = 16 * (lpos ^ kswz(lrow_j[j]));
    vpos_j[j] = 16 * (lpos ^ vswz(lrow_j[j]));
  }
  const char* kb8 = reinterpret_cast<const char*>(kbase);
  const char* vb8 = reinterpret_cast<const char*>(vbase);
  auto gload1 = [&](int kt, int st, int idx) {  // idx < NLW: K, else V
    const int j = idx % NLW;
    const int key = min(kt * kBK + lrow_j[j], L - 1);
    const uint32_t off = __umul24((uint32_t)key, row_bytes) + (idx < NLW ? kpos_j[j] : vpos_j[j]);
    char* dst = ring + st * kStageBytes + (idx >= NLW ? kTileBytes : 0) + (LW * j + lw_s) * 1024;
    load_lds16(reinterpret_cast<const bf16*>((idx < NLW ? kb8 : vb8) + off), dst);
  };
  auto gload = [&](int kt, int st) {
#pragma unroll
    for (int idx = 0; idx < 2 * NLW; ++idx) gload1(kt, st, idx);
  };
  // V^T fragment addresses (see the transposing read above): for keys
  // kb + 4 (lane / 32) + 0..3 (and + 8) of dh rows 32 dt + lane % 32, lane
  // s supplies key row kb + 4 (s / 32) + (s % 16) / 4, dh column
  // 32 dt + 16 ((s / 16) % 2) + 4 (s % 4)
  const int vtr_row = 4 * (lane >> 5) + ((lane & 15) >> 2);  // + kb
  const int vtr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // + 32 dt
  auto vtr_addr = [&](const char* Vs, int row, int dcol) {
    const int c = dcol >> 3;
    return Vs + row * 256 + ((c ^ vswz(row)) << 4) + ((dcol & 7) << 1);
  };

  f32x16 acc_o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[dt][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  // the first NS - 1 tiles (a tile past the range re-reads the last one,
  // unused, so the vector-memory count per tile stays fixed)
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (kt_lo < kt_hi) gload(min(kt_lo + j, kt_hi - 1), j);
  // This wave's first tile and Q fragments have landed (and, after the
  // barrier, every wave's); only the later tiles' loads may remain. Waiting
  // on every path into the key loop also keeps the compiler from waiting on
  // the vector-memory counter before the first score MFMAs, which would wait
  // for the next tiles' loads too.
  if constexpr (NS == 2)
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // vmcnt(0) only
  else
    __builtin_amdgcn_s_waitcnt(((NS - 2) * 2 * NLW) | (0x7 << 4) | (0xF << 8));
  __syncthreads();

  for (int it = 0; it < niter; ++it) {
    const int kt = kt_lo + it;
    const int st = it % NS;
    // the prefetch of tile kt + NS - 1 into the slot tile kt - 1 used (a
    // tile past the range re-reads the last one, unused, so the loads need
    // no branch and can sit among the score MFMAs)
    const int ktn = max(min(kt + NS - 1, kt_hi - 1), 0);
    const int stn = (it + NS - 1) % NS;
    const int k0 = kt * kBK;
    // skip tiles past the group's range (its last step when it has one tile
    // fewer) and tiles whose every key is in this wave's future (wave-uniform)
    if (__builtin_amdgcn_readfirstlane(kt < kt_hi && k0 <= wave_qmax)) {
      const char* Ks = ring + st * kStageBytes;
      const char* Vs = Ks + kTileBytes;
      f32x16 sc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[t][r] = 0.f;
        const int krow = 32 * t + col;
        const char* kr = Ks + krow * 256;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const bf16x8 kf =
              *reinterpret_cast<const bf16x8*>(kr + (((2 * s + hi) ^ kswz(krow)) << 4));
          sc[t] = mfma_32x32x16(kf, qf[s], sc[t]);
          if (s % kMpl == kMpl - 1) gload1(ktn, stn, (8 / kMpl) * t + s / kMpl);
        }
      }
      // issue order: per kMpl score MFMAs, their K-fragment reads, the MFMAs
      // and one 16-byte global load of a later tile, so the loads' issue
      // overlaps the matrix work instead of stalling the wave ahead of it
#pragma unroll
      for (int g8 = 0; g8 < 16 / kMpl; ++g8) {
        __builtin_amdgcn_sched_group_barrier(0x100, kMpl, 0);  // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, kMpl, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);     // global load
      }
      // mask, tile max (raw scores; the scale is positive and applied in the
      // exponent). Register r of half t holds key 32t + 8(r/4) + 4hi + r%4.
      // The mask test is wave-uniform (readfirstlane), so the common unmasked
      // tile carries no per-element code.
      const bool need_mask = __builtin_amdgcn_readfirstlane(
          (k0 + kBK - 1 > P + q0 + wave * 32) || (k0 + kBK > L));
      if (need_mask) {
        // keys past min(my_pos, L - 1), relative to this lane's first key:
        // one compare per score against a constant offset
        const int lim = min(my_pos, L - 1) - (k0 + 4 * hi);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sc[t][r] = 32 * t + 8 * (r >> 2) + (r & 3) > lim ? -INFINITY : sc[t][r];
      }
      float mt = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sc[t][r]);
      mt = xor32_max(mt) * p.scale_log2;
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
        const int kb = 32 * (u >> 1) + 16 * (u & 1);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lptr4_t)vtr_addr(Vs, kb + vtr_row, 32 * dt + vtr_col));
          const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lptr4_t)vtr_addr(Vs, kb + 8 + vtr_row, 32 * dt + vtr_col));
          const bf16x8 vf = __builtin_bit_cast(
              bf16x8, (s16x8){lo[0], lo[1], lo[2], lo[3], hi4[0], hi4[1], hi4[2], hi4[3]});
          acc_o[dt] = mfma_32x32x16(vf, pf[u], acc_o[dt]);
        }
      }
    } else {
      gload(ktn, stn);
    }
    // this wave's loads of the next tile have landed (only the NS - 2 tiles
    // after it may still be out); after the barrier every wave's have, and
    // every wave is done with this tile's slot
    if constexpr (NS == 2)
      __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // vmcnt(0) only
    else
      __builtin_amdgcn_s_waitcnt(((NS - 2) * 2 * NLW) | (0x7 << 4) | (0xF << 8));
    __syncthreads();
  }
  if constexpr (NS > 2) {
    // the last steps' unused re-reads land before the LDS is reused
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // vmcnt(0) only
    __syncthreads();
  }

  // merge: group 1 hands its state to group 0 through LDS (the rings are
  // free: every tile read ended before the loop's last barrier). A lane's
  // state is relative to its own reference maximum m_run; a group that saw
  // no key of this query has m_run = -inf and contributes nothing.
  static_assert(!KSPLIT || 4 * 64 * 64 * 4 <= kRing, "merge state fits group 0's ring");
  float* mst = reinterpret_cast<float*>(lds) + wave * (64 * 64) + lane;
  float* mls = reinterpret_cast<float*>(lds + NG * kRing) + wave * 128 + lane;
  if (KSPLIT && grp == 1) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mst[(16 * dt + r) * 64] = acc_o[dt][r];
    mls[0] = m_run;
    mls[64] = l_run;
  }
  if (KSPLIT) __syncthreads();
  if (KSPLIT && grp == 1) continue;  // (the next pass starts with a barrier)
  if (KSPLIT) {
    const float m1 = mls[0], l1 = mls[64];
    const float m = fmaxf(m_run, m1);  // finite: every query sees key 0
    const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m);
    const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
    l_run = a0 * l_run + a1 * l1;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[dt][r] = a0 * acc_o[dt][r] + a1 * mst[(16 * dt + r) * 64];
  }
  const float l_tot = xor32_sum(l_run);
  const float inv = 1.0f / l_tot;
  // The fp32 output as a bf16 pair: hi = RNE(o) at column c, lo = RNE(o - hi)
  // at column c + lo_off (the O projection multiplies both). A lane holds 16
  // pieces of 4 values of one query row, so the rows are staged through LDS
  // as [query][dh] (in the ring of group 1, or of the only group: every tile
  // read ended before the loop's last barrier) and stored as whole 256-byte
  // rows, 16 lanes to a row, rather than as 8-byte pieces of 32 rows. Rows
  // past the sequence (a ragged last tile) are computed and not stored.
  // staging: 64 rows (hi, then lo) of 256 bytes per wave, chunk c of row r
  // at position c ^ (r mod 16)
  static_assert(HEADS2 || 4 * 64 * 256 <= kRing, "output staging fits one ring");
  char* so = lds + (KSPLIT ? kRing : 0) + (HEADS2 ? (int)(threadIdx.x >> 6) : wave) * (64 * 256);
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
      const int pos = ((4 * dt + c) ^ kswz(col)) << 4;
      *reinterpret_cast<bf16x4*>(so + col * 256 + pos + 8 * hi) = vh;
      *reinterpret_cast<bf16x4*>(so + (32 + col) * 256 + pos + 8 * hi) = vl;
    }
  // (the wave's own LDS writes and reads run in order; the fences keep the
  // compiler from moving the reads above the writes)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  bf16x8 h8[8], l8[8];  // query rows 4 i + lane / 16, columns 8 (lane % 16) ..
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 4 * i + (lane >> 4);
    const int pos = ((lane & 15) ^ kswz(r)) << 4;
    h8[i] = *reinterpret_cast<const bf16x8*>(so + r * 256 + pos);
    l8[i] = *reinterpret_cast<const bf16x8*>(so + (32 + r) * 256 + pos);
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
  // key-row offsets within one sequence's cache are 32-bit (24-bit factors)
  if ((long long)a.T_max * a.n_kv_heads * kDh * 2 >= (1LL << 32) || a.T_max >= (1 << 24))
    return hipErrorInvalidValue;
  // (a.S: the longest sequence's new rows when seq_start is set)
  const int nqt = (a.S + kBQ - 1) / kBQ;
  const long pairs = (long)((nqt + 1) / 2) * a.n_q_heads * a.B;
  const long tiles = (long)nqt * a.n_q_heads * a.B;
  AttnPrefillArgs b = a;
  const int G = a.n_kv_heads > 0 ? a.n_q_heads / a.n_kv_heads : 0;
  if (pairs >= 2L * kCUs && G % 2 == 0) {
    // enough tile pairs (equal work each) for one 8-wave block per CU whose
    // two groups are two query heads of one KV group sharing each K/V tile
    b.pair = true;
    b.gx = (nqt + 1) / 2;
    b.gy = a.n_q_heads / 2;
    b.gtotal = b.gx * b.gy * a.B;
    hipLaunchKernelGGL(attn_prefill_kernel<kHeads2>, dim3(8 * ((b.gtotal + 7) / 8)), dim3(512), 0,
                       s, b);
  } else if (pairs >= 2L * kCUs) {
    // enough tile pairs (equal work each) for two 4-wave blocks per CU
    b.pair = true;
    b.gx = (nqt + 1) / 2;
    b.gy = a.n_q_heads;
    b.gtotal = b.gx * b.gy * a.B;
    hipLaunchKernelGGL(attn_prefill_kernel<kPlain>, dim3(8 * ((b.gtotal + 7) / 8)), dim3(256), 0,
                       s, b);
  } else if (pairs >= kCUs || tiles <= kCUs) {
    // one 8-wave block per CU, each tile's keys split between its two groups:
    // tile pairs when they fill the CUs, else single tiles
    b.pair = pairs >= kCUs;
    b.gx = b.pair ? (nqt + 1) / 2 : nqt;
    b.gy = a.n_q_heads;
    b.gtotal = b.gx * b.gy * a.B;
    hipLaunchKernelGGL(attn_prefill_kernel<kKsplit>, dim3(8 * ((b.gtotal + 7) / 8)), dim3(512), 0,
                       s, b);
  } else {
    // single tiles, longest first, two 4-wave blocks per CU
    b.pair = false;
    b.gx = nqt;
    b.gy = a.n_q_heads;
    b.gtotal = b.gx * b.gy * a.B;
    hipLaunchKernelGGL(attn_prefill_kernel<kPlain>, dim3(8 * ((b.gtotal + 7) / 8)), dim3(256), 0,
                       s, b);
  }
  return hipGetLastError();
}

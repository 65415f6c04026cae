// Large-tile bf16 GEMMs on MFMA for the projections, C = A * B^T.
//
// A is [M, Ka] (token rows), B is [N, Kb] (a weight in the [out, in] storage
// convention of "Qwen2.5-7B 结构拆解" §03.1); both K-contiguous. Token rows never
// interact in a projection (§03.2 of the same page), so M = B*S rows form one
// GEMM. A plain bf16 A has Ka = Kb; an fp32 activation arrives as a bf16 pair
// [hi | lo] (hi = RNE(a), lo = RNE(a - hi), row pitch 2 Kb), and the tile sums
// hi*W + lo*W, keeping the activation to about 16 significant bits.
//
// Design (gfx950, wave64), prefill tiles (gemm2_kernel, four kinds, see there):
// * 8 waves on a 256-column weight tile, 32x32x16 MFMAs with fp32 accumulators;
//   256 token rows (plain A, or a pair whose 32-deep stages hold the hi, lo and
//   weight rows together) or 128 token rows of a pair.
// * global -> LDS directly (global_load_lds_dwordx4: 16 B per lane, lane i
//   writes 16 i bytes past a wave-uniform LDS base); each load instruction
//   moves whole 128-byte (or 64-byte) row pieces. A ring of two or three
//   stages: the next stages are requested while one is multiplied.
// * LDS chunks XOR-swizzled by row so fragment reads are free of bank
//   conflicts. A direct load cannot scatter, so each lane picks the global
//   chunk that belongs at its fixed LDS slot.
// * split-K over work items when the tile grid alone is too small for the
//   chip: each split writes an fp32 partial tile and a second kernel sums the
//   partials and applies the epilogue; a host plan picks the tile kind, the
//   split count and an optional split-K tail launch.
// * epilogue through LDS, half a tile at a time (the ring is reused): every
//   thread then handles 8 consecutive columns of one row, so stores are
//   16/32-byte contiguous and SwiGLU can pair a gate column with its up column.
// Decode tiles (gemm2_dec_kernel): 4 waves, an A tile of the batch's rows, a
// 3-4 slot ring of weight stages, work cut stream-K over 256 blocks with fp32
// partials summed by the reduce kernel.
//
// Epilogues (one rounding at the stored tensor):
//   BIAS      Q/K/V projection: + bias, QK-norm, RoPE; q -> q_out, k/v -> cache
//   RESID_F32 out_f32 = resid_bf16 + acc        R = X + O W_O^T
//   RESID_OUT out     = bf16(resid_f32 + acc)   Y = R + H W_down^T
//   SWIGLU    h = SiLU(g) * u (bf16, or a [hi | lo] pair)  B tile = [128 W_gate rows | 128 W_up rows]
//   MOE_GU    SWIGLU on gathered token rows with one expert's weights per tile
//   MOE_DOWN  out     = fp32 (or bf16) acc for one expert's slot rows
//   GATED_F32 out_f32 = resid + sigmoid(gate_logit[row]) * acc  (a shared
//             expert scaled by its per-token gate; resid fp32, bf16 or none)
// With split-K each split stores its fp32 partial tile and the reduce kernel
// applies the epilogue.
// ("推理系统 03：逐项算清一个真实 Qwen3 Transformer 层" §4, §9, §10.)
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace {

enum : int { G2_BIAS = 0, G2_RESID_F32, G2_RESID_OUT, G2_SWIGLU, G2_MOE_GU, G2_MOE_DOWN,
             G2_GATED_F32 };

constexpr int BN = 256, BK = 64;  // weight-tile columns, k depth of a stage
constexpr int kGroupM = 4;  // tile rows per L2 group
constexpr int kRowChunks = BK / 8;                     // 16-byte chunks per LDS row
constexpr int kPitch = BN + 4;                         // fp32 epilogue tile pitch
constexpr int kEpiBytes = 128 * kPitch * 4;            // 128 rows of the output tile

struct G2Args {
  const bf16* A;
  int lda, M, Ka;
  const bf16* B;
  const bf16* B2;  // BIAS: rows [seg1, seg2) come from B2, [seg2, N) from B3; SWIGLU: up
  const bf16* B3;
  int seg1, seg2;
  int ldb, Kb;
  int tiles_m, tiles_n, splits, ksteps_per_split;
  int tn_base;  // first weight column tile of this launch (its tiles_n tiles follow)
  float* out_f32;
  bf16* out_bf16;
  int ldo;
  int out_lo;  // SWIGLU: > 0 stores h as a [hi | lo] pair, lo at + out_lo elements
  const float* gate_logit;  // GATED_F32: the row's gate logit at gate_logit[row * gate_ld]
  int gate_ld;
  const bf16* bias;
  const bf16* bias2;
  const bf16* bias3;
  const bf16* resid_bf16;
  const float* resid_f32;
  int ldr;
  float* part;  // [splits][M][tiles_n * BN]
  // stream-K (decode tiles): the tile-major (tile, k step) units are cut into
  // sk_grid contiguous runs, one per block; partial index = ordinal of the
  // block among those touching the tile
  int streamk, sk_grid, rows_per_tile;
  // BIAS (the QKV projection): per-head QK-norm, RoPE and the cache write
  // fused into the epilogue
  int S, pos_offset, T_max, n_q_heads, n_kv_heads;
  const int* cache_len;  // decode: row b is sequence b at cache row cache_len[b]
  const int* seq_start;  // varlen prefill: [nseq + 1] first row of each sequence
  const int* prefix;     // varlen prefill: [nseq] cache rows before each sequence's new ones
  int nseq;
  float eps;
  const double* omega;  // [64] RoPE frequencies
  const bf16* q_norm_g;
  const bf16* k_norm_g;
  bf16* q_out;          // [M, Hq*128]
  bf16* k_cache;        // [B, T_max, Hkv, 128]
  bf16* v_cache;
  // MoE expert tiles: tile i covers slot rows [tile_row0[i], + tile_rows[i])
  // of expert tile_expert[i]; *num_tiles tiles exist. MOE_GU gathers A row
  // row_index[slot]; expert e's weights start e * b_expert_stride elements in.
  const int* row_index;
  const int* tile_expert;
  const int* tile_row0;
  const int* tile_rows;
  const int* num_tiles;
  size_t b_expert_stride;
};

// The value of the lane 8 places away within its row of 16 lanes (lane
// i ^ 8): a DPP row rotate by 8, no LDS round trip. Both lanes of a pair
// are active together wherever it is used.
QL_DEV float xor8_lane(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
}

// QKV epilogue for 8 columns [col, col + 8) of token row `row`, bias added.
// The 16 lanes of an aligned lane group hold one head (128 columns), so the
// per-head sum of squares of QK-norm is a 16-lane reduction and the RoPE
// partner of column i (i + 64) sits 8 lanes away. q goes to q_out; k and v go
// to cache row (row % S) of sequence row / S (prefill), or to cache row
// cache_len[row] of sequence row (decode; nothing is written to the cache
// when that length is outside [0, T_max)). ("推理系统 03：逐项算清一个真实 Qwen3
// Transformer 层" §5 QK-norm, §6 rotate_half RoPE with omega_i = theta^(-2i/dh),
// §12 the cache keeps post-norm, post-RoPE keys.)
template <bool DEC>
QL_DEV void qkv_finish(const G2Args& p, size_t row, int col, float (&v)[8]) {
  const int qd = p.n_q_heads * 128, kvd = p.n_kv_heads * 128;
  int part = 0, c = col;
  if (col >= qd + kvd) {
    part = 2;
    c = col - qd - kvd;
  } else if (col >= qd) {
    part = 1;
    c = col - qd;
  }
  const int head = c >> 7, d0 = c & 127;
  int b, t;  // sequence, cache row
  if constexpr (DEC) {
    b = (int)row;
    t = p.cache_len[b];
  } else if (p.seq_start) {
    // varlen: the last sequence starting at or before the row
    int lo = 0, hi = p.nseq - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.seq_start[mid] <= (int)row) lo = mid;
      else hi = mid - 1;
    }
    b = lo;
    t = (int)row - p.seq_start[b] + (p.prefix ? p.prefix[b] : 0);
  } else {
    b = (int)(row / p.S);
    t = (int)(row % p.S);
  }
  if (part < 2) {
    const bf16* gam = part == 0 ? p.q_norm_g : p.k_norm_g;
    if (gam) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
      ss = row16_sum(ss);
      const float inv = __builtin_amdgcn_rsqf(ss / 128.f + p.eps);
      float g[8];
      unpack8(load_bf16x8(gam + d0), g);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = g[e] * (v[e] * inv);
    }
    // rotate_half partner of column d0 + e: column d0 + e +- 64, held by the
    // lane 8 places away in the head's 16-lane group
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = xor8_lane(v[e]);
    // Columns d0 + e and d0 + e + 64 turn by the same angle pos * omega_i,
    // i = (d0 + e) mod 64, so the two partner lanes each take four of the
    // eight angles and swap the results. An angle is taken in turns, reduced
    // to [-1/2, 1/2] in fp64 (pos may be large), and the hardware sine and
    // cosine of that fraction of a turn are used: their error, ~1e-6, is far
    // below the bf16 rounding of q and k (a full-precision sincosf per
    // element dominated the epilogue of a 256-row tile).
    const double pos = (double)t + (double)p.pos_offset;
    constexpr double kInvTwoPi = 0.15915494309189533576888376337251;
    const bool upper = d0 >= 64;
    float sn_own[4], cs_own[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = upper ? i + 4 : i;
      double turns = pos * (p.omega[(d0 + e) & 63] * kInvTwoPi);
      turns -= rint(turns);
      const float r = (float)turns;
      sn_own[i] = __builtin_amdgcn_sinf(r);
      cs_own[i] = __builtin_amdgcn_cosf(r);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float sn_p = xor8_lane(sn_own[i]), cs_p = xor8_lane(cs_own[i]);
      const float sn_a = upper ? sn_p : sn_own[i], cs_a = upper ? cs_p : cs_own[i];  // e = i
      const float sn_b = upper ? sn_own[i] : sn_p, cs_b = upper ? cs_own[i] : cs_p;  // e = i + 4
      v[i] = upper ? v[i] * cs_a + o[i] * sn_a : v[i] * cs_a - o[i] * sn_a;
      v[i + 4] = upper ? v[i + 4] * cs_b + o[i + 4] * sn_b : v[i + 4] * cs_b - o[i + 4] * sn_b;
    }
  }
  if (part == 0) {
    store_bf16x8(p.q_out + row * qd + c, pack8(v));
  } else if (!DEC || (t >= 0 && t < p.T_max)) {
    bf16* cache = part == 1 ? p.k_cache : p.v_cache;
    store_bf16x8(cache + (((size_t)b * p.T_max + t) * p.n_kv_heads + head) * 128 + d0, pack8(v));
  }
}

// GATED_F32 epilogue of 8 columns: v = resid + sigmoid(gate) * v.
QL_DEV void gated_finish(const G2Args& p, size_t row, int col, float (&v)[8]) {
  const float g = 1.0f / (1.0f + __expf(-p.gate_logit[row * p.gate_ld]));
  float r8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (p.resid_f32) {
    const float* rr = p.resid_f32 + row * p.ldr + col;
    const f32x4 r0 = *reinterpret_cast<const f32x4*>(rr);
    const f32x4 r1 = *reinterpret_cast<const f32x4*>(rr + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r8[e] = r0[e];
      r8[e + 4] = r1[e];
    }
  } else if (p.resid_bf16) {
    unpack8(load_bf16x8(p.resid_bf16 + row * p.ldr + col), r8);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = r8[e] + g * v[e];
}

// SwiGLU hidden values of columns [col, col + 8) of `row`: bf16, or the
// [hi | lo] pair (hi = RNE(h), lo = RNE(h - hi)) that keeps h to about 16
// significant bits for the down projection.
QL_DEV void store_h(const G2Args& p, size_t row, int col, const float (&h)[8]) {
  bf16* o = p.out_bf16 + row * p.ldo + col;
  const bf16x8 hi = pack8(h);
  store_bf16x8(o, hi);
  if (p.out_lo > 0) {
    float lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) lo[e] = h[e] - (float)hi[e];
    store_bf16x8(o + p.out_lo, pack8(lo));
  }
}

// Block that owns unit u when U units are cut into G contiguous runs
// [floor(b U / G), floor((b + 1) U / G)).
QL_HD int sk_owner(long long u, long long U, int G) { return (int)(((u + 1) * G - 1) / U); }

// LDS slot of chunk c of row r is c ^ swz(r). A 16-byte read by the lanes of
// one MFMA fragment touches 16 consecutive rows (from a multiple of 16) at one
// chunk; with 128-byte rows this puts them on 16 distinct 16-byte positions of
// a 256-byte bank line, so the read is free of bank conflicts.
QL_DEV int swz(int r) { return (r >> 1) & 7; }
// The same for 64-byte rows (4 chunks): rows r and r + 4 share a 64-byte
// position of the bank line, so the chunk order turns with r / 4.
template <int RC>
QL_DEV int swz_rc(int r) {
  static_assert(RC == 8 || RC == 4, "row chunks");
  return RC == 8 ? swz(r) : (r >> 2) & 3;
}

// Typed address-space casts for the direct-to-LDS load builtin.
typedef const void __attribute__((address_space(1)))* gptr_t;
typedef void __attribute__((address_space(3)))* lptr_t;

QL_DEV void load_lds16(const bf16* g, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((gptr_t)g, (lptr_t)lds_wave_base, 16, 0, 0);
}
// The same with the non-temporal hint (cache-policy bit nt), for weights that
// a decode call reads once: the stream then leaves the activation rows, which
// every block re-reads, in the caches.
QL_DEV void load_lds16_nt(const bf16* g, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((gptr_t)g, (lptr_t)lds_wave_base, 16, 0, 2);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
QL_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Prefill tiles. PART: write this split's fp32 partial tile instead of
// MODE's epilogue. KIND selects the tile:
//  0  256 token rows, A plain bf16 (or a pair over the doubled K); 8 waves as
//     2 (rows) x 4 (columns), a wave owns 128 x 64; two 64-deep ring stages
//     (2 x 64 KiB).
//  1  [hi | lo] pair, 128 token rows: LDS rows 0..127 hold the hi halves,
//     128..255 the lo halves at the same k, so each B tile serves both and the
//     k loop runs over Kb only; the lo accumulators (waves wm = 1) are added to
//     the hi ones through LDS in the epilogue. Same MFMA work as the doubled K,
//     twice the tiles at half the k steps.
//  2  [hi | lo] pair, 256 token rows: a stage holds 32 k of the 256 hi rows,
//     of the 256 lo rows and of the 256 weight rows (48 KiB), so each weight
//     fragment feeds a hi and a lo MFMA into the same accumulators; three ring
//     stages (two in flight while one is multiplied). 8 waves as 4 x 2, a wave
//     owns 64 token rows x 128 columns: per 16-deep step it reads 8 fragments
//     for 16 MFMAs (kind 0 reads 6 for 8), and the block moves 48 KiB from L2
//     per 256 x 256 x 64 of MFMA work instead of 64.
//  3  [hi | lo] pair, 128 token rows, for the MoE expert projections: a
//     stage holds 32 k of the 128 hi, 128 lo and 256 weight rows (32 KiB);
//     two ring slots and 64-row epilogue passes keep the block at 65 KiB of
//     LDS and 128 registers, so two blocks share a CU and one block's
//     prologue, epilogue and barrier waits overlap the other's MFMAs (expert
//     tiles are many and short). 8 waves as 2 x 4, a wave owns 64 token rows
//     x 64 columns.
// Kinds 0-2: two waves share each SIMD, so one wave's MFMAs run while the
// other waits; kind 3: four.
template <int MODE, bool PART, int KIND>
__global__ __launch_bounds__(512, KIND == 3 ? 4 : 1) void gemm2_kernel(const G2Args p) {
  constexpr bool HL = KIND == 1;
  constexpr bool K3 = KIND == 3;
  constexpr bool P2 = KIND == 2 || K3;  // pair stages: hi, lo and weight rows together
  constexpr int BMT = 256;
  constexpr int RT = HL || K3 ? BMT / 2 : BMT;  // token rows per tile
  constexpr int NW = BMT / 32;          // waves
  constexpr int NT = NW * 64;           // threads
  constexpr int WMW = K3 ? 2 : (P2 ? 4 : BMT / 128);  // waves along M
  constexpr int WNW = NW / WMW;         // waves along N
  constexpr int WROWS = P2 ? 64 : 128;  // LDS A rows per wave (per half for P2)
  constexpr int WCOLS = BN / WNW;       // columns per wave
  constexpr int TI = WROWS / 32;        // 32-row MFMA tiles per wave along M
  constexpr int TJ = WCOLS / 32;        // 32-wide MFMA tiles per wave along N
  constexpr int SBK = P2 ? 32 : BK;     // k depth of a stage
  constexpr int RC = SBK / 8;           // 16-byte chunks per LDS row
  constexpr int AROWS = P2 ? 2 * RT : BMT;  // LDS rows of A per stage
  constexpr int AC = AROWS * RC;        // A chunks per stage
  constexpr int CH = AC + BN * RC;
  constexpr int LPT = CH / NT;          // direct loads per thread per stage
  constexpr int LPA = AC / NT;          // ... of which A
  constexpr int SB = CH * 16;           // stage bytes
  constexpr int NS = KIND == 2 ? 3 : 2;  // ring stages
  constexpr int kEpiRows = K3 ? 64 : 128;  // output rows per epilogue pass
  constexpr int kEpiB = kEpiRows * kPitch * 4;
  constexpr int kLds = NS * SB > kEpiB ? NS * SB : kEpiB;
  constexpr bool kDual = MODE == G2_SWIGLU || MODE == G2_MOE_GU;
  constexpr bool kMoe = MODE == G2_MOE_GU || MODE == G2_MOE_DOWN;
  static_assert(CH % NT == 0 && AC % NT == 0, "whole loads per thread");
  static_assert(kLds <= 160 * 1024, "LDS");
  static_assert(!kMoe || !PART, "expert tiles run whole");
  __shared__ __attribute__((aligned(1024))) char smem[kLds];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform, so the direct loads' LDS addresses (M0) come from scalar
  // arithmetic instead of a vector add and a lane read per load
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WNW, wn = wave % WNW;

  const int nks_all = p.Ka / BK;
  int split = 0, tm = 0, tn = 0, ks0 = 0, nk = 0;
  int m0, rows_valid;
  size_t eoff = 0;  // expert weight offset
  if constexpr (kMoe) {
    // The grid covers the most tiles routing can produce; the tile count is
    // known on the device only. Work item w = tile * tiles_n + tn, split into
    // 8 contiguous stretches by XCD as below, so the column tiles of an
    // expert tile, and the tiles of one expert, run close together on one
    // XCD and share A and B through its L2.
    const int total = *p.num_tiles * p.tiles_n;
    const int chunk = (total + 7) / 8;
    if ((int)(blockIdx.x / 8) >= chunk) return;
    const int w = (int)(blockIdx.x % 8) * chunk + (int)(blockIdx.x / 8);
    if (w >= total) return;
    const int ti = w / p.tiles_n;
    tn = w % p.tiles_n;
    m0 = p.tile_row0[ti];
    rows_valid = p.tile_rows[ti];
    eoff = (size_t)p.tile_expert[ti] * p.b_expert_stride;
    nk = nks_all;
  } else {
    // XCD-aware tile order. Consecutive block ids go to the 8 XCDs
    // round-robin, each XCD with its own L2; so block b works on item
    // (b % 8) * chunk + b / 8 of the work list, and every XCD walks a
    // contiguous stretch of it. The list orders (split, tile) split-major,
    // tiles in groups of kGroupM tile rows x all tile columns, column-major
    // inside a group: the blocks an XCD runs at once share a few A and B
    // tiles, which its L2 then serves.
    const int ntiles = p.tiles_m * p.tiles_n;
    const int total = ntiles * p.splits;
    const int chunk = (total + 7) / 8;
    const int w = (int)(blockIdx.x % 8) * chunk + (int)(blockIdx.x / 8);
    if (w >= total) return;
    split = w / ntiles;
    const int pid = w % ntiles;
    const int group = pid / (kGroupM * p.tiles_n);
    const int first_m = group * kGroupM;
    const int gsize = min(p.tiles_m - first_m, kGroupM);
    const int in_group = pid % (kGroupM * p.tiles_n);
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
    ks0 = split * p.ksteps_per_split;
    nk = min(p.ksteps_per_split, nks_all - ks0);
    m0 = tm * RT;
    rows_valid = min(RT, p.M - m0);
  }
  const int n0 = (tn + p.tn_base) * (kDual ? BN / 2 : BN);  // first output column of the tile

  // QKV: a 256-column tile lies inside one of the three weight matrices
  const bf16* Bw = p.B + eoff;
  const bf16* bias = p.bias;
  int nb = n0;
  if constexpr (MODE == G2_BIAS) {
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

  // Direct-load plan: per stage the block fills CH 16-byte LDS chunks (A
  // first, then B); load j of wave w covers chunks (NW j + w) * 64 + lane, i.e.
  // 8 whole 128-byte rows, each one full cache line of A or B.
  const bf16* src[LPT];
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int P = (NW * j + wave) * 64 + lane;
    const bool is_a = j < LPA;
    const int Q = is_a ? P : P - AC;
    const int row = Q / RC;
    const int c = (Q % RC) ^ swz_rc<RC>(row);
    if (is_a) {
      // rows past the tile re-read a valid row; pairs: rows RT.. are the lo halves
      const bool lo = (HL || P2) && row >= RT;
      const int rr = min(lo ? row - RT : row, rows_valid - 1);
      const size_t ar = MODE == G2_MOE_GU ? (size_t)p.row_index[m0 + rr] : (size_t)(m0 + rr);
      src[j] = p.A + ar * p.lda + (lo ? p.Kb : 0) + c * 8;
    } else {
      const bf16* base;
      if constexpr (kDual) {
        base = row < BN / 2 ? Bw + (size_t)(n0 + row) * p.ldb
                            : p.B2 + eoff + (size_t)(n0 + row - BN / 2) * p.ldb;
      } else {
        base = Bw + (size_t)(nb + row) * p.ldb;
      }
      src[j] = base + c * 8;
    }
  }

  auto issue = [&](int kt) {  // stage kt of this split -> ring slot kt % NS
    const int ka = (ks0 + kt) * SBK;
    int kb = ka;
    if (!P2 && kb >= p.Kb) kb -= p.Kb;  // [hi | lo] A over the doubled K: B is read twice
    char* slot = smem + (kt % NS) * SB;
#pragma unroll
    for (int j = 0; j < LPT; ++j)
      load_lds16(src[j] + (j < LPA ? ka : kb), slot + (NW * j + wave) * 1024);
  };

  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // fragment read offsets (bytes within a stage) for k16 step ks; P2: the lo
  // row of a hi row sits RT LDS rows further
  const int fr = lane & 31;
  const int fk = lane >> 5;
  constexpr int KS = SBK / 16;  // 16-deep MFMA steps per stage
  int aoff[KS][TI], boff[KS][TJ];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int c = 2 * ks + fk;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int ra = wm * WROWS + 32 * i + fr;
      aoff[ks][i] = (ra * RC + (c ^ swz_rc<RC>(ra))) * 16;
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int rb = wn * WCOLS + 32 * j + fr;
      boff[ks][j] = AC * 16 + (rb * RC + (c ^ swz_rc<RC>(rb))) * 16;
    }
  }
  static_assert(!P2 || (RT % 16 == 0 && ((RT >> 2) & 3) == 0), "lo rows keep the hi rows' swizzle");
  constexpr int kLoOff = RT * RC * 16;  // P2: bytes from a hi row to its lo row

  // One stage: the fragments of k steps (0, 1) are read, then those of (2, 3)
  // are requested before the MFMAs of (0, 1) run, so only the first reads of
  // a stage sit in front of its MFMAs. Expert tiles are often part-filled:
  // their 32-row MFMA tiles made only of padding rows are skipped, the MFMAs
  // only (the fragment reads stay unconditional: reads inside the branches
  // made the compiler wait for them before every pair of MFMAs; the padding
  // rows hold copies of a valid row).
  bool act[TI];
  {
    const int wmu = __builtin_amdgcn_readfirstlane(wm);
#pragma unroll
    for (int i = 0; i < TI; ++i) act[i] = !kMoe || (wmu * WROWS + 32 * i) % RT < rows_valid;
    (void)wmu;
  }
  if constexpr (!P2) {
    auto read2 = [&](const char* st, int kh, bf16x8 (&af)[2][TI], bf16x8 (&bfr)[2][TJ]) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int i = 0; i < TI; ++i) af[ks][i] = *reinterpret_cast<const bf16x8*>(st + aoff[kh + ks][i]);
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          bfr[ks][j] = *reinterpret_cast<const bf16x8*>(st + boff[kh + ks][j]);
      }
    };
    auto mma2 = [&](const bf16x8 (&af)[2][TI], const bf16x8 (&bfr)[2][TJ]) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < TI; ++i)
          if (act[i])
#pragma unroll
            for (int j = 0; j < TJ; ++j) acc[i][j] = mfma_32x32x16(af[ks][i], bfr[ks][j], acc[i][j]);
    };
    static_assert(KS == 4, "two halves of two k steps per stage");

    // Two stages; stage kt+1 is requested right after the barrier that
    // publishes stage kt and lands while stage kt is multiplied.
    if (nk > 0) issue(0);
    for (int kt = 0; kt < nk; ++kt) {
      wait_vmcnt<0>();  // this wave's part of stage kt (the only stage in flight)
      // every wave's part of stage kt has landed and every wave is done with
      // the other slot. A bare s_barrier: __syncthreads' release fence adds
      // nothing here; the acquire fence keeps the LDS reads below it.
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      if (kt + 1 < nk) issue(kt + 1);
      const char* st = smem + (kt % NS) * SB;
      bf16x8 a0[2][TI], b0[2][TJ], a1[2][TI], b1[2][TJ];
      read2(st, 0, a0, b0);
      __builtin_amdgcn_sched_barrier(0);
      read2(st, 2, a1, b1);
      __builtin_amdgcn_sched_barrier(0);
      mma2(a0, b0);
      __builtin_amdgcn_sched_barrier(0);
      mma2(a1, b1);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    static_assert(KS == 2 && NS == (K3 ? 2 : 3), "two k steps per stage, three ring slots (two in kind 3)");
    // one 16-deep step: hi and lo fragments of the wave's rows, weight fragments
    auto read1 = [&](const char* st, int ks, bf16x8 (&ah)[TI], bf16x8 (&al)[TI], bf16x8 (&bw)[TJ]) {
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        ah[i] = *reinterpret_cast<const bf16x8*>(st + aoff[ks][i]);
        al[i] = *reinterpret_cast<const bf16x8*>(st + aoff[ks][i] + kLoOff);
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) bw[j] = *reinterpret_cast<const bf16x8*>(st + boff[ks][j]);
    };
    // all hi products, then all lo products: eight independent MFMAs sit
    // between two that update the same accumulators
    auto mma1 = [&](const bf16x8 (&ah)[TI], const bf16x8 (&al)[TI], const bf16x8 (&bw)[TJ]) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
        if (act[i])
#pragma unroll
          for (int j = 0; j < TJ; ++j) acc[i][j] = mfma_32x32x16(ah[i], bw[j], acc[i][j]);
#pragma unroll
      for (int i = 0; i < TI; ++i)
        if (act[i])
#pragma unroll
          for (int j = 0; j < TJ; ++j) acc[i][j] = mfma_32x32x16(al[i], bw[j], acc[i][j]);
    };

    // Three slots: stages kt+1 and kt+2 are in flight while stage kt is
    // multiplied. Stage kt+2 goes to the slot stage kt-1 used, which every
    // wave has finished reading once it passes the barrier of stage kt.
    // Kind 3 (two blocks per CU): two slots, stage kt+1 in flight.
    if (nk > 0) issue(0);
    if (!K3 && nk > 1) issue(1);
    for (int kt = 0; kt < nk; ++kt) {
      // this wave's part of stage kt (loads complete in order: only stage
      // kt+1's may still be out)
      if (!K3 && kt + 1 < nk) wait_vmcnt<(K3 ? 0 : LPT)>();
      else wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      // the first step's fragment reads go out before the next stage's
      // loads, and the compiler may interleave the second step's reads with
      // the first step's MFMAs (Qwen3-8B 2048-token gate/up 724 -> 671 us)
      const char* st = smem + (kt % NS) * SB;
      bf16x8 h0[TI], l0[TI], w0[TJ], h1[TI], l1[TI], w1[TJ];
      read1(st, 0, h0, l0, w0);
      __builtin_amdgcn_sched_barrier(0);
      if (kt + NS - 1 < nk) issue(kt + NS - 1);
      __builtin_amdgcn_sched_barrier(0);
      read1(st, 1, h1, l1, w1);
      mma1(h0, l0, w0);
      __builtin_amdgcn_sched_barrier(0);
      mma1(h1, l1, w1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();  // the ring is reused for the epilogue

  // ---- epilogue: 128 rows (one row of waves) at a time through LDS ----
  float* C = reinterpret_cast<float*>(smem);
  constexpr int NH = HL ? 1 : RT / kEpiRows;  // epilogue passes
  constexpr int WPH = kEpiRows / WROWS;  // wave rows per pass
#pragma unroll
  for (int half = 0; half < NH; ++half) {
    // HL: the hi rows (wm 0) are stored, then the lo rows (wm 1) added on top
#pragma unroll
    for (int pass = 0; pass < (HL ? 2 : 1); ++pass) {
      if ((HL ? wm == pass : wm / WPH == half)) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = (wm % WPH) * WROWS + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
              float* dst = C + row * kPitch + wn * WCOLS + 32 * j + (lane & 31);
              *dst = (HL && pass == 1) ? *dst + acc[i][j][r] : acc[i][j][r];
            }
      }
      if (HL && pass == 0) __syncthreads();
    }
    __syncthreads();
    const int rbase = half * kEpiRows;
    if constexpr (PART) {
      const int ldp = p.tiles_n * BN;
      float* dst = p.part + (size_t)split * p.M * ldp;
      const int seg = tid & 31;
      for (int r = tid >> 5; r < kEpiRows; r += NT / 32) {
        if (rbase + r >= rows_valid) break;
        const float* c = C + r * kPitch + seg * 8;
        float* o = dst + (size_t)(m0 + rbase + r) * ldp + tn * BN + seg * 8;
        *reinterpret_cast<f32x4*>(o) = *reinterpret_cast<const f32x4*>(c);
        *reinterpret_cast<f32x4*>(o + 4) = *reinterpret_cast<const f32x4*>(c + 4);
      }
    } else if constexpr (kDual) {
      const int seg = tid & 15;
      for (int r = tid >> 4; r < kEpiRows; r += NT / 16) {
        if (rbase + r >= rows_valid) break;
        const float* g = C + r * kPitch + seg * 8;
        const float* u = g + BN / 2;
        float hv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) hv[e] = silu_f32(g[e]) * u[e];
        store_h(p, (size_t)(m0 + rbase + r), n0 + seg * 8, hv);
      }
    } else {
      const int seg = tid & 31;
      const int col = n0 + seg * 8;
      float badd[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) badd[e] = 0.f;
      if constexpr (MODE == G2_BIAS) {
        if (bias) unpack8(load_bf16x8(bias + nb + seg * 8), badd);
      }
      for (int r = tid >> 5; r < kEpiRows; r += NT / 32) {
        if (rbase + r >= rows_valid) break;
        const float* c = C + r * kPitch + seg * 8;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = c[e] + badd[e];
        const size_t row = (size_t)(m0 + rbase + r);
        if constexpr (MODE == G2_BIAS) {
          qkv_finish<false>(p, row, col, v);
          continue;
        }
        if constexpr (MODE == G2_RESID_F32) {
          float x[8];
          unpack8(load_bf16x8(p.resid_bf16 + row * p.ldr + col), x);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] += x[e];
        }
        if constexpr (MODE == G2_GATED_F32) gated_finish(p, row, col, v);
        if constexpr (MODE == G2_RESID_OUT) {
          const float* rr = p.resid_f32 + row * p.ldr + col;
          const f32x4 r0 = *reinterpret_cast<const f32x4*>(rr);
          const f32x4 r1 = *reinterpret_cast<const f32x4*>(rr + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] += r0[e];
            v[e + 4] += r1[e];
          }
          store_bf16x8(p.out_bf16 + row * p.ldo + col, pack8(v));
        } else if constexpr (MODE == G2_MOE_DOWN) {
          if (p.out_f32) {
            float* o = p.out_f32 + row * p.ldo + col;
            *reinterpret_cast<f32x4*>(o) = f32x4{v[0], v[1], v[2], v[3]};
            *reinterpret_cast<f32x4*>(o + 4) = f32x4{v[4], v[5], v[6], v[7]};
          } else {
            store_bf16x8(p.out_bf16 + row * p.ldo + col, pack8(v));
          }
        } else {  // RESID_F32, GATED_F32: fp32 rows
          float* o = p.out_f32 + row * p.ldo + col;
          *reinterpret_cast<f32x4*>(o) = f32x4{v[0], v[1], v[2], v[3]};
          *reinterpret_cast<f32x4*>(o + 4) = f32x4{v[4], v[5], v[6], v[7]};
        }
      }
    }
    __syncthreads();
  }
}

// Decode tiles: 4 waves as 1 x 4, each owning all RA LDS rows of A x 64
// columns. Few-row batches stream their weights from HBM, and covering HBM
// latency at full bandwidth takes about three 32 KiB weight stages in flight
// per CU; so the A tile holds only RA rows (the batch rounded up to 32, 64 or
// 128, [hi | lo] pairs counted twice) and the ring has four slots when RA <=
// 64 (three stages in flight while one is multiplied), three otherwise.
// HL: A is a [hi | lo] pair and the tile covers RA / 2 token rows; LDS rows
// below RA / 2 hold the hi halves and the rest the lo halves at the same k,
// so each B tile is fetched once and serves both, and each wave adds its lo
// accumulators to its hi ones. The k loop then runs over Kb only; the QKV
// epilogue takes the rows as sequences. In plain tiles, 32-row MFMA tiles
// made only of padding rows are multiplied too and never stored: the matrix
// cores are far from busy here, and a branch around them made the compiler
// move the accumulators between register files at every step (gate/up and
// down at 64 rows ran 13 % slower); hi/lo tiles skip them.
// Work is cut stream-K: the tile-major (tile, k step) units are split into
// gridDim.x contiguous runs, one per block. The ring runs on across the
// tiles of a run; each tile's fp32 partial goes out straight from the
// accumulators, at partial index = the block's ordinal among the blocks
// touching the tile, and the reduce kernel sums them. Stores count in the
// same vector-memory counter as the ring's loads, so a store in mid-run
// would hold up the next stage's wait: for a plain A with RA <= 64 (long
// gate/up and down runs) the first tile's accumulators are parked in a
// second register set and every partial is stored after the last stage (a
// run crossing more than one tile boundary stores the middle tiles as it
// leaves them); otherwise (short Q/K/V and O runs, or no room for two sets)
// each tile is stored as the run leaves it.
template <int MODE, bool HL, int RA>
__global__ __launch_bounds__(256, 1) void gemm2_dec_kernel(const G2Args p) {
  constexpr int NT = 256, WCOLS = 64, TJ = 2;
  constexpr int NI = RA / 32;           // 32-row MFMA tiles of A
  constexpr int AC = RA * kRowChunks;   // A chunks per stage
  constexpr int CH = AC + BN * kRowChunks;
  constexpr int LPT = CH / NT;          // direct loads per thread per stage
  constexpr int LPA = AC / NT;          // ... of which A
  constexpr int SB = CH * 16;           // stage bytes
  constexpr int NS = RA <= 64 ? 4 : 3;  // ring slots
  constexpr bool kDual = MODE == G2_SWIGLU;
  constexpr int RT = HL ? RA / 2 : RA;  // token rows per tile
  constexpr int NO = HL ? NI / 2 : NI;  // 32-row tiles stored
  static_assert(CH % NT == 0 && AC % NT == 0, "whole loads per thread");
  static_assert(NS * SB <= 160 * 1024, "LDS");
  static_assert(NS * LPT <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char smem[NS * SB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wn = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar M0 addresses)
  const int nks = p.Ka / BK;
  const int U = p.tiles_m * p.tiles_n * nks;
  const int u0 = __builtin_amdgcn_readfirstlane((int)((long long)blockIdx.x * U / p.sk_grid));
  const int total = __builtin_amdgcn_readfirstlane(
      (int)((long long)(blockIdx.x + 1) * U / p.sk_grid) - u0);
  const int ldp = p.tiles_n * BN;

  // issue side: load plan of the tile whose stages are being requested
  int itile = -1;
  const bf16* src[LPT];
  auto plan = [&](int t) {
    const int m0 = (t % p.tiles_m) * RT;
    const int rows_valid = min(RT, p.M - m0);
    const int n0 = (t / p.tiles_m) * (kDual ? BN / 2 : BN);
    const bf16* Bw = p.B;
    int nb = n0;
    if constexpr (MODE == G2_BIAS) {  // a 256-column tile lies inside one of Wq, Wk, Wv
      if (n0 >= p.seg2) {
        Bw = p.B3;
        nb = n0 - p.seg2;
      } else if (n0 >= p.seg1) {
        Bw = p.B2;
        nb = n0 - p.seg1;
      }
    }
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
      const int P = (4 * j + wn) * 64 + lane;
      const bool is_a = j < LPA;
      const int Q = is_a ? P : P - AC;
      const int row = Q / kRowChunks;
      const int c = (Q % kRowChunks) ^ swz(row);
      if (is_a) {
        // rows past the tile re-read a valid row; HL: rows RT.. are the lo halves
        const int rr = min(HL ? row % RT : row, rows_valid - 1);
        const int kofs = HL && row >= RT ? p.Kb : 0;
        src[j] = p.A + (size_t)(m0 + rr) * p.lda + kofs + c * 8;
      } else {
        const bf16* base;
        if constexpr (kDual) {
          base = row < BN / 2 ? p.B + (size_t)(n0 + row) * p.ldb
                              : p.B2 + (size_t)(n0 + row - BN / 2) * p.ldb;
        } else {
          base = Bw + (size_t)(nb + row) * p.ldb;
        }
        src[j] = base + c * 8;
      }
    }
  };
  // (integer division runs on the vector ALU; readfirstlane keeps the
  // block-uniform tile index scalar, so branches on it stay scalar)
  auto tile_of = [&](int uu) { return __builtin_amdgcn_readfirstlane(uu / nks); };
  auto issue = [&](int g) {  // stage g of the run -> ring slot g % NS
    const int uu = u0 + g;
    const int t = tile_of(uu);
    if (t != itile) {
      plan(t);
      itile = t;
    }
    const int ka = (uu - t * nks) * BK;
    char* slot = smem + (g % NS) * SB;
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
      if (j < LPA)
        load_lds16(src[j] + ka, slot + (4 * j + wn) * 1024);
      else  // weights (Qwen2.5-7B batch-32 layer 178 -> 165 us)
        load_lds16_nt(src[j] + ka, slot + (4 * j + wn) * 1024);
    }
  };

  f32x16 acc[NI][TJ], park[NI][TJ];
  auto zero = [&]() {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  };
  zero();
  // fp32 partial of tile t from accumulator set a
  auto store_part = [&](f32x16 (&a)[NI][TJ], int t) {
    const int m0 = __builtin_amdgcn_readfirstlane((t % p.tiles_m) * RT);
    const int rows_valid = min(RT, p.M - m0);
    if constexpr (HL) {
#pragma unroll
      for (int i = 0; i < NO; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) a[i][j][r] += a[i + NO][j][r];
    }
    // element offsets (partials stay far below 2^32 elements): the uniform
    // part per store, the lane's column and row parity
    const int ord = __builtin_amdgcn_readfirstlane(
        (int)blockIdx.x - sk_owner((long long)t * nks, U, p.sk_grid));
    const uint32_t tile_off = (uint32_t)(((uint32_t)ord * p.M + m0) * ldp) +
                              (uint32_t)((t / p.tiles_m) * BN + wn * WCOLS);
    const uint32_t lane_off = (uint32_t)(4 * (lane >> 5) * ldp + (lane & 31));
    const int lrow = 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < NO; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rowc = 32 * i + 8 * (r >> 2) + (r & 3);
        if (rowc + lrow < rows_valid) {
          const uint32_t o = tile_off + (uint32_t)(rowc * ldp) + lane_off;
#pragma unroll
          for (int j = 0; j < TJ; ++j) p.part[o + 32 * j] = a[i][j][r];
        }
      }
  };
  int t_park = -1;  // the run's first tile once its accumulators are parked

  const int fr = lane & 31;
  const int fk = lane >> 5;
  constexpr int KS = BK / 16;
  int aoff[KS][NI], boff[KS][TJ];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int c = 2 * ks + fk;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int ra = 32 * i + fr;
      aoff[ks][i] = (ra * kRowChunks + (c ^ swz(ra))) * 16;
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int rb = wn * WCOLS + 32 * j + fr;
      boff[ks][j] = AC * 16 + (rb * kRowChunks + (c ^ swz(rb))) * 16;
    }
  }

  // hi/lo tiles skip their padding-only 32-row MFMA tiles (wave-uniform
  // branches); plain tiles multiply them (see above)
  bool act[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) act[i] = true;
  auto read2 = [&](const char* st, int kh, bf16x8 (&af)[2][NI], bf16x8 (&bfr)[2][TJ]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
        if (!HL || act[i]) af[ks][i] = *reinterpret_cast<const bf16x8*>(st + aoff[kh + ks][i]);
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        bfr[ks][j] = *reinterpret_cast<const bf16x8*>(st + boff[kh + ks][j]);
    }
  };
  auto mma2 = [&](const bf16x8 (&af)[2][NI], const bf16x8 (&bfr)[2][TJ]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < NI; ++i)
        if (!HL || act[i])
#pragma unroll
          for (int j = 0; j < TJ; ++j) acc[i][j] = mfma_32x32x16(af[ks][i], bfr[ks][j], acc[i][j]);
  };
  static_assert(KS == 4, "two halves of two k steps per stage");

#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < total) issue(j);
  for (int g = 0; g < total; ++g) {
    // this wave's part of stage g has landed: loads complete in order, so the
    // loads of the (up to NS - 2) later stages already requested may remain
    // (stores of partials only make the wait longer)
    const int later = min(NS - 2, total - 1 - g);
    if (NS == 4 && later == 2)
      wait_vmcnt<2 * LPT>();
    else if (later >= 1)
      wait_vmcnt<LPT>();
    else
      wait_vmcnt<0>();
    // every wave's part of stage g has landed and every wave is done with
    // the slot of stage g - 1
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (g + NS - 1 < total) issue(g + NS - 1);
    const int uu = u0 + g;
    const int t = tile_of(uu);
    if constexpr (HL) {
      const int m0 = __builtin_amdgcn_readfirstlane((t % p.tiles_m) * RT);
      const int rows_valid = min(RT, p.M - m0);
#pragma unroll
      for (int i = 0; i < NI; ++i) act[i] = (32 * i) % RT < rows_valid;
    }
    const char* st = smem + (g % NS) * SB;
    bf16x8 a0[2][NI], b0[2][TJ], a1[2][NI], b1[2][TJ];
    read2(st, 0, a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    read2(st, 2, a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    mma2(a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    mma2(a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    if (uu - t * nks == nks - 1 && g + 1 < total) {  // the run moves on to the next tile
      if (!HL && RA <= 64 && t_park < 0) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j) park[i][j] = acc[i][j];
        t_park = t;
      } else {
        store_part(acc, t);
      }
      zero();
    }
  }
  if (total > 0) {
    store_part(acc, tile_of(u0 + total - 1));
    if (t_park >= 0) store_part(park, t_park);
  }
}

// Sum of the split-K / stream-K partials + the epilogue of MODE. A block is
// one 256-column weight tile by 4 waves of rows; in a wave, each group of S
// lanes (32, or 16 for SwiGLU's gate/up pairs) is one row and a lane owns 8
// output columns (and the up columns BN/2 further for SwiGLU). Every row of
// a wave lies in one GEMM tile, so all its lanes sum the same number of
// partials; a lane requests up to four of them at once, and the residual or
// bias with the first, so the wave waits on memory about once. The 16 lanes
// of an aligned group hold one head of 128 columns for the QKV epilogue.
template <int MODE>
__global__ __launch_bounds__(256) void gemm2_reduce_kernel(const G2Args p) {
  constexpr bool kDual = MODE == G2_SWIGLU;
  constexpr int NV = kDual ? 16 : 8;        // values summed per lane (gate and up for SwiGLU)
  constexpr int S = kDual ? BN / 16 : BN / 8;  // lanes per row
  constexpr int RW = 64 / S;                // rows per wave
  const int ldp = p.tiles_n * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tn = blockIdx.x;
  const int row = (blockIdx.y * 4 + wave) * RW + lane / S;
  if (row >= p.M) return;  // whole groups of S lanes
  const int j = lane % S;
  const size_t pstride = (size_t)p.M * ldp;
  int cnt = p.splits;
  if (p.streamk) {  // blocks whose runs touched this tile (the same for every row of the wave)
    const int nks = p.Ka / BK;
    const long long U = (long long)p.tiles_m * p.tiles_n * nks;
    const long long t = (long long)tn * p.tiles_m + row / p.rows_per_tile;
    cnt = sk_owner(t * nks + nks - 1, U, p.sk_grid) - sk_owner(t * nks, U, p.sk_grid) + 1;
  }
  cnt = __builtin_amdgcn_readfirstlane(cnt);
  // partial columns of this lane: [c0, c0 + 8) (and the up half at + BN / 2)
  const int c0 = tn * BN + j * 8;
  const int tg = tn + p.tn_base;  // the tile's place among the weight's columns
  const float* q0 = p.part + (size_t)row * ldp + c0;
  auto load = [&](int s, f32x4 (&x)[NV / 4]) {
    const float* q = q0 + s * pstride;
    x[0] = *reinterpret_cast<const f32x4*>(q);
    x[1] = *reinterpret_cast<const f32x4*>(q + 4);
    if constexpr (kDual) {
      x[2] = *reinterpret_cast<const f32x4*>(q + BN / 2);
      x[3] = *reinterpret_cast<const f32x4*>(q + BN / 2 + 4);
    }
  };
  float v[NV];
#pragma unroll
  for (int e = 0; e < NV; ++e) v[e] = 0.f;
  auto sum = [&](int s0, auto n_c) {  // n_c partials from s0, all requested first
    constexpr int n = decltype(n_c)::value;
    f32x4 x[n][NV / 4];
#pragma unroll
    for (int i = 0; i < n; ++i) load(s0 + i, x[i]);
#pragma unroll
    for (int i = 0; i < n; ++i)
#pragma unroll
      for (int h = 0; h < NV / 4; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * h + e] += x[i][h][e];
  };
  // epilogue inputs requested alongside the partials
  const int col = tg * (kDual ? BN / 2 : BN) + j * 8;
  float extra[8];
  if constexpr (MODE == G2_RESID_F32) {
    unpack8(load_bf16x8(p.resid_bf16 + (size_t)row * p.ldr + col), extra);
  } else if constexpr (MODE == G2_RESID_OUT) {
    const float* rr = p.resid_f32 + (size_t)row * p.ldr + col;
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(rr);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(rr + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      extra[e] = a0[e];
      extra[e + 4] = a1[e];
    }
  }
  int s = 0;
  for (; s + 4 <= cnt; s += 4) sum(s, std::integral_constant<int, 4>{});
  switch (cnt - s) {
    case 3: sum(s, std::integral_constant<int, 3>{}); break;
    case 2: sum(s, std::integral_constant<int, 2>{}); break;
    case 1: sum(s, std::integral_constant<int, 1>{}); break;
    default: break;
  }
  if constexpr (kDual) {
    float h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = silu_f32(v[e]) * v[e + 8];
    store_h(p, (size_t)row, col, h);
  } else {
    float (&w8)[8] = *reinterpret_cast<float (*)[8]>(v);
    if constexpr (MODE == G2_BIAS) {
      const bf16* bias = p.bias;
      int nb = col;
      if (col >= p.seg2) {
        bias = p.bias3;
        nb = col - p.seg2;
      } else if (col >= p.seg1) {
        bias = p.bias2;
        nb = col - p.seg1;
      }
      if (bias) {
        float b8[8];
        unpack8(load_bf16x8(bias + nb), b8);
#pragma unroll
        for (int e = 0; e < 8; ++e) w8[e] += b8[e];
      }
      if (p.cache_len)
        qkv_finish<true>(p, (size_t)row, col, w8);
      else
        qkv_finish<false>(p, (size_t)row, col, w8);
      return;
    }
    if constexpr (MODE == G2_RESID_F32 || MODE == G2_RESID_OUT) {
#pragma unroll
      for (int e = 0; e < 8; ++e) w8[e] += extra[e];
    }
    if constexpr (MODE == G2_GATED_F32) gated_finish(p, (size_t)row, col, w8);
    if constexpr (MODE == G2_RESID_OUT) {
      store_bf16x8(p.out_bf16 + (size_t)row * p.ldo + col, pack8(w8));
    } else {
      float* o = p.out_f32 + (size_t)row * p.ldo + col;
      *reinterpret_cast<f32x4*>(o) = f32x4{w8[0], w8[1], w8[2], w8[3]};
      *reinterpret_cast<f32x4*>(o + 4) = f32x4{w8[4], w8[5], w8[6], w8[7]};
    }
  }
}

// Tile shapes: 256 token rows of a plain bf16 A (8 waves); 128 or 256 token
// rows from a [hi | lo] pair (8 waves); the 4-wave decode tiles with an A tile
// of 32, 64 or 128 LDS rows, from a plain bf16 A or from a [hi | lo] pair (16,
// 32 or 64 token rows).
enum : int { T256 = 0, P128_HL, P256, D32, D64, D128, D32_HL, D64_HL, D128_HL };
constexpr int shape_ra(int sh) { return sh == D32 || sh == D32_HL ? 32 : (sh == D64 || sh == D64_HL ? 64 : 128); }
constexpr bool shape_hl(int sh) { return sh >= D32_HL || sh == P128_HL || sh == P256; }
constexpr bool shape_dec(int sh) { return sh >= D32; }
constexpr int shape_kind(int sh) { return sh == P256 ? 2 : (sh == P128_HL ? 1 : 0); }
// (a pair needs its hi and lo rows in different 32-row MFMA tiles: RA >= 64)
int decode_shape(int M, bool pair) {
  if (pair) return M <= 32 ? D64_HL : D128_HL;
  return M <= 32 ? D32 : (M <= 64 ? D64 : D128);
}

template <int MODE, int SHAPE>
hipError_t launch(const G2Args& a, dim3 grid, hipStream_t s) {
  constexpr bool HL = shape_hl(SHAPE);
  // Q/K/V and O always take a [hi | lo] pair; gate/up, down and the gated
  // shared-expert down take a pair or plain bf16
  constexpr bool kPairOnly = MODE == G2_BIAS || MODE == G2_RESID_F32;
  constexpr bool kMoe = MODE == G2_MOE_GU || MODE == G2_MOE_DOWN;
  constexpr bool kDec = shape_dec(SHAPE);
  if constexpr ((kPairOnly && !HL) || (SHAPE != T256 && (kMoe || SHAPE == D32_HL))) {
    return hipErrorInvalidValue;
  } else if constexpr (kDec) {  // decode tiles: stream-K partials
    hipLaunchKernelGGL((gemm2_dec_kernel<MODE, HL, shape_ra(SHAPE)>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
  } else {
    if (a.splits == 1)
      hipLaunchKernelGGL((gemm2_kernel<MODE, false, shape_kind(SHAPE)>), grid, dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((gemm2_kernel<MODE, true, shape_kind(SHAPE)>), grid, dim3(512), 0, s, a);
    return hipGetLastError();
  }
}

int rows_per_tile(int shape) {
  if (shape == T256 || shape == P256) return 256;
  if (shape == P128_HL) return 128;
  return shape_hl(shape) ? shape_ra(shape) / 2 : shape_ra(shape);
}

// stream-K cut of the (tile, k step) units over at most kSkBlocks blocks
constexpr int kSkBlocks = 256;
int sk_grid(long long units) { return (int)std::min<long long>(kSkBlocks, units); }
int sk_max_count(int tiles, int nks, int G) {
  const long long U = (long long)tiles * nks;
  int mx = 1;
  for (int t = 0; t < tiles; ++t)
    mx = std::max(mx, sk_owner((long long)t * nks + nks - 1, U, G) -
                          sk_owner((long long)t * nks, U, G) + 1);
  return mx;
}

template <int MODE>
hipError_t run(G2Args a, int shape, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  const int rt = rows_per_tile(shape);
  a.rows_per_tile = rt;
  a.tiles_m = (a.M + rt - 1) / rt;
  const int nks = a.Ka / BK;
  dim3 grid;
  if (shape_dec(shape)) {  // decode tiles: stream-K, always through the partials
    a.streamk = 1;
    a.sk_grid = sk_grid((long long)a.tiles_m * a.tiles_n * nks);
    a.splits = 1;
    grid = dim3(a.sk_grid);
  } else {
    a.splits = a.splits < 1 ? 1 : (a.splits > nks ? nks : a.splits);
    a.ksteps_per_split = (nks + a.splits - 1) / a.splits;
    a.splits = (nks + a.ksteps_per_split - 1) / a.ksteps_per_split;
    const int total = a.tiles_m * a.tiles_n * a.splits;
    grid = dim3(8 * ((total + 7) / 8));
  }
  hipError_t e;
  switch (shape) {
    case T256: e = launch<MODE, T256>(a, grid, s); break;
    case P128_HL: e = launch<MODE, P128_HL>(a, grid, s); break;
    case P256: e = launch<MODE, P256>(a, grid, s); break;
    case D32: e = launch<MODE, D32>(a, grid, s); break;
    case D64: e = launch<MODE, D64>(a, grid, s); break;
    case D128: e = launch<MODE, D128>(a, grid, s); break;
    case D64_HL: e = launch<MODE, D64_HL>(a, grid, s); break;
    case D128_HL: e = launch<MODE, D128_HL>(a, grid, s); break;
    default: e = hipErrorInvalidValue;
  }
  if (e != hipSuccess || (!a.streamk && a.splits == 1)) return e;
  constexpr int kRowsPerBlock = 4 * (MODE == G2_SWIGLU ? 4 : 2);  // 4 waves x rows per wave
  hipLaunchKernelGGL(gemm2_reduce_kernel<MODE>, dim3((unsigned)a.tiles_n, (unsigned)((a.M + kRowsPerBlock - 1) / kRowsPerBlock)),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

// Prefill GEMMs of a [hi | lo] pair A: 256-row tiles (32-deep stages of hi,
// lo and weight rows), or 128-row tiles holding hi and lo rows over 64-deep
// stages (same MFMA work per stage, twice the tiles at half the stages).
// Shape and split count minimise an estimate in units of one stage of a
// block (256 x 256 x 64 of MFMA work, about 1.9 us measured):
// waves of up to 256 blocks times k steps per block, plus, with split-K, a
// reduce launch and the partials' write and read back at ~5 TB/s. A tile
// count just past a whole number of waves leaves most CUs idle in the last
// one; then the first columns can run as whole tiles and the last
// `tail_cols` column tiles as a second launch split `tail_splits` ways
// (Qwen2.5-7B 4 x 512 QKV: 288 tiles, 190 -> 157 us).
struct PairPlan {
  int shape, splits, tail_cols, tail_splits;
};
PairPlan pair_plan(int M, int N, int K) {
  PairPlan best{P256, 1, 0, 1};
  double best_c = 1e30;
  auto waves = [](long long blocks) { return (double)((blocks + 255) / 256); };
  auto part_cost = [&](int sp, int cols) { return (5.0 + 2.0 * sp * M * (double)cols * 4 / 5e6) / 1.9; };
  for (int shape : {P256, P128_HL}) {
    const int rows = shape == P256 ? 256 : 128;
    const int ks = (shape == P256 ? 2 * K : K) / BK;
    // a 256-row stage (hi, lo and weight rows together) runs faster than a
    // 128-row one: weighing it at 0.93 moved plans that cut the dense prefill
    // layers by 2-5 % (Qwen2.5-7B 1 x 1024 1044 -> 991 us, 4 x 512 1839 ->
    // 1749, Qwen3-32B 2048 3666 -> 3533); 0.88 gained another 0-6 % on single
    // GEMMs (Qwen3-8B down 384 -> 361 us), 0.97 lost 3-6 %
    const double unit = shape == P256 ? 0.88 : 1.0;
    const int tiles_m = (M + rows - 1) / rows, tiles_n = N / BN;
    auto consider = [&](double c, PairPlan pl) {
      if (c < best_c - 1e-9) {
        best_c = c;
        best = pl;
      }
    };
    for (int sp = 1; sp <= 8 && sp * 8 <= ks; ++sp) {
      const int per = (ks + sp - 1) / sp;
      if ((ks + per - 1) / per != sp) continue;
      double c = waves((long long)tiles_m * tiles_n * sp) * per * unit;
      if (sp > 1) c += part_cost(sp, N);
      consider(c, {shape, sp, 0, 1});
    }
    for (int tc = 1; tc < tiles_n; ++tc)
      for (int st = 2; st <= 8 && st * 8 <= ks; ++st) {
        const int per = (ks + st - 1) / st;
        if ((ks + per - 1) / per != st) continue;
        // + the second GEMM launch, 5 units beyond the partials' traffic
        // (weighed at 20, the plans kept Qwen3-30B-A3B 4096-token Q/K/V on
        // 2.5 waves of 128-row tiles: 209.5 us; at 5 it takes one wave of
        // 256-row tiles and a 4-way split tail: 196.4 us; Qwen3-8B Q/K/V
        // 224.9 -> 219.7 us, Qwen3-32B O 336.0 -> 329.2 us)
        const double c = (waves((long long)tiles_m * (tiles_n - tc)) * ks +
                          waves((long long)tiles_m * tc * st) * per) * unit +
                         part_cost(st, tc * BN) + 5.0;
        consider(c, {shape, 1, tc, st});
      }
  }
  return best;
}

G2Args base(const bf16* A, int M, int Ka, const bf16* B, int Kb, int splits, void* part) {
  G2Args a{};
  a.A = A;
  a.lda = Ka;
  a.M = M;
  a.Ka = Ka;
  a.B = B;
  a.ldb = Kb;
  a.Kb = Kb;
  a.seg1 = a.seg2 = 0x7fffffff;
  a.splits = splits;
  a.part = static_cast<float*>(part);
  return a;
}

}  // namespace

size_t ql_gemm2_part_bytes(int M, int b_rows, int splits) {
  return splits <= 1 ? 0 : (size_t)splits * M * ((b_rows + BN - 1) / BN) * BN * 4;
}

bool ql_gemm2_ok(int N, int Kb, bool dual) {
  return Kb % BK == 0 && (dual ? N % (BN / 2) == 0 : N % BN == 0);
}

size_t ql_gemm2_pair_part_bytes(int M, int N, int K) {
  if (M <= 0) return 0;
  const PairPlan pl = pair_plan(M, N, K);
  return pl.tail_cols > 0 ? ql_gemm2_part_bytes(M, pl.tail_cols * BN, pl.tail_splits)
                          : ql_gemm2_part_bytes(M, N, pl.splits);
}

size_t ql_gemm2_decode_part_bytes(int M, int b_rows, int K, bool pair) {
  if (M <= 0) return 0;
  const int shape = decode_shape(M, pair);
  const int rt = rows_per_tile(shape);
  const int tiles = ((M + rt - 1) / rt) * ((b_rows + BN - 1) / BN);
  const int nks = K / BK;
  const int G = sk_grid((long long)tiles * nks);
  return (size_t)sk_max_count(tiles, nks, G) * M * ((b_rows + BN - 1) / BN) * BN * 4;
}

namespace {
// a prefill pair plan: one launch over every column tile, or whole tiles
// for the first columns and a split-K launch for the last tail_cols
template <int MODE>
hipError_t run_pair(const G2Args& a, const PairPlan& pl, hipStream_t s) {
  if (pl.tail_cols <= 0) return run<MODE>(a, pl.shape, s);
  G2Args m = a, t = a;
  m.tiles_n = a.tiles_n - pl.tail_cols;
  m.splits = 1;
  t.tn_base = m.tiles_n;
  t.tiles_n = pl.tail_cols;
  t.splits = pl.tail_splits;
  hipError_t e = run<MODE>(m, pl.shape, s);
  return e != hipSuccess ? e : run<MODE>(t, pl.shape, s);
}
}  // namespace

hipError_t ql_gemm2_qkv(const bf16* A2, int M, const bf16* Wq, const bf16* Wk, const bf16* Wv,
                        int q, int kv, int K, const bf16* bq, const bf16* bk, const bf16* bv,
                        const QkvFinish& f, bool rows128, int splits, void* part, hipStream_t s) {
  if (rows128 != (f.cache_len != nullptr)) return hipErrorInvalidValue;  // decode <=> 128 rows
  const PairPlan pl = rows128 ? PairPlan{decode_shape(M, true), 1, 0, 1} : pair_plan(M, q + 2 * kv, K);
  (void)splits;
  G2Args a = base(A2, M, pl.shape == P256 ? 2 * K : K, Wq, K, pl.splits, part);
  a.lda = 2 * K;
  a.S = f.S;
  a.pos_offset = f.pos_offset;
  a.T_max = f.T_max;
  a.cache_len = f.cache_len;
  a.seq_start = f.seq_start;
  a.prefix = f.prefix;
  a.nseq = f.nseq;
  a.n_q_heads = q / 128;
  a.n_kv_heads = kv / 128;
  a.eps = f.eps;
  a.omega = f.omega;
  a.q_norm_g = f.q_norm_g;
  a.k_norm_g = f.k_norm_g;
  a.q_out = f.q_out;
  a.k_cache = f.k_cache;
  a.v_cache = f.v_cache;
  a.B2 = Wk;
  a.B3 = Wv;
  a.seg1 = q;
  a.seg2 = q + kv;
  a.bias = bq;
  a.bias2 = bk;
  a.bias3 = bv;
  a.ldo = q + 2 * kv;
  a.tiles_n = (q + 2 * kv) / BN;
  return run_pair<G2_BIAS>(a, pl, s);
}

hipError_t ql_gemm2_resid_f32(const bf16* A2, int M, const bf16* W, int N, int K,
                              const bf16* resid, float* out, bool rows128, int splits, void* part,
                              hipStream_t s) {
  const PairPlan pl = rows128 ? PairPlan{decode_shape(M, true), 1, 0, 1} : pair_plan(M, N, K);
  (void)splits;
  G2Args a = base(A2, M, pl.shape == P256 ? 2 * K : K, W, K, pl.splits, part);
  a.lda = 2 * K;
  a.resid_bf16 = resid;
  a.ldr = N;
  a.out_f32 = out;
  a.ldo = N;
  a.tiles_n = N / BN;
  return run_pair<G2_RESID_F32>(a, pl, s);
}

// A of a gate/up, down or shared-expert GEMM, and its launch plan. A pair
// input on the prefill tiles takes the same plan as Q/K/V and O (256-row
// tiles over a doubled K or 128-row hi/lo tiles, split count, and a split-K
// tail when the last wave of tiles would be nearly empty); on the decode
// tiles hi and lo rows sit side by side (each weight tile serves both). A
// plain bf16 input on the prefill tiles splits `splits` ways.
namespace {
struct AbPlan {
  G2Args a;
  PairPlan pl;
};
AbPlan base_ab(const bf16* A, int M, const bf16* W, int N, int K, bool pair, bool rows128,
               int splits, void* part) {
  PairPlan pl{T256, splits, 0, 1};
  if (rows128) pl = PairPlan{decode_shape(M, pair), 1, 0, 1};
  else if (pair) pl = pair_plan(M, N, K);
  G2Args a = base(A, M, pl.shape == P256 ? 2 * K : K, W, K, pl.splits, part);
  if (pair) a.lda = 2 * K;
  return {a, pl};
}
}  // namespace

hipError_t ql_gemm2_resid_out(const bf16* A, int M, const bf16* W, int N, int K,
                              const float* resid, bf16* out, bool rows128, int splits, void* part,
                              hipStream_t s, bool pair_in) {
  AbPlan ab = base_ab(A, M, W, N, K, pair_in, rows128, splits, part);
  G2Args& a = ab.a;
  a.resid_f32 = resid;
  a.ldr = N;
  a.out_bf16 = out;
  a.ldo = N;
  a.tiles_n = N / BN;
  return run_pair<G2_RESID_OUT>(a, ab.pl, s);
}

hipError_t ql_gemm2_gated_out(const bf16* A, int M, const bf16* W, int N, int K,
                              const float* gate_logit, int gate_ld, const float* resid_f32,
                              const bf16* resid_bf16, float* out, bool rows128, int splits,
                              void* part, hipStream_t s, bool pair_in) {
  AbPlan ab = base_ab(A, M, W, N, K, pair_in, rows128, splits, part);
  G2Args& a = ab.a;
  a.gate_logit = gate_logit;
  a.gate_ld = gate_ld;
  a.resid_f32 = resid_f32;
  a.resid_bf16 = resid_bf16;
  a.ldr = N;
  a.out_f32 = out;
  a.ldo = N;
  a.tiles_n = N / BN;
  return run_pair<G2_GATED_F32>(a, ab.pl, s);
}

hipError_t ql_gemm2_swiglu(const bf16* A, int M, const bf16* Wg, const bf16* Wu, int F, int K,
                           bf16* out, bool rows128, int splits, void* part, hipStream_t s,
                           bool pair) {
  AbPlan ab = base_ab(A, M, Wg, 2 * F, K, pair, rows128, splits, part);
  G2Args& a = ab.a;
  a.B2 = Wu;
  a.out_bf16 = out;
  a.ldo = pair ? 2 * F : F;
  a.out_lo = pair ? F : 0;
  a.tiles_n = F / (BN / 2);
  return run_pair<G2_SWIGLU>(a, ab.pl, s);
}

hipError_t ql_gemm2_moe_gu(const bf16* Z2, const int* slot_token, const bf16* Wg, const bf16* Wu,
                           int mf, int d, const int* tile_expert, const int* tile_row0,
                           const int* tile_rows, const int* num_tiles, int max_tiles, int bm,
                           bf16* H2, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  if (bm != 128 && bm != 256) return hipErrorInvalidValue;
  // [hi | lo] rows: 256- or 128-row pair tiles over 32-deep stages (2 x Kb
  // for the step count; the 128-row ones two blocks per CU)
  G2Args a = base(Z2, 0, 2 * d, Wg, d, 1, nullptr);
  a.lda = 2 * d;
  a.B2 = Wu;
  a.b_expert_stride = (size_t)mf * d;
  a.row_index = slot_token;
  a.tile_expert = tile_expert;
  a.tile_row0 = tile_row0;
  a.tile_rows = tile_rows;
  a.num_tiles = num_tiles;
  a.out_bf16 = H2;
  a.ldo = 2 * mf;
  a.out_lo = mf;
  a.tiles_n = mf / (BN / 2);
  const int total = max_tiles * a.tiles_n;
  if (bm == 256)
    hipLaunchKernelGGL((gemm2_kernel<G2_MOE_GU, false, 2>), dim3(8 * ((total + 7) / 8)), dim3(512),
                       0, s, a);
  else
    hipLaunchKernelGGL((gemm2_kernel<G2_MOE_GU, false, 3>), dim3(8 * ((total + 7) / 8)), dim3(512),
                       0, s, a);
  return hipGetLastError();
}

hipError_t ql_gemm2_moe_down(const bf16* H2, const bf16* Wd, int mf, int d,
                             const int* tile_expert, const int* tile_row0, const int* tile_rows,
                             const int* num_tiles, int max_tiles, int bm, float* out,
                             hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  if (bm != 128 && bm != 256) return hipErrorInvalidValue;
  G2Args a = base(H2, 0, 2 * mf, Wd, mf, 1, nullptr);  // both kinds step over 2 mf
  a.lda = 2 * mf;
  a.b_expert_stride = (size_t)d * mf;
  a.tile_expert = tile_expert;
  a.tile_row0 = tile_row0;
  a.tile_rows = tile_rows;
  a.num_tiles = num_tiles;
  a.out_f32 = out;
  a.ldo = d;
  a.tiles_n = d / BN;
  const int total = max_tiles * a.tiles_n;
  if (bm == 256)
    hipLaunchKernelGGL((gemm2_kernel<G2_MOE_DOWN, false, 2>), dim3(8 * ((total + 7) / 8)),
                       dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((gemm2_kernel<G2_MOE_DOWN, false, 3>), dim3(8 * ((total + 7) / 8)),
                       dim3(512), 0, s, a);
  return hipGetLastError();
}

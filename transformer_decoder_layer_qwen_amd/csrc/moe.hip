// Routing side of the sparse-MoE FFN: router + top-k, token permutation and
// the weighted combine.
//
// Router ("Qwen2.5-7B 结构拆解" §10.2; "MoE 初步：参数量计算、Qwen3-30B-A3B、GQA
// 与 Sparse MoE" Router 机制): logits = z W_router^T over all E experts, the k
// largest are kept (ties to the lower expert index), and their gate weights
// are a softmax over the k selected logits (norm_topk_prob) or the raw
// probabilities of a softmax over all E logits.
//   z is the fp32 RMSNorm2 output. It is split as z = hi + lo with hi, lo
//   bf16 (hi = RNE(z), lo = RNE(z - hi)), so two bf16 MFMAs against the exact
//   bf16 router weights give the logits to about 2^-16 relative precision of
//   z, with fp32 accumulation.
//
// Permutation: a histogram of expert ids per 256-token block, one scan that
// turns counts into expert segments and a tile table for the grouped GEMM,
// and a stable scatter that lists each expert's tokens in token order (up to
// 256 tokens, all three steps run in one block). Every step is integer work,
// so the permutation is exactly reproducible.
//
// Combine ("Qwen2.5-7B 结构拆解" §10.2: the k outputs are added elementwise
// with their gate weights, no further normalisation): y = r + sum_i w_i out_i
// in rank order, no atomics.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kTok = 16;  // tokens per router block (the MFMA's N)
constexpr int kRW = 8;    // waves per router block; they split K
constexpr int kEP = kTok + 4;  // LDS pitch (floats) of one expert's token row

// logits[t][e] = z_t . w_e with z fp32 (a bf16 hi + lo pair on the MFMA) and
// w bf16. A block takes 16 tokens x 16 MT experts; wave w sums K range
// [w d/8, (w+1) d/8), KU 32-deep k steps per round with all of the round's
// loads in flight (no branches inside a round); the waves' partial logits
// meet in LDS (expert rows padded to 20 floats so the 16 token lanes and the
// 4 expert groups of a write land on distinct banks) and the block writes
// its logits to `logits` [N, E]. Blocks go to the XCDs in contiguous
// stretches of (token block, expert group) with the expert group fastest,
// so the groups of a token block share its z rows through one L2.
template <int MT, int KU>
__global__ __launch_bounds__(kRW * 64) void router_logits_kernel(const RouterArgs p, int ngroups) {
  constexpr int EB = 16 * MT;  // experts per block
  __shared__ float part[kRW / 2][EB * kEP];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int ntb = (p.N + kTok - 1) / kTok;
  const int total = ntb * ngroups;
  const int chunk = (total + 7) / 8;
  if ((int)(blockIdx.x / 8) >= chunk) return;
  const int wk = (int)(blockIdx.x % 8) * chunk + (int)(blockIdx.x / 8);
  if (wk >= total) return;
  const int t0 = (wk / ngroups) * kTok;
  const int e0 = (wk % ngroups) * EB;

  // B operand: z^T; lane (token col, k group grp)
  const int tok = t0 + col;
  const bool tv = tok < p.N;
  const int kw = p.d / kRW;  // K per wave (a multiple of 32 KU)
  const float* zr = p.zf + (size_t)(tv ? tok : 0) * p.d + wave * kw + 8 * grp;
  // rows E .. E + n_extra - 1 come from w_extra (a shared expert's gate);
  // rows past them (a last, part-filled tile) re-read the last row and are
  // never stored
  const int etot = p.E + p.n_extra;
  const bf16* wr[MT];
#pragma unroll
  for (int et = 0; et < MT; ++et) {
    const int row = min(e0 + 16 * et + col, etot - 1);
    wr[et] = (row < p.E ? p.wr + (size_t)row * p.d : p.w_extra + (size_t)(row - p.E) * p.d) +
             wave * kw + 8 * grp;
  }

  f32x4 acc[MT];
#pragma unroll
  for (int et = 0; et < MT; ++et) acc[et] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < kw; k += 32 * KU) {
    f32x4 z[KU][2];
    bf16x8 wf[KU][MT];
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      z[u][0] = *reinterpret_cast<const f32x4*>(zr + k + 32 * u);
      z[u][1] = *reinterpret_cast<const f32x4*>(zr + k + 32 * u + 4);
#pragma unroll
      for (int et = 0; et < MT; ++et) wf[u][et] = load_bf16x8(wr[et] + k + 32 * u);
    }
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      bf16x8 zh, zl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v0 = tv ? z[u][0][i] : 0.f, v1 = tv ? z[u][1][i] : 0.f;
        zh[i] = (bf16)v0;
        zl[i] = (bf16)(v0 - (float)zh[i]);
        zh[i + 4] = (bf16)v1;
        zl[i + 4] = (bf16)(v1 - (float)zh[i + 4]);
      }
#pragma unroll
      for (int et = 0; et < MT; ++et) {
        acc[et] = mfma_16x16x32(wf[u][et], zh, acc[et]);
        acc[et] = mfma_16x16x32(wf[u][et], zl, acc[et]);
      }
    }
  }
  // lane holds D[expert 16 et + 4 grp + r][token col]; the upper half of the
  // waves parks its partials, the lower half adds its own, then slot sums
  constexpr int kHalf = kRW / 2;
  if (wave >= kHalf) {
#pragma unroll
    for (int et = 0; et < MT; ++et)
#pragma unroll
      for (int r = 0; r < 4; ++r) part[wave - kHalf][(et * 16 + 4 * grp + r) * kEP + col] = acc[et][r];
  }
  __syncthreads();
  if (wave < kHalf) {
#pragma unroll
    for (int et = 0; et < MT; ++et)
#pragma unroll
      for (int r = 0; r < 4; ++r) part[wave][(et * 16 + 4 * grp + r) * kEP + col] += acc[et][r];
  }
  __syncthreads();
  for (int i = tid; i < kTok * EB; i += kRW * 64) {
    const int tl = i / EB, e = i % EB;  // expert fastest: coalesced stores
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kHalf; ++w) v += part[w][e * kEP + tl];
    if (t0 + tl < p.N && e0 + e < etot) p.logits[(size_t)(t0 + tl) * etot + e0 + e] = v;
  }
}

// Top-k and gate weights, one wave per token. Expert i's rank is the number
// of experts j with logit_j > logit_i, plus those with an equal logit and
// j < i (descending logit, ties to the lower index; a NaN logit counts as
// -inf); the k experts of rank < k are the selection, in rank order. Each
// lane ranks its PER experts against the token's whole row, read from LDS as
// broadcasts: one compare and one add per pair for "greater", the same for
// "equal", and only a lane that sees a tie counts the lower-index equals.
// Weights: a softmax over the selected logits (norm_topk_prob), else the
// selected probabilities of a softmax over all E.
template <int PER>
__global__ __launch_bounds__(256) void router_topk_kernel(const RouterArgs p) {
  __shared__ __attribute__((aligned(16))) float row[4][kMaxExperts];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= p.N) return;  // wave-uniform: the other waves use only their own rows
  const int E = p.E;
  float v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = lane + 64 * j;
    float x = -INFINITY;
    if (e < E) {
      x = p.logits[(size_t)t * (E + p.n_extra) + e];
      x = x == x ? x : -INFINITY;
    }
    // entries up to the next multiple of 4 are read by the rank loop below:
    // -inf there never counts as a greater logit
    if (e < ((E + 3) & ~3)) row[wave][e] = x;
    v[j] = x;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  int gt[PER], eq[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) gt[j] = eq[j] = 0;
  for (int j0 = 0; j0 < E; j0 += 4) {
    const f32x4 o = *reinterpret_cast<const f32x4*>(&row[wave][j0]);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        gt[j] += o[q] > v[j] ? 1 : 0;
        eq[j] += o[q] == v[j] ? 1 : 0;
      }
  }
  int rank[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = lane + 64 * j;
    rank[j] = gt[j];
    if (eq[j] > 1 && e < E) {  // a tie: the equal experts below e come first
      for (int jj = 0; jj < e; ++jj) rank[j] += row[wave][jj] == v[j] ? 1 : 0;
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < PER; ++j) mx = fmaxf(mx, v[j]);
  mx = wave_max(mx);
  float den_sel = 0.f, den_all = 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const bool live = lane + 64 * j < E;
    const float ex = (live && v[j] != -INFINITY) ? __expf(v[j] - mx) : 0.f;
    den_all += ex;
    if (live && rank[j] < p.k) den_sel += ex;
  }
  den_sel = wave_sum(den_sel);
  den_all = wave_sum(den_all);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = lane + 64 * j;
    if (e < E && rank[j] < p.k) {
      const float ex = v[j] != -INFINITY ? __expf(v[j] - mx) : 0.f;
      p.idx[(size_t)t * p.k + rank[j]] = e;
      p.w[(size_t)t * p.k + rank[j]] = ex / (p.norm_topk ? den_sel : den_all);
    }
  }
}

__global__ __launch_bounds__(256) void moe_hist_kernel(const PermuteArgs p) {
  __shared__ int h[kMaxExperts];
  for (int e = threadIdx.x; e < p.E; e += 256) h[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t < p.N)
    for (int i = 0; i < p.k; ++i) atomicAdd(&h[p.idx[(size_t)t * p.k + i]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < p.E; e += 256) p.hist[blockIdx.x * p.E + e] = h[e];
}

// single block: expert segments, per-block bases and the tile table
__global__ __launch_bounds__(256) void moe_scan_kernel(const PermuteArgs p) {
  __shared__ int tot[kMaxExperts];
  __shared__ int ntile[kMaxExperts];
  const int e = threadIdx.x;
  const int nblk = (p.N + 255) / 256;
  if (e < p.E) {
    int s = 0;
    for (int b = 0; b < nblk; ++b) s += p.hist[b * p.E + e];
    tot[e] = s;
    ntile[e] = (s + p.bm - 1) / p.bm;
  }
  __syncthreads();
  if (e < p.E) {
    int off = 0, toff = 0;
    for (int j = 0; j < e; ++j) {  // E <= 256: a plain prefix is cheap enough
      off += tot[j];
      toff += ntile[j];
    }
    p.offsets[e] = off;
    int run = off;
    for (int b = 0; b < nblk; ++b) {
      p.blkoff[b * p.E + e] = run;
      run += p.hist[b * p.E + e];
    }
    for (int j = 0; j < ntile[e]; ++j) {
      p.tile_expert[toff + j] = e;
      p.tile_row0[toff + j] = off + j * p.bm;
      p.tile_rows[toff + j] = min(p.bm, tot[e] - j * p.bm);
    }
    if (e == p.E - 1) {
      p.offsets[p.E] = off + tot[e];
      *p.num_tiles = toff + ntile[e];
    }
  }
}

__global__ __launch_bounds__(256) void moe_scatter_kernel(const PermuteArgs p) {
  __shared__ uint32_t bits[kMaxExperts][8];
  for (int i = threadIdx.x; i < p.E * 8; i += 256) bits[i / 8][i % 8] = 0u;
  __syncthreads();
  const int tl = threadIdx.x;
  const int t = blockIdx.x * 256 + tl;
  const bool tv = t < p.N;
  if (tv)
    for (int i = 0; i < p.k; ++i)
      atomicOr(&bits[p.idx[(size_t)t * p.k + i]][tl >> 5], 1u << (tl & 31));
  __syncthreads();
  if (!tv) return;
  for (int i = 0; i < p.k; ++i) {
    const int e = p.idx[(size_t)t * p.k + i];
    int rank = __popc(bits[e][tl >> 5] & ((1u << (tl & 31)) - 1u));
    for (int w = 0; w < (tl >> 5); ++w) rank += __popc(bits[e][w]);
    const int pos = p.blkoff[blockIdx.x * p.E + e] + rank;
    p.slot_token[pos] = t;
    p.pos_of[(size_t)t * p.k + i] = pos;
  }
}

// Up to 256 tokens: the histogram, the scan with the tile table and the
// scatter in one block (the same slots as the three kernels: experts in
// order, tokens ascending within an expert). Per expert a 256-bit token mask
// in LDS gives both the expert's count and each token's rank.
__global__ __launch_bounds__(256) void moe_permute_small_kernel(const PermuteArgs p) {
  __shared__ uint32_t bits[kMaxExperts][8];
  __shared__ int tot[kMaxExperts];
  __shared__ int ntile[kMaxExperts];
  __shared__ int base[kMaxExperts];
  const int tl = threadIdx.x;
  for (int i = tl; i < p.E * 8; i += 256) bits[i / 8][i % 8] = 0u;
  __syncthreads();
  const bool tv = tl < p.N;
  if (tv)
    for (int i = 0; i < p.k; ++i) atomicOr(&bits[p.idx[(size_t)tl * p.k + i]][tl >> 5], 1u << (tl & 31));
  __syncthreads();
  const int e = tl;
  if (e < p.E) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) c += __popc(bits[e][w]);
    tot[e] = c;
    ntile[e] = (c + p.bm - 1) / p.bm;
  }
  __syncthreads();
  if (e < p.E) {
    int off = 0, toff = 0;
    for (int j = 0; j < e; ++j) {  // E <= 256: a plain prefix is cheap enough
      off += tot[j];
      toff += ntile[j];
    }
    base[e] = off;
    p.offsets[e] = off;
    for (int j = 0; j < ntile[e]; ++j) {
      p.tile_expert[toff + j] = e;
      p.tile_row0[toff + j] = off + j * p.bm;
      p.tile_rows[toff + j] = min(p.bm, tot[e] - j * p.bm);
    }
    if (e == p.E - 1) {
      p.offsets[p.E] = off + tot[e];
      *p.num_tiles = toff + ntile[e];
    }
  }
  __syncthreads();
  if (!tv) return;
  for (int i = 0; i < p.k; ++i) {
    const int x = p.idx[(size_t)tl * p.k + i];
    int rank = __popc(bits[x][tl >> 5] & ((1u << (tl & 31)) - 1u));
    for (int w = 0; w < (tl >> 5); ++w) rank += __popc(bits[x][w]);
    const int pos = base[x] + rank;
    p.slot_token[pos] = tl;
    p.pos_of[(size_t)tl * p.k + i] = pos;
  }
}

template <class TR>
QL_DEV void load8(const TR* p, float (&f)[8]);
template <>
QL_DEV void load8<float>(const float* p, float (&f)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[j] = a[j];
    f[j + 4] = b[j];
  }
}
template <>
QL_DEV void load8<bf16>(const bf16* p, float (&f)[8]) {
  unpack8(load_bf16x8(p), f);
}

// One wave per (token, 512-column chunk), 8 consecutive columns per lane:
// small batches still spread over many waves, and a wave waits on memory
// twice (slot indices, weights and residual, then the expert rows). The
// expert rows are read 8 at a time with their loads issued together and
// summed in rank order in fp32, then added to the residual.
template <class TR>
__global__ __launch_bounds__(256) void moe_combine_kernel(const CombineArgs p, const TR* resid) {
  constexpr int kGroup = 8;
  const int lane = threadIdx.x & 63;
  const int nchunk = (p.d + 511) / 512;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gw >= p.N * nchunk) return;
  const int t = gw / nchunk;
  const int c = (gw - t * nchunk) * 512 + lane * 8;
  if (c >= p.d) return;  // d % 256 == 0: the upper half of a last, half chunk
  float acc[8];
  load8<TR>(resid + (size_t)t * p.d + c, acc);
  float sum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; i0 < p.k; i0 += kGroup) {
    f32x4 o[kGroup][2];
    float w[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const int r = min(i0 + i, p.k - 1);
      const float* src = p.out_slot + (size_t)p.pos_of[(size_t)t * p.k + r] * p.d + c;
      o[i][0] = *reinterpret_cast<const f32x4*>(src);
      o[i][1] = *reinterpret_cast<const f32x4*>(src + 4);
      w[i] = i0 + i < p.k ? p.w[(size_t)t * p.k + r] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < kGroup; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sum[j] += w[i] * o[i][0][j];
        sum[j + 4] += w[i] * o[i][1][j];
      }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] += sum[j];
  store_bf16x8(p.y + (size_t)t * p.d + c, pack8(acc));
}

}  // namespace

hipError_t ql_router_topk(const RouterArgs& a, hipStream_t s) {
  if (a.N <= 0) return hipSuccess;
  if (!a.logits || a.E < 1 || a.E > kMaxExperts || a.d % (32 * kRW) || a.n_extra < 0 ||
      a.n_extra > 16 || (a.n_extra > 0 && !a.w_extra))
    return hipErrorInvalidValue;
  const int ntb = (a.N + kTok - 1) / kTok;
  const int etot = a.E + a.n_extra;
  const int et = (etot + 15) / 16;
  // expert tiles per block: all of them when token blocks alone fill the
  // chip (z rows read once) and the tiles are whole, else one (more blocks,
  // one round of loads each; the expert groups of a token block share its z
  // rows through one L2)
  const int mt = (ntb >= 128 && etot % 16 == 0) ? et : 1;
  const int ngroups = et / mt;
  const int kw = a.d / kRW;
  const int ku = (kw % 256 == 0 && mt == 1) ? 8 : (kw % 128 == 0 && mt <= 4) ? 4 : (kw % 64 == 0 && mt <= 8) ? 2 : 1;
  const int total = ntb * ngroups;
  const dim3 grid(8 * ((total + 7) / 8)), block(kRW * 64);
  switch (mt * 16 + ku) {
#define QL_R(MT, KU)                                                                        \
  case MT * 16 + KU:                                                                        \
    hipLaunchKernelGGL((router_logits_kernel<MT, KU>), grid, block, 0, s, a, ngroups);      \
    break;
    QL_R(1, 1) QL_R(1, 2) QL_R(1, 4) QL_R(1, 8)
    QL_R(2, 1) QL_R(2, 2) QL_R(2, 4) QL_R(3, 1) QL_R(3, 2) QL_R(3, 4) QL_R(4, 1) QL_R(4, 2) QL_R(4, 4)
    QL_R(5, 1) QL_R(5, 2) QL_R(6, 1) QL_R(6, 2) QL_R(7, 1) QL_R(7, 2) QL_R(8, 1) QL_R(8, 2)
    QL_R(9, 1) QL_R(10, 1) QL_R(11, 1) QL_R(12, 1) QL_R(13, 1) QL_R(14, 1) QL_R(15, 1) QL_R(16, 1)
#undef QL_R
    default:
      return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 tgrid((a.N + 3) / 4);
  switch ((a.E + 63) / 64) {
    case 1: hipLaunchKernelGGL(router_topk_kernel<1>, tgrid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL(router_topk_kernel<2>, tgrid, dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL(router_topk_kernel<3>, tgrid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL(router_topk_kernel<4>, tgrid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t ql_moe_permute(const PermuteArgs& a, hipStream_t s) {
  if (a.N <= 0) return hipSuccess;
  if (a.N <= 256) {
    hipLaunchKernelGGL(moe_permute_small_kernel, dim3(1), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const int nblk = (a.N + 255) / 256;
  hipLaunchKernelGGL(moe_hist_kernel, dim3(nblk), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(moe_scan_kernel, dim3(1), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(moe_scatter_kernel, dim3(nblk), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t ql_moe_combine(const CombineArgs& a, const void* resid, int resid_is_f32,
                          hipStream_t s) {
  if (a.N <= 0) return hipSuccess;
  if (a.d % 8) return hipErrorInvalidValue;
  const int blocks = (a.N * ((a.d + 511) / 512) + 3) / 4;
  if (resid_is_f32)
    hipLaunchKernelGGL(moe_combine_kernel<float>, dim3(blocks), dim3(256), 0, s, a,
                       static_cast<const float*>(resid));
  else
    hipLaunchKernelGGL(moe_combine_kernel<bf16>, dim3(blocks), dim3(256), 0, s, a,
                       static_cast<const bf16*>(resid));
  return hipGetLastError();
}

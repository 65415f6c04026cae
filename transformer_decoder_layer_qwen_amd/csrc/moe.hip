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
// and a stable scatter that lists each expert's tokens in token order. Every
// step is integer work, so the permutation is exactly reproducible.
//
// Combine ("Qwen2.5-7B 结构拆解" §10.2: the k outputs are added elementwise
// with their gate weights, no further normalisation): y = r + sum_i w_i out_i
// in rank order, no atomics.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kTok = 16;  // tokens per router block (the MFMA's N)
constexpr int kRW = 8;    // waves per router block; they split K

// logits[t][e] = z_t . w_e with z fp32 (a bf16 hi + lo pair on the MFMA) and
// w bf16; wave w sums K range [w d/8, (w+1) d/8) for every expert tile, KU
// 32-deep k steps per round with all of the round's loads in flight; the
// waves' partial logits meet in LDS. Then one wave per token picks the top k
// (descending logit, ties to the lower expert index) and forms the weights.
// MT: expert tiles held per wave (E <= 16 MT); KU: k steps per round.
template <int MT, int KU>
__global__ __launch_bounds__(kRW * 64) void router_topk_kernel(const RouterArgs p) {
  extern __shared__ float part[];  // [kRW / 2][kTok][E]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int t0 = blockIdx.x * kTok;
  const int E = p.E;
  const int etiles = E / 16;

  // B operand: z^T; lane (token col, k group grp)
  const int tok = t0 + col;
  const bool tv = tok < p.N;
  const int kw = p.d / kRW;  // K per wave (a multiple of 32: d % 256 == 0)
  const float* zr = p.zf + (size_t)(tv ? tok : 0) * p.d + wave * kw + 8 * grp;
  const bf16* wr = p.wr + (size_t)col * p.d + wave * kw + 8 * grp;

  f32x4 acc[MT];
#pragma unroll
  for (int et = 0; et < MT; ++et) acc[et] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < kw; k += 32 * KU) {
    f32x4 z[KU][2];
    bf16x8 wf[KU][MT];
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      if (k + 32 * u >= kw) break;  // the wave's K range ends inside the round
      z[u][0] = *reinterpret_cast<const f32x4*>(zr + k + 32 * u);
      z[u][1] = *reinterpret_cast<const f32x4*>(zr + k + 32 * u + 4);
#pragma unroll
      for (int et = 0; et < MT; ++et)
        if (et < etiles) wf[u][et] = load_bf16x8(wr + (size_t)et * 16 * p.d + k + 32 * u);
    }
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      if (k + 32 * u >= kw) break;
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
        if (et < etiles) {
          acc[et] = mfma_16x16x32(wf[u][et], zh, acc[et]);
          acc[et] = mfma_16x16x32(wf[u][et], zl, acc[et]);
        }
      }
    }
  }
  // lane holds D[expert 16 et + 4 grp + r][token col]; the upper half of the
  // waves parks its partials, the lower half adds its own, then slot sums
  constexpr int kHalf = kRW / 2;
  if (wave >= kHalf) {
#pragma unroll
    for (int et = 0; et < MT; ++et)
      if (et < etiles)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          part[((wave - kHalf) * kTok + col) * E + et * 16 + 4 * grp + r] = acc[et][r];
  }
  __syncthreads();
  if (wave < kHalf) {
#pragma unroll
    for (int et = 0; et < MT; ++et)
      if (et < etiles)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          part[(wave * kTok + col) * E + et * 16 + 4 * grp + r] += acc[et][r];
  }
  __syncthreads();
  for (int i = tid; i < kTok * E; i += kRW * 64) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kHalf; ++w) v += part[w * kTok * E + i];
    part[i] = v;  // slot 0 now holds the logits; each i is read and written by one thread
  }
  __syncthreads();

  // top-k: one wave per token; lane holds experts lane, lane + 64, ...
  const int per = (E + 63) / 64;
  for (int tl = wave; tl < kTok; tl += kRW) {
    const int t = t0 + tl;
    if (t >= p.N) break;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      v[j] = (j < per && e < E) ? part[tl * E + e] : -INFINITY;
    }
    if (p.logits) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j < per && lane + 64 * j < E) p.logits[(size_t)t * E + lane + 64 * j] = v[j];
    }
    // full-softmax statistics (used when norm_topk_prob == 0)
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) mx = fmaxf(mx, v[j]);
    mx = wave_max(mx);
    float den_all = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) den_all += (v[j] == -INFINITY) ? 0.f : __expf(v[j] - mx);
    den_all = wave_sum(den_all);

    // selection i lands in lane i (k <= 32 < 64 lanes)
    float my_v = -INFINITY, top = -INFINITY;
    int my_i = 0;
    for (int i = 0; i < p.k; ++i) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = lane + 64 * j;
        if (v[j] > bv || (v[j] == bv && e < bi && v[j] != -INFINITY)) {
          bv = v[j];
          bi = e;
        }
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const float ov = __shfl_xor(bv, m, kWave);
        const int oi = __shfl_xor(bi, m, kWave);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      // NaN logits compare false everywhere: keep the index in range so the
      // permutation never addresses outside its tables
      if (bi < 0 || bi >= E) bi = i % E;
      if (i == 0) top = bv;
      if (lane == i) {
        my_v = bv;
        my_i = bi;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (lane + 64 * j == bi) v[j] = -INFINITY;
    }
    const bool mine = lane < p.k;
    const float ew = mine ? __expf(my_v - top) : 0.f;
    const float den = wave_sum(ew);
    if (mine) {
      const float w = p.norm_topk ? ew / den : __expf(my_v - mx) / den_all;
      p.idx[(size_t)t * p.k + lane] = my_i;
      p.w[(size_t)t * p.k + lane] = w;
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

// One wave per token, 8 consecutive columns per lane; the expert rows are
// read 8 at a time with their loads issued together and summed in rank
// order in fp32, then added to the residual.
template <class TR>
__global__ __launch_bounds__(256) void moe_combine_kernel(const CombineArgs p, const TR* resid) {
  constexpr int kGroup = 8;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= p.N) return;
  for (int c = lane * 8; c < p.d; c += 512) {
    float sum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < p.k; i0 += kGroup) {
      bf16x8 o[kGroup];
      float w[kGroup];
#pragma unroll
      for (int i = 0; i < kGroup; ++i) {
        const int r = min(i0 + i, p.k - 1);
        o[i] = load_bf16x8(p.out_slot + (size_t)p.pos_of[(size_t)t * p.k + r] * p.d + c);
        w[i] = i0 + i < p.k ? p.w[(size_t)t * p.k + r] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < kGroup; ++i) {
        float f[8];
        unpack8(o[i], f);
#pragma unroll
        for (int j = 0; j < 8; ++j) sum[j] += w[i] * f[j];
      }
    }
    float acc[8];
    load8<TR>(resid + (size_t)t * p.d + c, acc);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] += sum[j];
    store_bf16x8(p.y + (size_t)t * p.d + c, pack8(acc));
  }
}

}  // namespace

hipError_t ql_router_topk(const RouterArgs& a, hipStream_t s) {
  if (a.N <= 0) return hipSuccess;
  const int blocks = (a.N + kTok - 1) / kTok;
  const size_t lds = (size_t)(kRW / 2) * kTok * a.E * sizeof(float);
  const int et = a.E / 16;
  if (et <= 2) hipLaunchKernelGGL((router_topk_kernel<2, 4>), dim3(blocks), dim3(kRW * 64), lds, s, a);
  else if (et <= 4) hipLaunchKernelGGL((router_topk_kernel<4, 4>), dim3(blocks), dim3(kRW * 64), lds, s, a);
  else if (et <= 8) hipLaunchKernelGGL((router_topk_kernel<8, 2>), dim3(blocks), dim3(kRW * 64), lds, s, a);
  else hipLaunchKernelGGL((router_topk_kernel<16, 1>), dim3(blocks), dim3(kRW * 64), lds, s, a);
  return hipGetLastError();
}

hipError_t ql_moe_permute(const PermuteArgs& a, hipStream_t s) {
  if (a.N <= 0) return hipSuccess;
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
  const int blocks = (a.N + 3) / 4;
  if (resid_is_f32)
    hipLaunchKernelGGL(moe_combine_kernel<float>, dim3(blocks), dim3(256), 0, s, a,
                       static_cast<const float*>(resid));
  else
    hipLaunchKernelGGL(moe_combine_kernel<bf16>, dim3(blocks), dim3(256), 0, s, a,
                       static_cast<const bf16*>(resid));
  return hipGetLastError();
}

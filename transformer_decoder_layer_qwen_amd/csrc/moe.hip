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

constexpr int kTok = 16;  // tokens per router block

__global__ __launch_bounds__(256) void router_topk_kernel(const RouterArgs p) {
  extern __shared__ float logit_lds[];  // [kTok][E]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int t0 = blockIdx.x * kTok;
  const int E = p.E;
  const int etiles = E / 16;

  // B operand: z^T split into hi/lo bf16; lane (token col, group grp)
  const int tok = t0 + col;
  const bool tv = tok < p.N;
  const float* zr = p.zf + (size_t)(tv ? tok : 0) * p.d + 8 * grp;

  for (int et0 = wave; et0 < etiles; et0 += 8) {
    // two expert tiles per pass (et0 and et0 + 4) share the z fragments
    const int et1 = et0 + 4;
    const bool two = et1 < etiles;
    const bf16* w0 = p.wr + (size_t)(et0 * 16 + col) * p.d + 8 * grp;
    const bf16* w1 = p.wr + (size_t)((two ? et1 : et0) * 16 + col) * p.d + 8 * grp;
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < p.d; k += 32) {
      float zv[8];
      if (tv) {
        const f32x4 z0 = *reinterpret_cast<const f32x4*>(zr + k);
        const f32x4 z1 = *reinterpret_cast<const f32x4*>(zr + k + 4);
        zv[0] = z0[0]; zv[1] = z0[1]; zv[2] = z0[2]; zv[3] = z0[3];
        zv[4] = z1[0]; zv[5] = z1[1]; zv[6] = z1[2]; zv[7] = z1[3];
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) zv[i] = 0.f;
      }
      bf16x8 zh, zl;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        zh[i] = (bf16)zv[i];
        zl[i] = (bf16)(zv[i] - (float)zh[i]);
      }
      const bf16x8 wf0 = load_bf16x8(w0 + k);
      a0 = mfma_16x16x32(wf0, zh, a0);
      a0 = mfma_16x16x32(wf0, zl, a0);
      if (two) {
        const bf16x8 wf1 = load_bf16x8(w1 + k);
        a1 = mfma_16x16x32(wf1, zh, a1);
        a1 = mfma_16x16x32(wf1, zl, a1);
      }
    }
    // lane holds D[expert 4*grp + r][token col]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      logit_lds[col * E + et0 * 16 + 4 * grp + r] = a0[r];
      if (two) logit_lds[col * E + et1 * 16 + 4 * grp + r] = a1[r];
    }
  }
  __syncthreads();

  // top-k: one wave per token; lane holds experts lane, lane+64, ...
  const int per = (E + 63) / 64;
  for (int tl = wave; tl < kTok; tl += 4) {
    const int t = t0 + tl;
    if (t >= p.N) break;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      v[j] = (j < per && e < E) ? logit_lds[tl * E + e] : -INFINITY;
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

    float sel_v[kMaxTopK];
    int sel_i[kMaxTopK];
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
      sel_v[i] = bv;
      sel_i[i] = bi;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (lane + 64 * j == bi) v[j] = -INFINITY;
    }
    if (lane == 0) {
      float den = 0.f;
      for (int i = 0; i < p.k; ++i) den += __expf(sel_v[i] - sel_v[0]);
      for (int i = 0; i < p.k; ++i) {
        const float w = p.norm_topk ? __expf(sel_v[i] - sel_v[0]) / den
                                    : __expf(sel_v[i] - mx) / den_all;
        p.idx[(size_t)t * p.k + i] = sel_i[i];
        p.w[(size_t)t * p.k + i] = w;
      }
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
__global__ __launch_bounds__(256) void moe_combine_kernel(const CombineArgs p, const TR* resid) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= p.N) return;
  int pos[kMaxTopK];
  float w[kMaxTopK];
  for (int i = 0; i < p.k; ++i) {
    pos[i] = p.pos_of[(size_t)t * p.k + i];
    w[i] = p.w[(size_t)t * p.k + i];
  }
  for (int c = lane * 4; c < p.d; c += 256) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < p.k; ++i) {
      const f32x4 o = *reinterpret_cast<const f32x4*>(p.out_slot + (size_t)pos[i] * p.d + c);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] += w[i] * o[j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      p.y[(size_t)t * p.d + c + j] = (bf16)(to_f32(resid[(size_t)t * p.d + c + j]) + acc[j]);
  }
}

}  // namespace

hipError_t ql_router_topk(const RouterArgs& a, hipStream_t s) {
  if (a.N <= 0) return hipSuccess;
  const int blocks = (a.N + kTok - 1) / kTok;
  hipLaunchKernelGGL(router_topk_kernel, dim3(blocks), dim3(256), kTok * a.E * sizeof(float), s,
                     a);
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

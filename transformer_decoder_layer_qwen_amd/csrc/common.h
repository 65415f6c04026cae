// Device-side building blocks shared by the gfx950 kernels of the layer:
// element types, 16-byte vector types, MFMA wrappers and wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

#define QL_DEV __device__ __forceinline__
#define QL_HD __host__ __device__ __forceinline__

constexpr int kWave = 64;

// bf16 -> fp32 is exact; fp32 -> bf16 rounds to nearest even (v_cvt_pk_bf16_f32).
QL_DEV float to_f32(bf16 x) { return (float)x; }
QL_DEV float to_f32(float x) { return x; }
template <class T> QL_DEV T from_f32(float x);
template <> QL_DEV float from_f32<float>(float x) { return x; }
template <> QL_DEV bf16 from_f32<bf16>(float x) { return (bf16)x; }

QL_DEV bf16x8 load_bf16x8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
QL_DEV void store_bf16x8(bf16* p, bf16x8 v) { *reinterpret_cast<bf16x8*>(p) = v; }

QL_DEV void unpack8(bf16x8 v, float* f) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (float)v[i];
}
QL_DEV bf16x8 pack8(const float* f) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (bf16)f[i];
  return v;
}

// D = A * B + C on one wave.
// 16x16x32: lane l supplies A[l%16][kslot(l/16, 0..7)] and B[kslot(l/16, 0..7)][l%16];
//           lane l receives D[4*(l/16) + r][l%16], r = 0..3.
// 32x32x16: lane l supplies A[l%32][kslot(l/32, 0..7)] and B[kslot(l/32, 0..7)][l%32];
//           lane l receives D[8*(r/4) + 4*(l/32) + r%4][l%32], r = 0..15.
// A and B lanes of the same k-group share the same k indices, so any
// consistent assignment of k values to slots yields the same product.
QL_DEV f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
QL_DEV f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// A lane's value combined with the lane 16 (or 32) places away, i ^ 16 (i ^ 32),
// by gfx950's row swaps (v_permlane16_swap / v_permlane32_swap: no LDS round
// trip). Swapping a register with itself leaves each lane holding its own
// value and its partner's, in an order that differs by half; max and sum do
// not depend on it.
QL_DEV float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
QL_DEV float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
QL_DEV float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
QL_DEV float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Value of the lane k places earlier in its row of 16 lanes (a DPP row rotate).
template <int K>
QL_DEV float row_ror(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + K, 0xF, 0xF, false));
}
// Sum / max over the lane's row of 16 lanes, left in every lane of the row:
// rotations by 8, 4, 2 and 1 reach every lane of the row (no LDS round trip).
QL_DEV float row16_sum(float x) {
  x += row_ror<8>(x);
  x += row_ror<4>(x);
  x += row_ror<2>(x);
  return x + row_ror<1>(x);
}
QL_DEV float row16_max(float x) {
  x = fmaxf(x, row_ror<8>(x));
  x = fmaxf(x, row_ror<4>(x));
  x = fmaxf(x, row_ror<2>(x));
  return fmaxf(x, row_ror<1>(x));
}
// Sum / max over the wave, in every lane. These and the row and half exchanges
// above read other lanes' registers directly, so every lane of the wave must
// be active where they are used (all call sites are wave-uniform).
QL_DEV float wave_sum(float v) { return xor32_sum(xor16_sum(row16_sum(v))); }
QL_DEV float wave_max(float v) { return xor32_max(xor16_max(row16_max(v))); }

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
QL_DEV float group_sum(float v, int width) {
  for (int m = width >> 1; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// SiLU(z) = z * sigmoid(z); the hardware reciprocal (about 1 ulp) instead of
// a correctly rounded division, which takes ten instructions
QL_DEV float silu_f32(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

constexpr float kLog2e = 1.4426950408889634f;

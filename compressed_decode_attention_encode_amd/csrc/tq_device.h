// Device helpers for the gfx950 kernels: input conversion, exact fp64 -> fp16
// rounding, and wavefront (64-lane) reductions.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/tq.h"

namespace tq {

constexpr int kWave = 64;

// fp16 / bf16 storage bits -> float (exact).
template <int DT>
__device__ __forceinline__ float in_to_f32(uint32_t bits16) {
  if constexpr (DT == TQ_F16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
  } else {
    return __uint_as_float(bits16 << 16);
  }
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// float64 -> fp16 bits, round to nearest even, computed directly from the double
// (no intermediate float rounding).  Overflow gives +-inf.
__device__ __forceinline__ uint32_t f64_to_f16_rne(double x) {
  uint64_t b = (uint64_t)__double_as_longlong(x);
  uint32_t sign = (uint32_t)(b >> 48) & 0x8000u;
  b &= 0x7FFFFFFFFFFFFFFFull;
  if (b >= 0x7FF0000000000000ull) return sign | 0x7C00u | (b > 0x7FF0000000000000ull ? 0x200u : 0u);
  if (b == 0) return sign;
  int e = (int)(b >> 52) - 1023;
  uint64_t m = (b & 0x000FFFFFFFFFFFFFull) | 0x0010000000000000ull;  // 53-bit significand
  if (e < -25) return sign;                                             // below half the smallest subnormal
  int shift = (e >= -14) ? 42 : 42 + (-14 - e);                        // bits to drop
  uint64_t keep = m >> shift;
  uint64_t rem = m & ((1ull << shift) - 1);
  uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (keep & 1))) keep += 1;
  if (e >= -14) {
    int ee = e + 15;
    if (keep == (1ull << 11)) { keep >>= 1; ee += 1; }
    if (ee >= 31) return sign | 0x7C00u;
    return sign | ((uint32_t)ee << 10) | ((uint32_t)keep & 0x3FFu);
  }
  return sign | (uint32_t)keep;  // subnormal (keep == 0x400 encodes the smallest normal)
}

// Lane exchange with lane ^ M (M = 1, 2, 4, 8) through DPP moves (VALU, no LDS):
//   xor 1 / xor 2: quad_perm [1,0,3,2] / [2,3,0,1];
//   xor 4: row_half_mirror (i -> 7-i in 8 lanes) then quad_perm [3,2,1,0];
//   xor 8: row_mirror (i -> 15-i in 16 lanes) then row_half_mirror.
template <int M>
__device__ __forceinline__ uint32_t xor_lanes_u32(uint32_t v) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8, "DPP xor covers 1, 2, 4, 8");
  if constexpr (M == 1) {
    return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);
  } else if constexpr (M == 2) {
    return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);
  } else if constexpr (M == 4) {
    const uint32_t t = __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);
    return __builtin_amdgcn_mov_dpp(t, 0x1B, 0xF, 0xF, false);
  } else {
    const uint32_t t = __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false);
    return __builtin_amdgcn_mov_dpp(t, 0x141, 0xF, 0xF, false);
  }
}

template <int M>
__device__ __forceinline__ double xor_lanes(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = xor_lanes_u32<M>((uint32_t)u);
  const uint32_t hi = xor_lanes_u32<M>((uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

template <int M>
__device__ __forceinline__ float xor_lanes(float x) {
  return __uint_as_float(xor_lanes_u32<M>(__float_as_uint(x)));
}

// Value of lane + 1 within the lane's row of 16 (row_shl:1); the last lane of a row gets 0.
__device__ __forceinline__ uint32_t next_lane_u32(uint32_t v) {
  return __builtin_amdgcn_mov_dpp(v, 0x101, 0xF, 0xF, true);
}

// Sum over the N consecutive lanes sharing lane / N (N <= 16), by DPP exchanges.
// Packed fp16 pairs held in a 32-bit word (low half = first element).
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// c + a.lo * b.lo + a.hi * b.hi: fp16 products (exact in fp32), fp32 sum.
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
}

// Two floats rounded to fp16 (nearest-even) and packed, lo in the low half.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f16x2_t r;
  r.x = (_Float16)lo;
  r.y = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

template <int N>
__device__ __forceinline__ double group_sum_dpp(double v) {
  if constexpr (N >= 2) v += xor_lanes<1>(v);
  if constexpr (N >= 4) v += xor_lanes<2>(v);
  if constexpr (N >= 8) v += xor_lanes<4>(v);
  if constexpr (N >= 16) v += xor_lanes<8>(v);
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

// Sum over the `n` consecutive lanes that share lane / n (n a power of two <= 64).
template <int N, typename T>
__device__ __forceinline__ T group_sum(T v) {
#pragma unroll
  for (int m = 1; m < N; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

}  // namespace tq

// Device-side helpers shared by the gfx950 kernels: vector types for the
// MFMA builtins, bf16 <-> fp32 conversion, and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16x2 (round to nearest even), low half = a.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __bf16 lo = (__bf16)a;
  __bf16 hi = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, kWave));
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Workgroup id remap so that consecutive logical ids stay on one XCD:
// the hardware deals workgroups round-robin over 8 XCDs (id % 8), so
// logical = (xcd's share start) + (id / 8).  A bijection on [0, n).
__device__ __forceinline__ int xcd_remap(int id, int n) {
  const int q = n >> 3, r = n & 7;
  const int xcd = id & 7, local = id >> 3;
  return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// Workgroup id remap that keeps the whole chip on one stretch of logical
// ids: XCD x's k-th workgroup (hardware id 8 k + x) works in window
// w = k / c of 8 c logical ids, on its slice (x + w) % 8 of c consecutive
// ids.  All eight XCDs share each window, and the slice an XCD takes turns
// with the window, so an XCD does not meet the same part of every head
// (where work varies along the sequence).  The last partial window falls
// back to xcd_remap.  A bijection on [0, n).
__device__ __forceinline__ int xcd_window_remap(int id, int n, int c) {
  const int s = 8 * c, full = n / s * s;
  if (id >= full) return full + xcd_remap(id - full, n - full);
  const int k = id >> 3, x = id & 7, w = k / c;
  return w * s + ((x + w) & 7) * c + k % c;
}

}  // namespace sa

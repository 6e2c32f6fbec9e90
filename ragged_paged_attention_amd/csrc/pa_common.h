// Device-side helpers shared by the HIP kernels of libpa (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// ---------------------------------------------------------------------------
// 16-bit float formats <-> float32
// ---------------------------------------------------------------------------
// A bfloat16 value is the upper half of the float32 with the same bits.
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even; NaN stays a quiet NaN with its sign.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// Storage traits: T is the stored element type, load() widens to float and
// store() rounds to nearest-even.
struct F32 {
  using T = float;
  static __device__ __forceinline__ float load(T x) { return x; }
  static __device__ __forceinline__ T store(float x) { return x; }
};
struct BF16 {
  using T = uint16_t;
  static __device__ __forceinline__ float load(T x) { return bf16_bits_to_f32(x); }
  static __device__ __forceinline__ T store(float x) { return f32_to_bf16_bits(x); }
};
struct F16 {
  using T = uint16_t;
  static __device__ __forceinline__ float load(T x) { return f16_bits_to_f32(x); }
  static __device__ __forceinline__ T store(float x) { return f32_to_f16_bits(x); }
};

// ---------------------------------------------------------------------------
// errors
// ---------------------------------------------------------------------------
__device__ __forceinline__ void flag(int32_t* d_err, int32_t bits) {
  if (d_err) atomicOr(d_err, bits);
}

__host__ __device__ __forceinline__ int32_t ceil_div(int32_t a, int32_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// wave64 reductions: butterfly over lane distances 32..1 with __shfl_xor
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace pa

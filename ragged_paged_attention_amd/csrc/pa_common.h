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
// KV write: one token row into its cache slot
// ---------------------------------------------------------------------------
// With the cache laid out [num_blocks, block_size, Hkv, D], the K (or V) of
// all heads of one slot is one contiguous row of Hkv*D elements, like a row of
// the new k/v [T, Hkv, D] ("vLLM Continuous Batching：从 Forward Shape 理解两个
// 核心参数" §2.3 第一步: slot_mapping names each token's physical slot).  One
// wave copies row t: the slot is one load, then each lane copies VEC-byte
// chunks, two K and two V loads in flight per pass, every access coalesced.
// A negative slot is skipped (a padding token); a slot past the pool flags
// PA_DERR_SLOT_OOB and writes nothing.
template <int VEC>
struct KvVec;
template <> struct KvVec<16> { using T = uint4; };
template <> struct KvVec<8> { using T = uint2; };
template <> struct KvVec<4> { using T = uint32_t; };
template <> struct KvVec<2> { using T = uint16_t; };

template <int VEC>
__device__ __forceinline__ void write_kv_row(const char* __restrict__ k, const char* __restrict__ v,
                                             const int32_t* __restrict__ slot_mapping, int64_t t, int64_t row_bytes,
                                             char* __restrict__ k_cache, char* __restrict__ v_cache,
                                             int64_t num_slots, int32_t* d_err, int lane) {
  using V = typename KvVec<VEC>::T;
  const int32_t slot = slot_mapping[t];
  if (slot < 0) return;
  if (slot >= num_slots) {
    if (lane == 0) flag(d_err, PA_DERR_SLOT_OOB);
    return;
  }
  const int64_t per_row = row_bytes / VEC;
  const V* ks = reinterpret_cast<const V*>(k + t * row_bytes);
  const V* vs = reinterpret_cast<const V*>(v + t * row_bytes);
  V* kd = reinterpret_cast<V*>(k_cache + static_cast<int64_t>(slot) * row_bytes);
  V* vd = reinterpret_cast<V*>(v_cache + static_cast<int64_t>(slot) * row_bytes);
  for (int64_t c = lane; c < per_row; c += 128) {
    const bool two = c + 64 < per_row;
    const V k0 = ks[c], v0 = vs[c];
    V k1 = k0, v1 = v0;
    if (two) {
      k1 = ks[c + 64];
      v1 = vs[c + 64];
    }
    kd[c] = k0;
    vd[c] = v0;
    if (two) {
      kd[c + 64] = k1;
      vd[c + 64] = v1;
    }
  }
}

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

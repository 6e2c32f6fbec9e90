// MFMA helpers shared by the fast attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_common.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kD = 128;          // head_dim of the fast paths
constexpr int kChunk = 16;       // tokens per MFMA tile edge
constexpr int kVRowBytes = 288;  // LDS row pitch of a staged V tile: 256 B + 32 B, so the
                                 // 16 rows one transposed read touches start in distinct banks

// Per-dtype MFMA.  qk: v_mfma_f32_16x16x32 (8 elements per lane per operand);
// pv16: v_mfma_f32_16x16x16 (4 per lane); mm32: v_mfma_f32_32x32x16 (8 per
// lane, 16 results).
//   A[m = lane%16][k = 8*(lane/16) + j]  (16x16x32)   A[m][k = 4*(lane/16) + j]  (16x16x16)
//   B[k = same][n = lane%16]             D[m = 4*(lane/16) + j][n = lane%16]
//   32x32x16: A[m = lane%32][k = 8*(lane/32) + j], B[k = same][n = lane%32],
//             result r: D[m = 8*(r/4) + 4*(lane/32) + r%4][n = lane%32]
// (all layouts checked on the GPU with small integer operands).
// dot1: the sum of a packed pair plus c, in one v_dot2 against (1, 1).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

template <class F> struct Mma;
template <> struct Mma<BF16> {
  static constexpr uint32_t kOnePair = 0x3F803F80u;  // two bf16 1.0
  // two floats -> two bf16 (nearest-even) in one 32-bit word, low half first
  static __device__ __forceinline__ uint32_t pk(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
  }
  static __device__ __forceinline__ f32x4_t qk(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t pv(i16x4_t a, i16x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16_t mm32(uint4 a, uint4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ float dot1(uint32_t p, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, p), __builtin_bit_cast(bf16x2_t, kOnePair),
                                           c, false);
  }
  static __device__ __forceinline__ uint16_t cvt(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
  }
};
template <> struct Mma<F16> {
  static constexpr uint32_t kOnePair = 0x3C003C00u;  // two f16 1.0
  static __device__ __forceinline__ uint32_t pk(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), f16x2_t));
  }
  static __device__ __forceinline__ f32x4_t qk(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t pv(i16x4_t a, i16x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16_t mm32(uint4 a, uint4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ float dot1(uint32_t p, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, p), __builtin_bit_cast(f16x2_t, kOnePair), c, false);
  }
  static __device__ __forceinline__ uint16_t cvt(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  }
};

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// Streaming (non-temporal) 16-byte load: data read once is not kept in the
// caches, which lets a pure HBM stream run closer to peak.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_nt(const uint16_t* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float xor_max(float v, int m) { return fmaxf(v, __shfl_xor(v, m, 64)); }
__device__ __forceinline__ float xor_sum(float v, int m) { return v + __shfl_xor(v, m, 64); }

// Combine the four 16-lane groups (lanes l, l^16, l^32, l^48) with gfx950's
// VALU lane swaps instead of LDS-based shuffles.  With both operands equal to
// x, v_permlane32_swap leaves x[l] and x[l ^ 32] in the two results, and
// v_permlane16_swap x[l] and x[l ^ 16] (lane layout checked on the GPU).
__device__ __forceinline__ float group_max4(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float m32 = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(m32);
  const auto b = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum4(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float s32 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t w = __float_as_uint(s32);
  const auto b = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Transposed LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane L
// supplies the address of 4 consecutive 16-bit elements; lanes 4j..4j+3
// together supply row j (16 elements) of a 4x16 tile, and lane i receives
// column i, i.e. element i of rows 0..3.
__device__ __forceinline__ i16x4_t lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(p));
}

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) {
  return static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
}

}  // namespace pa

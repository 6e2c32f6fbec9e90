// pa_write_kv: scatter this step's new K/V rows into the paged cache.
//
// "vLLM Continuous Batching：从 Forward Shape 理解两个核心参数" §2.3 第一步:
// slot_mapping gives, for every flat token, the physical slot its K/V goes to;
// "vLLM 原理" §3.7 stores the rows before attention runs.
//
// With the cache laid out [num_blocks, block_size, Hkv, D], all heads of one
// slot are one contiguous row of Hkv*D elements, exactly like a row of the
// new k/v [T, Hkv, D].  So the scatter is a copy of T rows of row_bytes each:
// every thread moves VEC bytes (16 when the row size and pointers allow),
// consecutive threads cover consecutive bytes of a row, so both the loads and
// the stores are fully coalesced.  HBM-bound: 2 x 2 x T x row_bytes bytes.
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

template <int VEC>
struct Vec;
template <> struct Vec<16> { using T = uint4; };
template <> struct Vec<8> { using T = uint2; };
template <> struct Vec<4> { using T = uint32_t; };
template <> struct Vec<2> { using T = uint16_t; };

template <int VEC>
__global__ __launch_bounds__(256) void write_kv_kernel(
    const char* __restrict__ k, const char* __restrict__ v, const int32_t* __restrict__ slot_mapping,
    int32_t T, int64_t row_bytes, char* __restrict__ k_cache, char* __restrict__ v_cache,
    int64_t num_slots, int32_t* __restrict__ d_err) {
  using V = typename Vec<VEC>::T;
  const int64_t per_row = row_bytes / VEC;
  const int64_t total = static_cast<int64_t>(T) * per_row;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; c < total; c += stride) {
    const int64_t t = c / per_row;
    const int64_t off = (c - t * per_row) * VEC;
    const int32_t slot = slot_mapping[t];
    if (slot < 0) continue;
    if (slot >= num_slots) {
      if (off == 0) flag(d_err, PA_DERR_SLOT_OOB);
      continue;
    }
    const int64_t src = t * row_bytes + off;
    const int64_t dst = static_cast<int64_t>(slot) * row_bytes + off;
    *reinterpret_cast<V*>(k_cache + dst) = *reinterpret_cast<const V*>(k + src);
    *reinterpret_cast<V*>(v_cache + dst) = *reinterpret_cast<const V*>(v + src);
  }
}

}  // namespace

hipError_t launch_write_kv(const void* k, const void* v, const int32_t* slot_mapping, int32_t T,
                           int64_t row_bytes, void* k_cache, void* v_cache, int64_t num_slots,
                           int32_t* d_err, hipStream_t stream) {
  if (T == 0 || row_bytes == 0) return hipSuccess;
  const uintptr_t align = reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) |
                          reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache) |
                          static_cast<uintptr_t>(row_bytes);
  int vec = 16;
  while (vec > 2 && (align % vec) != 0) vec >>= 1;
  const int64_t chunks = static_cast<int64_t>(T) * (row_bytes / vec);
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  const dim3 grid(static_cast<unsigned>(blocks));
  const char* kc = static_cast<const char*>(k);
  const char* vc = static_cast<const char*>(v);
  char* kd = static_cast<char*>(k_cache);
  char* vd = static_cast<char*>(v_cache);
  launch_mark("write_kv_kernel", stream);
  switch (vec) {
    case 16: write_kv_kernel<16><<<grid, 256, 0, stream>>>(kc, vc, slot_mapping, T, row_bytes, kd, vd, num_slots, d_err); break;
    case 8: write_kv_kernel<8><<<grid, 256, 0, stream>>>(kc, vc, slot_mapping, T, row_bytes, kd, vd, num_slots, d_err); break;
    case 4: write_kv_kernel<4><<<grid, 256, 0, stream>>>(kc, vc, slot_mapping, T, row_bytes, kd, vd, num_slots, d_err); break;
    default: write_kv_kernel<2><<<grid, 256, 0, stream>>>(kc, vc, slot_mapping, T, row_bytes, kd, vd, num_slots, d_err); break;
  }
  launch_done(stream);
  return hipGetLastError();
}

}  // namespace pa

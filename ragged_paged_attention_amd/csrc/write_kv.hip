// pa_write_kv: scatter this step's new K/V rows into the paged cache.
//
// "vLLM Continuous Batching：从 Forward Shape 理解两个核心参数" §2.3 第一步:
// slot_mapping gives, for every flat token, the physical slot its K/V goes to;
// "vLLM 原理" §3.7 stores the rows before attention runs.
//
// With the cache laid out [num_blocks, block_size, Hkv, D], all heads of one
// slot are one contiguous row of Hkv*D elements, exactly like a row of the
// new k/v [T, Hkv, D].  So the scatter is a copy of T rows of row_bytes each:
// one wave per row, lanes on consecutive VEC-byte chunks (16 when the row size
// and pointers allow), so both the loads and the stores are fully coalesced.
// HBM-bound: 2 x 2 x T x row_bytes bytes.
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

// One wave per token row (write_kv_row), four rows per workgroup.
template <int VEC>
__global__ __launch_bounds__(256) void write_kv_kernel(
    const char* __restrict__ k, const char* __restrict__ v, const int32_t* __restrict__ slot_mapping,
    int32_t T, int64_t row_bytes, char* __restrict__ k_cache, char* __restrict__ v_cache,
    int64_t num_slots, int32_t* __restrict__ d_err) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= T) return;
  write_kv_row<VEC>(k, v, slot_mapping, t, row_bytes, k_cache, v_cache, num_slots, d_err, threadIdx.x & 63);
}

// Validation (pa_set_validation): flags PA_DERR_DUP_SLOT when two rows of
// one write carry the same in-range slot ("vLLM 原理" §2.1: copy-on-write
// keeps any two writers off one block, so a repeated slot is a caller bug).
// Row t compares its slot with every row before it: rows are taken 256 at a
// time into LDS and read back as broadcasts.  O(T^2 / 2) compares in all; a
// debugging aid, off by default.
constexpr int kDupRows = 256;
__global__ __launch_bounds__(kDupRows) void dup_slot_kernel(const int32_t* __restrict__ slot_mapping, int32_t T,
                                                          int64_t num_slots, int32_t* __restrict__ d_err) {
  __shared__ int32_t tile[kDupRows];
  const int32_t t = static_cast<int32_t>(blockIdx.x) * kDupRows + static_cast<int32_t>(threadIdx.x);
  const int32_t mine = t < T ? slot_mapping[t] : -1;
  const bool live = mine >= 0 && mine < num_slots;
  bool dup = false;
  // every row before this workgroup's last row; the trip count is uniform
  const int32_t end = min(T, (static_cast<int32_t>(blockIdx.x) + 1) * kDupRows);
  for (int32_t base = 0; base < end; base += kDupRows) {
    __syncthreads();
    tile[threadIdx.x] = base + static_cast<int32_t>(threadIdx.x) < T ? slot_mapping[base + threadIdx.x] : -1;
    __syncthreads();
    if (live) {
      const int32_t n = min(kDupRows, t - base);  // rows u < t of this tile
      for (int32_t j = 0; j < n; ++j) dup |= tile[j] == mine;
    }
  }
  if (dup) flag(d_err, PA_DERR_DUP_SLOT);
}

}  // namespace

hipError_t launch_write_kv(const void* k, const void* v, const int32_t* slot_mapping, int32_t T,
                           int64_t row_bytes, void* k_cache, void* v_cache, int64_t num_slots,
                           int32_t* d_err, bool validate, hipStream_t stream) {
  if (T == 0 || row_bytes == 0) return hipSuccess;
  if (validate && d_err) {
    launch_mark("dup_slot_kernel", stream);
    dup_slot_kernel<<<static_cast<unsigned>((static_cast<int64_t>(T) + kDupRows - 1) / kDupRows), kDupRows, 0,
                      stream>>>(slot_mapping, T, num_slots, d_err);
    launch_done(stream);
  }
  const uintptr_t align = reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) |
                          reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache) |
                          static_cast<uintptr_t>(row_bytes);
  int vec = 16;
  while (vec > 2 && (align % vec) != 0) vec >>= 1;
  const dim3 grid(static_cast<unsigned>((static_cast<int64_t>(T) + 3) / 4));  // 4 token rows per workgroup
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

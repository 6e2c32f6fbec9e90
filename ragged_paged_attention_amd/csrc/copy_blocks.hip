// pa_copy_blocks: whole-block copies for copy-on-write and swap.
//
// "vLLM 原理" §2.1: a block with reference count > 1 is copied before it is
// written, and the writer's table is repointed to the copy;
// "LLM 推理引擎 Continuous Batching 与 PagedAttention" §4.4: blocks are swapped
// out to CPU memory and back.  Both are copies of whole blocks by a list of
// (source, destination) pairs, for K and V; the pools may be the same device
// pool or pinned host memory.
//
// One workgroup per (pair, K or V): 256 threads move the block with 16-byte
// loads and stores, consecutive threads on consecutive bytes, four loads in
// flight per thread before their stores.
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(const uint8_t* __restrict__ src_k,
                                                          const uint8_t* __restrict__ src_v,
                                                          uint8_t* __restrict__ dst_k, uint8_t* __restrict__ dst_v,
                                                          int32_t src_nb, int32_t dst_nb,
                                                          const int32_t* __restrict__ pairs, int64_t block_bytes,
                                                          int32_t* __restrict__ d_err) {
  const int32_t pair = blockIdx.x >> 1;
  const bool is_v = blockIdx.x & 1;
  const int32_t sb = pairs[2 * pair], db = pairs[2 * pair + 1];
  if (sb < 0 || sb >= src_nb || db < 0 || db >= dst_nb) {
    if (threadIdx.x == 0 && !is_v) flag(d_err, PA_DERR_BLOCK_OOB);
    return;
  }
  const uint4* src = reinterpret_cast<const uint4*>((is_v ? src_v : src_k) + sb * block_bytes);
  uint4* dst = reinterpret_cast<uint4*>((is_v ? dst_v : dst_k) + db * block_bytes);
  const int64_t n = block_bytes / 16;
  int64_t i = threadIdx.x;
  for (; i + 3 * kThreads < n; i += 4 * kThreads) {
    const uint4 a = src[i], b = src[i + kThreads], c = src[i + 2 * kThreads], d = src[i + 3 * kThreads];
    dst[i] = a;
    dst[i + kThreads] = b;
    dst[i + 2 * kThreads] = c;
    dst[i + 3 * kThreads] = d;
  }
  for (; i < n; i += kThreads) dst[i] = src[i];
}

}  // namespace

hipError_t launch_copy_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v, int32_t src_nb,
                              int32_t dst_nb, const int32_t* pairs, int32_t num_pairs, int64_t block_bytes,
                              int32_t* d_err, hipStream_t stream) {
  if (num_pairs == 0) return hipSuccess;
  launch_mark("copy_blocks_kernel", stream);
  copy_blocks_kernel<<<static_cast<uint32_t>(2 * num_pairs), kThreads, 0, stream>>>(
      static_cast<const uint8_t*>(src_k), static_cast<const uint8_t*>(src_v), static_cast<uint8_t*>(dst_k),
      static_cast<uint8_t*>(dst_v), src_nb, dst_nb, pairs, block_bytes, d_err);
  launch_done(stream);
  return hipGetLastError();
}

}  // namespace pa

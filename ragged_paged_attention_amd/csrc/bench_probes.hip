// Bandwidth probes (pa_bench.h): ceilings for the attention kernels.
#include <hip/hip_runtime.h>

#include "pa_bench.h"
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ src, int64_t n,
                                                          uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  const u4v* s4 = reinterpret_cast<const u4v*>(src);
  for (; i + 7 * stride < n; i += 8 * stride) {
    u4v v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(s4 + i + u * stride);  // streaming
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0 && acc == 0x9e3779b9u) atomicOr(sink, acc);  // data-dependent, never elided
}

// One wave per (sequence, head, part of <= 48 chunks of 16 tokens); the same
// lane -> (token, 16 bytes) mapping as the decode kernel's K and V loads.
__global__ __launch_bounds__(64) void paged_read_kernel(const uint16_t* __restrict__ k_cache,
                                                        const uint16_t* __restrict__ v_cache,
                                                        const int32_t* __restrict__ block_tables,
                                                        const int32_t* __restrict__ seq_lens, int32_t S,
                                                        int32_t Hkv, int32_t bs, int32_t NB, int32_t MB,
                                                        int32_t P, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x, r = lane & 15, grp = lane >> 4;
  const int32_t item = blockIdx.x;
  const int32_t s = item % S, g = (item / S) % Hkv, part = item / S / Hkv;
  const int32_t L = seq_lens[s];
  const int32_t nchunks = ceil_div(L, 16);
  const int32_t c0 = part * pa::kPartChunks;
  if (c0 >= nchunks || part >= P) return;
  const int32_t c1 = min(nchunks, c0 + pa::kPartChunks);
  const int64_t slot_stride = static_cast<int64_t>(Hkv) * 128;
  const int32_t* bt = block_tables + static_cast<int64_t>(s) * MB;
  const int32_t cpb = bs / 16;
  uint32_t acc = 0;
  for (int32_t c = c0; c < c1; ++c) {
    int32_t b = bt[c / cpb];
    b = (b < 0 || b >= NB) ? 0 : b;
    const int64_t slot0 = static_cast<int64_t>(b) * bs + (c % cpb) * 16;
    const uint16_t* kp = k_cache + (slot0 + r) * slot_stride + g * 128 + 8 * grp;
    const uint16_t* vp = v_cache + (slot0 + grp) * slot_stride + g * 128 + 8 * r;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const uint4 kv = *reinterpret_cast<const uint4*>(kp + 32 * x);
      const uint4 vv = *reinterpret_cast<const uint4*>(vp + 4 * x * slot_stride);
      acc ^= kv.x ^ kv.y ^ kv.z ^ kv.w ^ vv.x ^ vv.y ^ vv.z ^ vv.w;
    }
  }
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if (lane == 0 && acc == 0x9e3779b9u) atomicOr(sink, acc);
}

}  // namespace
}  // namespace pa

extern "C" pa_status_t pa_bench_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink) return PA_ERR_NULL;
  if (bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16) return PA_ERR_SHAPE;
  (void)hipGetLastError();
  const int64_t n = static_cast<int64_t>(bytes / 16);
  int64_t blocks = (n + 2047) / 2048;
  if (blocks > 32768) blocks = 32768;
  if (blocks < 1) blocks = 1;
  pa::stream_read_kernel<<<static_cast<uint32_t>(blocks), 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint4*>(src), n, sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

extern "C" pa_status_t pa_bench_paged_read(const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                           const int32_t* seq_lens, int32_t num_seqs, int32_t num_kv_heads,
                                           int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                                           int32_t max_seq_len, uint32_t* sink, void* stream) {
  if (!k_cache || !v_cache || !block_tables || !seq_lens || !sink) return PA_ERR_NULL;
  if (num_seqs < 1 || num_kv_heads < 1 || block_size % 16 || num_blocks < 1 || max_seq_len < 1)
    return PA_ERR_SHAPE;
  (void)hipGetLastError();
  const int32_t P = (pa::ceil_div(max_seq_len, 16) + pa::kPartChunks - 1) / pa::kPartChunks;
  const int64_t items = static_cast<int64_t>(num_seqs) * num_kv_heads * P;
  pa::paged_read_kernel<<<static_cast<uint32_t>(items), 64, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache), block_tables, seq_lens,
      num_seqs, num_kv_heads, block_size, num_blocks, max_blocks_per_seq, P, sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

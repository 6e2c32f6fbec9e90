// pa_attention_noalloc: pa_attention with the workspace in a static device
// array of the library, for callers that cannot allocate device memory.
//
// The array is a file-scope __device__ object, so each device the library
// runs on holds its own copy (PA_NOALLOC_SCRATCH_BYTES) from the moment this
// code object is loaded on it until the process ends.  In host code the
// array's name is only a host-side stand-in: the device address of the
// current device's copy comes from hipGetSymbolAddress, looked up once per
// device on that device's first call and kept.  Kernels receive that
// address as their workspace, exactly as they receive a caller's workspace
// in pa_attention.  Nothing here allocates or frees.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pa.h"
#include "pa_internal.h"

namespace {

static_assert(PA_NOALLOC_SCRATCH_BYTES % 256 == 0, "whole 256-byte units");
__device__ __align__(256) uint8_t scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
bool g_scratch_done[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's copy of `scratch`.
pa_status_t scratch_lookup(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_done[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return PA_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
    g_scratch_done[dev] = true;
  }
  *ptr = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" pa_status_t pa_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                            const int32_t* block_tables, const int32_t* query_start_loc,
                                            const int32_t* seq_lens, int32_t num_seqs, int32_t num_tokens,
                                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                            int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                                            int32_t max_query_len, int32_t max_seq_len, float scale,
                                            pa_dtype_t dtype, void* out, int32_t* d_err, void* stream) {
  pa::AttnArgs a{q, k_cache, v_cache, block_tables, query_start_loc, seq_lens,
                 num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, block_size,
                 num_blocks, max_blocks_per_seq, max_query_len, max_seq_len, scale, dtype,
                 out, nullptr, 0, d_err};
  const pa::ScratchSource src{static_cast<size_t>(PA_NOALLOC_SCRATCH_BYTES), scratch_lookup};
  return pa::attention_entry(a, &src, static_cast<hipStream_t>(stream));
}

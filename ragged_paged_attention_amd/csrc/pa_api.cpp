// C-ABI layer of libpa: argument validation, path selection, launches.
// Every check here is on host-visible arguments only; nothing waits on the
// device.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "pa.h"
#include "pa_internal.h"

namespace {

// A debugging switch from the environment: set and not "" or "0".
int32_t env_flag(const char* name) {
  const char* v = std::getenv(name);
  return v && v[0] && std::strcmp(v, "0") != 0 ? 1 : 0;
}

std::atomic<int32_t> g_policy{PA_POLICY_AUTO};
std::atomic<int32_t> g_validate{env_flag("PA_VALIDATE")};
std::atomic<int32_t> g_trace{env_flag("PA_TRACE")};
thread_local char g_last_hip_error[256] = "";

// Clears an error left behind by earlier, unrelated HIP calls in this thread,
// so that the check after our launches reports only our own failures.
void clear_stale_error() { (void)hipGetLastError(); }

pa_status_t hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return PA_OK;
  snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s: %s (%d)", where, hipGetErrorString(e),
           static_cast<int>(e));
  return PA_ERR_HIP;
}

bool bad_dtype(pa_dtype_t d) { return d != PA_F32 && d != PA_BF16 && d != PA_F16; }
int64_t elem_bytes(pa_dtype_t d) { return d == PA_F32 ? 4 : 2; }

}  // namespace

namespace pa {

// Argument checks and path selection shared by pa_attention,
// pa_attention_noalloc and pa_write_kv_attention.  scratch: a workspace the
// library owns (its size is a.workspace_bytes); the caller's workspace
// arguments are then not used, and a call that would need more is refused
// with PA_ERR_WORKSPACE before any other HIP call is made.  w: a KV write
// (already checked) that must land before the attention reads the cache.
pa_status_t attention_entry(AttnArgs a, const ScratchSource* scratch, hipStream_t stream, const WriteJob* w) {
  if (bad_dtype(a.dtype)) return PA_ERR_DTYPE;
  if (a.S < 0 || a.T < 0 || a.Hq < 1 || a.Hkv < 1 || a.D < 1 || a.bs < 1 || a.NB < 1 || a.MB < 0)
    return PA_ERR_SHAPE;
  if (a.Hq % a.Hkv != 0) return PA_ERR_SHAPE;
  if (static_cast<int64_t>(a.NB) * a.bs > INT32_MAX) return PA_ERR_SHAPE;
  if (a.Hq > 65535) return PA_ERR_UNSUPPORTED;
  if (a.D > 256) return PA_ERR_UNSUPPORTED;
  if (a.T == 0) return PA_OK;
  if (a.S == 0) return PA_ERR_SHAPE;
  if (a.max_qlen < 1 || a.max_seqlen < 1) return PA_ERR_SHAPE;
  if (!std::isfinite(a.scale)) return PA_ERR_VALUE;
  if (!a.q || !a.k_cache || !a.v_cache || !a.block_tables || !a.qsl || !a.seq_lens || !a.out)
    return PA_ERR_NULL;

  const int32_t policy = g_policy.load();
  const size_t need = fast_workspace_bytes(a.S, a.T, a.Hq, a.Hkv, a.D, a.max_qlen, a.max_seqlen);
  if (scratch) {
    // the workspace is the library's static scratch: check the size first,
    // then look the device's copy up (alignment is checked on its address)
    if (need > scratch->bytes) return PA_ERR_WORKSPACE;
    void* p = nullptr;
    const pa_status_t st = scratch->lookup(&p);
    if (st != PA_OK) return st;
    a.workspace = p;
    a.workspace_bytes = scratch->bytes;
  }
  const bool fast_ok = fast_path_supported(a);
  hipError_t e;
  clear_stale_error();
  if (policy == PA_POLICY_GENERIC || (policy == PA_POLICY_AUTO && !fast_ok)) {
    e = w ? launch_write_kv(w->k, w->v, w->slot_mapping, w->T, w->row_bytes, w->k_cache, w->v_cache, w->num_slots,
                            w->d_err, w->validate, stream)
          : hipSuccess;
    if (e == hipSuccess) e = launch_attn_generic(a, stream);
  } else {
    if (!fast_ok) return PA_ERR_UNSUPPORTED;
    if (need > 0 && (!a.workspace || a.workspace_bytes < need)) return PA_ERR_WORKSPACE;
    e = launch_attn_fast(a, stream, /*side_stream_ok=*/scratch == nullptr, w);
    if (e == hipSuccess && !scratch && g_trace.load()) e = trace_attn_fast(a, stream, w);
    return hip_status(e, "pa_attention");
  }
  if (e == hipSuccess && !scratch && g_trace.load()) trace_attn_generic(a);
  return hip_status(e, "pa_attention");
}

}  // namespace pa

extern "C" {

const char* pa_status_string(pa_status_t s) {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: invalid size argument";
    case PA_ERR_DTYPE: return "PA_ERR_DTYPE: unknown dtype";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: shape or dtype not implemented";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_HIP: return "PA_ERR_HIP: HIP runtime or launch failure";
    case PA_ERR_VALUE: return "PA_ERR_VALUE: invalid argument value";
  }
  return "PA_ERR_UNKNOWN";
}

int32_t pa_version(void) { return 100; }

const char* pa_last_hip_error(void) { return g_last_hip_error; }

int32_t pa_set_validation(int32_t on) {
  if (on != 0 && on != 1) return -1;
  return g_validate.exchange(on);
}

int32_t pa_set_trace(int32_t on) {
  if (on != 0 && on != 1) return -1;
  return g_trace.exchange(on);
}

int32_t pa_set_kernel_policy(int32_t policy) {
  if (policy != PA_POLICY_AUTO && policy != PA_POLICY_GENERIC && policy != PA_POLICY_FAST) return -1;
  return g_policy.exchange(policy);
}

pa_status_t pa_build_metadata(const int32_t* query_lens, const int32_t* seq_lens, int32_t num_seqs,
                              int32_t num_tokens, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, int32_t block_size, int32_t num_blocks,
                              int32_t* query_start_loc, int32_t* seq_start_loc, int32_t* positions,
                              int32_t* token_to_seq, int32_t* slot_mapping, int32_t* stats,
                              int32_t* d_err, void* stream) {
  if (num_seqs < 0 || num_tokens < 0) return PA_ERR_SHAPE;
  if (!query_start_loc || !seq_start_loc) return PA_ERR_NULL;
  if (num_seqs > 0 && (!query_lens || !seq_lens)) return PA_ERR_NULL;
  if (num_tokens > 0 && (!positions || !token_to_seq)) return PA_ERR_NULL;
  if (block_tables) {
    if (max_blocks_per_seq < 0 || block_size < 1 || num_blocks < 1) return PA_ERR_SHAPE;
    if (static_cast<int64_t>(num_blocks) * block_size > INT32_MAX) return PA_ERR_SHAPE;
    if (num_tokens > 0 && !slot_mapping) return PA_ERR_NULL;
  } else {
    slot_mapping = nullptr;
  }
  clear_stale_error();
  hipError_t e = pa::launch_metadata(query_lens, seq_lens, num_seqs, num_tokens, block_tables,
                                     max_blocks_per_seq, block_size, num_blocks, query_start_loc,
                                     seq_start_loc, positions, token_to_seq, slot_mapping, stats, d_err,
                                     static_cast<hipStream_t>(stream));
  return hip_status(e, "pa_build_metadata");
}

pa_status_t pa_write_kv(const void* k, const void* v, const int32_t* slot_mapping, int32_t num_tokens,
                        int32_t num_kv_heads, int32_t head_dim, void* k_cache, void* v_cache,
                        int32_t num_blocks, int32_t block_size, pa_dtype_t dtype, int32_t* d_err,
                        void* stream) {
  if (bad_dtype(dtype)) return PA_ERR_DTYPE;
  if (num_tokens < 0 || num_kv_heads < 1 || head_dim < 1 || num_blocks < 1 || block_size < 1)
    return PA_ERR_SHAPE;
  if (static_cast<int64_t>(num_blocks) * block_size > INT32_MAX) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PA_ERR_NULL;
  const int64_t row_bytes = static_cast<int64_t>(num_kv_heads) * head_dim * elem_bytes(dtype);
  clear_stale_error();
  hipError_t e = pa::launch_write_kv(k, v, slot_mapping, num_tokens, row_bytes, k_cache, v_cache,
                                     static_cast<int64_t>(num_blocks) * block_size, d_err,
                                     g_validate.load() != 0, static_cast<hipStream_t>(stream));
  return hip_status(e, "pa_write_kv");
}

pa_status_t pa_copy_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                           int32_t src_num_blocks, int32_t dst_num_blocks, const int32_t* pairs,
                           int32_t num_pairs, int64_t block_bytes, int32_t* d_err, void* stream) {
  if (num_pairs < 0 || src_num_blocks < 1 || dst_num_blocks < 1 || block_bytes < 16 || block_bytes % 16)
    return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (num_pairs > (INT32_MAX >> 1)) return PA_ERR_SHAPE;
  if (!src_k || !src_v || !dst_k || !dst_v || !pairs) return PA_ERR_NULL;
  const uintptr_t align = reinterpret_cast<uintptr_t>(src_k) | reinterpret_cast<uintptr_t>(src_v) |
                          reinterpret_cast<uintptr_t>(dst_k) | reinterpret_cast<uintptr_t>(dst_v);
  if (align % 16) return PA_ERR_SHAPE;
  clear_stale_error();
  hipError_t e = pa::launch_copy_blocks(src_k, src_v, dst_k, dst_v, src_num_blocks, dst_num_blocks, pairs,
                                        num_pairs, block_bytes, d_err, static_cast<hipStream_t>(stream));
  return hip_status(e, "pa_copy_blocks");
}

size_t pa_attention_workspace_size(int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t max_query_len,
                                   int32_t max_seq_len) {
  if (num_seqs < 0 || num_tokens < 0 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1)
    return 0;
  return pa::fast_workspace_bytes(num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                                  max_query_len, max_seq_len);
}

pa_status_t pa_attention(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* query_start_loc,
                         const int32_t* seq_lens, int32_t num_seqs, int32_t num_tokens,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                         int32_t max_query_len, int32_t max_seq_len, float scale, pa_dtype_t dtype,
                         void* out, void* workspace, size_t workspace_bytes, int32_t* d_err,
                         void* stream) {
  pa::AttnArgs a{q, k_cache, v_cache, block_tables, query_start_loc, seq_lens,
                 num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, block_size,
                 num_blocks, max_blocks_per_seq, max_query_len, max_seq_len, scale, dtype,
                 out, workspace, workspace_bytes, d_err};
  return pa::attention_entry(a, nullptr, static_cast<hipStream_t>(stream));
}

pa_status_t pa_write_kv_attention(const void* k, const void* v, const int32_t* slot_mapping, const void* q,
                                  void* k_cache, void* v_cache, const int32_t* block_tables,
                                  const int32_t* query_start_loc, const int32_t* seq_lens, int32_t num_seqs,
                                  int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                  int32_t max_blocks_per_seq, int32_t max_query_len, int32_t max_seq_len,
                                  float scale, pa_dtype_t dtype, void* out, void* workspace,
                                  size_t workspace_bytes, int32_t* d_err, void* stream) {
  // pa_write_kv's checks first (the attention's follow in attention_entry);
  // nothing is enqueued unless both pass
  if (bad_dtype(dtype)) return PA_ERR_DTYPE;
  if (num_tokens < 0 || num_kv_heads < 1 || head_dim < 1 || num_blocks < 1 || block_size < 1)
    return PA_ERR_SHAPE;
  if (static_cast<int64_t>(num_blocks) * block_size > INT32_MAX) return PA_ERR_SHAPE;
  if (num_tokens > 0 && (!k || !v || !slot_mapping)) return PA_ERR_NULL;
  const pa::WriteJob w{k, v, slot_mapping, num_tokens,
                       static_cast<int64_t>(num_kv_heads) * head_dim * elem_bytes(dtype), k_cache, v_cache,
                       static_cast<int64_t>(num_blocks) * block_size, d_err, g_validate.load() != 0};
  pa::AttnArgs a{q, k_cache, v_cache, block_tables, query_start_loc, seq_lens,
                 num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, block_size,
                 num_blocks, max_blocks_per_seq, max_query_len, max_seq_len, scale, dtype,
                 out, workspace, workspace_bytes, d_err};
  return pa::attention_entry(a, nullptr, static_cast<hipStream_t>(stream), &w);
}

}  // extern "C"

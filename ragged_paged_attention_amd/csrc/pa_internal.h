// Host-side launch interfaces between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// Optional per-kernel timing (pa_bench.h).  launch_mark(name, stream) records
// an event before a launch and launch_done(stream) one after it; both are a
// single branch when timing is off.
void launch_mark(const char* name, hipStream_t stream);
void launch_done(hipStream_t stream);

// metadata.hip
hipError_t launch_metadata(const int32_t* query_lens, const int32_t* seq_lens, int32_t S, int32_t T,
                           const int32_t* block_tables, int32_t MB, int32_t bs, int32_t NB,
                           int32_t* qsl, int32_t* ssl, int32_t* positions, int32_t* token_to_seq,
                           int32_t* slot_mapping, int32_t* stats, int32_t* d_err, hipStream_t stream);

// write_kv.hip
hipError_t launch_write_kv(const void* k, const void* v, const int32_t* slot_mapping, int32_t T,
                           int64_t row_bytes, void* k_cache, void* v_cache, int64_t num_slots,
                           int32_t* d_err, bool validate, hipStream_t stream);

// copy_blocks.hip
hipError_t launch_copy_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v, int32_t src_nb,
                              int32_t dst_nb, const int32_t* pairs, int32_t num_pairs, int64_t block_bytes,
                              int32_t* d_err, hipStream_t stream);

// Shape of one pa_attention call, as the kernels see it.
struct AttnArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* qsl;
  const int32_t* seq_lens;
  int32_t S, T, Hq, Hkv, D, bs, NB, MB, max_qlen, max_seqlen;
  float scale;
  pa_dtype_t dtype;
  void* out;
  void* workspace;
  size_t workspace_bytes;
  int32_t* d_err;
};

// attn_generic.hip: any dtype, head_dim <= 256, any block size, fp32 math.
hipError_t launch_attn_generic(const AttnArgs& a, hipStream_t stream);
// Same kernel, skipping rows of sequences with query_len * (Hq/Hkv) <= skip_rows_le.
hipError_t launch_attn_generic_rows(const AttnArgs& a, int32_t skip_rows_le, hipStream_t stream);

// attn_fast.hip: bf16/f16, head_dim 64/128/256, a block size that is a
// multiple or a divisor of 16, G <= 16, scale > 0, 16-byte aligned buffers.
bool fast_path_supported(const AttnArgs& a);
size_t fast_workspace_bytes(int32_t S, int32_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t max_q,
                            int32_t max_seqlen);
// The KV write of pa_write_kv_attention: what launch_write_kv takes.
struct WriteJob {
  const void* k;
  const void* v;
  const int32_t* slot_mapping;
  int32_t T;
  int64_t row_bytes;
  void* k_cache;
  void* v_cache;
  int64_t num_slots;
  int32_t* d_err;
  bool validate;
};
// The planning launch can take the write as extra workgroups (16-byte rows
// and pointers; without validation, whose check is a launch of its own).
inline bool write_in_plan_ok(const WriteJob& w) {
  const uintptr_t align = reinterpret_cast<uintptr_t>(w.k) | reinterpret_cast<uintptr_t>(w.v) |
                          reinterpret_cast<uintptr_t>(w.k_cache) | reinterpret_cast<uintptr_t>(w.v_cache) |
                          static_cast<uintptr_t>(w.row_bytes);
  return !w.validate && align % 16 == 0;
}
// side_stream_ok: a large mixed batch may run its prefill kernel on the
// library's side stream beside the decode launches (decode_beside_prefill);
// false keeps every launch on `stream`.  A KV write w goes into the planning
// launch when the call has one (write_in_plan_ok), else first on `stream`.
hipError_t launch_attn_fast(const AttnArgs& a, hipStream_t stream, bool side_stream_ok,
                            const WriteJob* w = nullptr);
// A call whose decode launches run beside the prefill kernel (given a side
// stream): prefill rows, head_dim 128, a block size that is a multiple of 16,
// at least kBesideMinSeqs sequences and at most kBesideMaxMeanQuery new
// tokens per sequence on average (many decodes next to a few chunks).
bool decode_beside_prefill(const AttnArgs& a);
constexpr int kBesideMinSeqs = 64;
constexpr int kBesideMaxMeanQuery = 64;
constexpr size_t kBesideLdsPad = 20 << 10;  // prefill launch's extra LDS: 84 KB per workgroup, one per CU
// Plan trace (pa_set_trace): waits for `stream`, then prints the call's work
// split and plan to stderr; the generic path prints its header line only.
hipError_t trace_attn_fast(const AttnArgs& a, hipStream_t stream, const WriteJob* w = nullptr);
void trace_attn_generic(const AttnArgs& a);

// A workspace owned by the library (pa_attention_noalloc): its size, and how
// to find the current device's copy.
struct ScratchSource {
  size_t bytes;
  pa_status_t (*lookup)(void** ptr);
};
// pa_api.cpp: checks, path selection and launches of one attention call;
// w: the KV write to run first (pa_write_kv_attention), or null.
pa_status_t attention_entry(AttnArgs a, const ScratchSource* scratch, hipStream_t stream,
                            const WriteJob* w = nullptr);

// attn_prefill.hip: rows of sequences with query_len * (Hq/Hkv) > min_rows.
// Work plan of one call on the MFMA paths, written to the workspace by the
// planning kernel (attn_prefill.hip) and read by the prefill, decode and merge
// kernels:
//   int32 header[kPlanHeader]   [0] list entries, [1] cascade groups,
//                               [2], [3] one-tile / two-tile decode entries,
//                               [4], [5] chunks per decode part of the
//                               one-tile / two-tile list (plan_parts)
//   int2  entries[cap_entries]  (s >= 0, q-tile): a prefill query tile;
//                               (-(group + 1), part): a part of a cascade
//                               group's shared prefix
//   int4  groups[cap_groups]    (first member-list position, members,
//                               prefix tokens, parts | first prefix slot << 8)
//   int4  seq_prefix[S]         (prefix tokens, parts, first prefix slot, first
//                               row in the group) of the sequence's cascade
//                               group; all 0 if it has none
//   int32 members[S]            cascade members, each group a stretch
//   int2  match[S]              (leader, full blocks shared with it) of a
//                               cascade candidate, written by the matching
//                               kernel before the plan; (-1, 0) otherwise
//   int2  dec[2][S * P]         decode work lists, one-tile then two-tile:
//                               (sequence, part), heaviest part first
// Prefix partials live in their own workspace region: kCascadeEntries slots
// (one per prefix part) x KV heads x kCascadeRows rows x kPartFloats floats.
// Split-K decode: a context of `nchunks` 16-token chunks is cut into parts of
// about part_chunks chunks (kPartChunks, or twice that for a planned list
// that would otherwise need between one and two waves of the launch's wave
// slots), at most P parts (P from max_seq_len, at most kMaxParts), none
// empty.  Equal-sized parts keep the tail of the launch short however uneven
// the context lengths are.  The plan, the decode kernels and the merge call
// the same function with the same part_chunks, so their part ranges agree.
constexpr int kPartChunks = 48;  // default part: at most 48 chunks = 768 tokens
constexpr int kMaxParts = 64;    // parts per sequence (longer parts past 48k tokens)
__host__ __device__ __forceinline__ void plan_parts(int32_t nchunks, int32_t P, int32_t* nparts, int32_t* cpp,
                                                    int32_t part_chunks = kPartChunks) {
  int32_t np = (nchunks + part_chunks - 1) / part_chunks;
  if (np > P) np = P;
  if (np < 1) np = 1;
  int32_t c = (nchunks + np - 1) / np;
  if (c < 1) c = 1;
  *cpp = c;
  *nparts = (nchunks + c - 1) / c;
}

constexpr int kPlanHeader = 64;
constexpr int kPartFloats = 132;       // one split-K partial row: O[128], m (log2 units), l, pad
constexpr int kCascadeMaxParts = 16;   // prefix parts of one group
constexpr int kCascadeEntries = 64;    // prefix parts of one call, over all groups
constexpr int kCascadeRows = 128;      // rows of one group: members x query heads
constexpr int kCascadeMinTiles = 16;   // shortest shared prefix taken, in 64-token tiles
constexpr int kCascadeMaxSeqs = 1024;  // sequences the detection handles (one per plan thread)
struct PlanLayout {
  int32_t cap_entries, cap_groups;
  int64_t cap_dec;                                 // entries of each decode list
  size_t groups_off, seqpre_off, members_off, match_off, dec_off, bytes;  // byte offsets from the plan base; total
};
PlanLayout plan_layout(int32_t S, int32_t T, int32_t G, int32_t P, bool prefill_on, bool cascade_on);
// Shared-prefix (cascade) decode may run in this call: long enough contexts,
// a batch small enough for the detection.
bool cascade_possible(int32_t S, int32_t max_seqlen);
// dec_slots: list entries (each one wave per KV head) that one wave of the
// one-tile and of the two-tile decode launch holds, against which the plan
// sizes each list's parts.  w (may be null; write_in_plan_ok): a KV write
// that the planning launch also does, in workgroups of its own beside the
// planning one.
hipError_t launch_attn_plan(const AttnArgs& a, int32_t rows_cap, int32_t P, bool prefill_on, bool cascade_on,
                            const int32_t dec_slots[2], int32_t* plan, const WriteJob* w, hipStream_t stream);
// Prefill query tiles and cascade prefix parts (their partials go to ws_pre).
// lds_pad: extra dynamic LDS per workgroup (unused by the kernel; it caps
// the workgroups per CU).
hipError_t launch_attn_prefill(const AttnArgs& a, int32_t rows_cap, int32_t P, bool prefill_on, bool cascade_on,
                               const int32_t* plan, float* ws_pre, size_t lds_pad, hipStream_t stream);

}  // namespace pa

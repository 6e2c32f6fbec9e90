// pa_build_metadata kernels.
//
// "vLLM Continuous Batching：从 Forward Shape 理解两个核心参数" §2.1: the flat
// batch is sliced by query_start_loc, a running sum of query_lens with the
// total appended; every new token carries its position inside its sequence;
// §2.3 第一步/第二步: slot = block_table[pos / bs] * bs + pos % bs.
//
// Two parts:
//   scan  — one workgroup walks the S lengths in chunks, producing both offset
//           arrays, the counters and length checks.
//   fill  — one workgroup per sequence writes positions, token_to_seq and
//           slot_mapping for its rows and checks the used part of its
//           block-table row.
// A batch of up to kFusedMaxSeqs sequences takes one launch: workgroup 0
// scans (256 threads) and workgroup 1 + s fills sequence s, first summing the
// query lengths before s itself (at most kFusedMaxSeqs / 256 loads per
// thread), so no workgroup waits for another.  Larger batches take two
// launches, a 1024-thread scan, then the fill grid reading its offsets.
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kScanThreads = 1024;  // the scan launch of larger batches
constexpr int kFillThreads = 256;
constexpr int kFusedMaxSeqs = 1024;  // batches up to this size: one launch

// Inclusive scan of a 64-bit value over a workgroup of kThreads; returns this
// thread's inclusive prefix and writes the workgroup total to *total.
template <int kThreads>
__device__ int64_t block_inclusive_scan(int64_t x, int64_t* lds_waves, int64_t* total) {
  constexpr int kWaves = kThreads / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int off = 1; off < 64; off <<= 1) {
    int64_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) lds_waves[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int64_t w = lane < kWaves ? lds_waves[lane] : 0;
    for (int off = 1; off < kWaves; off <<= 1) {
      int64_t y = __shfl_up(w, off, 64);
      if (lane >= off) w += y;
    }
    if (lane < kWaves) lds_waves[lane] = w;
  }
  __syncthreads();
  int64_t prefix = wave > 0 ? lds_waves[wave - 1] : 0;
  *total = lds_waves[kWaves - 1];
  __syncthreads();
  return x + prefix;
}

// The scan, by a workgroup of kThreads.
template <int kThreads>
__device__ void scan_lengths(const int32_t* __restrict__ query_lens, const int32_t* __restrict__ seq_lens,
                             int32_t S, int32_t T, int32_t* __restrict__ qsl, int32_t* __restrict__ ssl,
                             int32_t* __restrict__ stats, int32_t* __restrict__ d_err) {
  constexpr int kWaves = kThreads / 64;
  __shared__ int64_t lds_q[kWaves];
  __shared__ int64_t lds_s[kWaves];
  int64_t carry_q = 0, carry_s = 0;
  int32_t n_dec = 0, n_pre = 0, dec_tok = 0, pre_tok = 0, max_q = 0, max_s = 0;
  int32_t err = 0;
  for (int32_t base = 0; base < S; base += kThreads) {
    const int32_t idx = base + threadIdx.x;
    int32_t q = 0, L = 0;
    if (idx < S) {
      q = query_lens[idx];
      L = seq_lens[idx];
      if (q < 0 || L < 0 || q > L) err |= PA_DERR_QLEN_GT_SEQLEN;
      q = q < 0 ? 0 : q;
      L = L < 0 ? 0 : L;
      n_dec += (q == 1);
      n_pre += (q > 1);
      dec_tok += (q == 1) ? 1 : 0;
      pre_tok += (q > 1) ? q : 0;
      max_q = max(max_q, q);
      max_s = max(max_s, L);
    }
    int64_t tot_q, tot_s;
    const int64_t iq = block_inclusive_scan<kThreads>(q, lds_q, &tot_q);
    const int64_t is = block_inclusive_scan<kThreads>(L, lds_s, &tot_s);
    if (idx < S) {
      const int64_t vq = carry_q + iq, vs = carry_s + is;
      if (vq > INT32_MAX || vs > INT32_MAX) err |= PA_DERR_OVERFLOW;
      qsl[idx + 1] = static_cast<int32_t>(vq > INT32_MAX ? INT32_MAX : vq);
      ssl[idx + 1] = static_cast<int32_t>(vs > INT32_MAX ? INT32_MAX : vs);
    }
    carry_q += tot_q;
    carry_s += tot_s;
  }
  if (threadIdx.x == 0) {
    qsl[0] = 0;
    ssl[0] = 0;
    if (carry_q != static_cast<int64_t>(T)) err |= PA_DERR_TOKEN_SUM;
  }
  if (err) flag(d_err, err);
  if (stats) {
    // workgroup reduction of the six counters: within each wave by shuffles,
    // then one value per wave through LDS
    int32_t v[6] = {n_dec, n_pre, dec_tok, pre_tok, max_q, max_s};
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] += __shfl_xor(v[c], off, 64);
      v[4] = max(v[4], __shfl_xor(v[4], off, 64));
      v[5] = max(v[5], __shfl_xor(v[5], off, 64));
    }
    __shared__ int32_t lds_red[kWaves][6];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0)
      for (int c = 0; c < 6; ++c) lds_red[wave][c] = v[c];
    __syncthreads();
    if (threadIdx.x < 6) {
      const int c = threadIdx.x;
      int32_t acc = lds_red[0][c];
      for (int w = 1; w < kWaves; ++w) acc = c < 4 ? acc + lds_red[w][c] : max(acc, lds_red[w][c]);
      stats[c] = acc;
    }
  }
}

__global__ __launch_bounds__(kScanThreads) void meta_scan_kernel(
    const int32_t* __restrict__ query_lens, const int32_t* __restrict__ seq_lens, int32_t S, int32_t T,
    int32_t* __restrict__ qsl, int32_t* __restrict__ ssl, int32_t* __restrict__ stats,
    int32_t* __restrict__ d_err) {
  scan_lengths<kScanThreads>(query_lens, seq_lens, S, T, qsl, ssl, stats, d_err);
}

// The fill of sequence s, whose rows start at flat token `start`.
__device__ void fill_sequence(int32_t s, int32_t start, const int32_t* __restrict__ query_lens,
                              const int32_t* __restrict__ seq_lens, int32_t T,
                              const int32_t* __restrict__ block_tables, int32_t MB, int32_t bs, int32_t NB,
                              int32_t* __restrict__ positions, int32_t* __restrict__ token_to_seq,
                              int32_t* __restrict__ slot_mapping, int32_t* __restrict__ d_err) {
  int32_t q = query_lens[s];
  const int32_t L = seq_lens[s];
  q = q < 0 ? 0 : q;
  const int32_t* row = block_tables ? block_tables + static_cast<int64_t>(s) * MB : nullptr;
  int32_t err = 0;
  for (int32_t i = threadIdx.x; i < q; i += blockDim.x) {
    const int64_t t = static_cast<int64_t>(start) + i;
    if (t >= T) {
      err |= PA_DERR_TOKEN_SUM;
      break;
    }
    const int32_t pos = L - q + i;
    positions[t] = pos;
    token_to_seq[t] = s;
    if (slot_mapping) {
      int32_t slot = -1;
      if (pos >= 0) {
        const int32_t lb = pos / bs;
        const int32_t b = lb < MB ? row[lb] : -1;
        if (b >= 0 && b < NB) slot = b * bs + pos % bs;
        else err |= PA_DERR_BLOCK_OOB;
      }
      slot_mapping[t] = slot;
    }
  }
  if (row && L > 0) {
    const int32_t used = ceil_div(L, bs);
    if (used > MB) err |= PA_DERR_BLOCK_OOB;
    const int32_t n = used < MB ? used : MB;
    for (int32_t j = threadIdx.x; j < n; j += blockDim.x) {
      const int32_t b = row[j];
      if (b < 0 || b >= NB) err |= PA_DERR_BLOCK_OOB;
    }
  }
  if (err) flag(d_err, err);
}

__global__ __launch_bounds__(kFillThreads) void meta_fill_kernel(
    const int32_t* __restrict__ query_lens, const int32_t* __restrict__ seq_lens, int32_t S, int32_t T,
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ block_tables, int32_t MB, int32_t bs,
    int32_t NB, int32_t* __restrict__ positions, int32_t* __restrict__ token_to_seq,
    int32_t* __restrict__ slot_mapping, int32_t* __restrict__ d_err) {
  for (int32_t s = blockIdx.x; s < S; s += gridDim.x)
    fill_sequence(s, qsl[s], query_lens, seq_lens, T, block_tables, MB, bs, NB, positions, token_to_seq,
                  slot_mapping, d_err);
}

// One launch for S <= kFusedMaxSeqs: workgroup 0 scans, workgroup 1 + s
// fills sequence s from the sum of the query lengths before it (negative
// ones count as 0, and a sum past INT32_MAX is clamped, as in the scan's
// offsets).
__global__ __launch_bounds__(kFillThreads) void meta_fused_kernel(
    const int32_t* __restrict__ query_lens, const int32_t* __restrict__ seq_lens, int32_t S, int32_t T,
    int32_t* __restrict__ qsl, int32_t* __restrict__ ssl, int32_t* __restrict__ stats,
    const int32_t* __restrict__ block_tables, int32_t MB, int32_t bs, int32_t NB,
    int32_t* __restrict__ positions, int32_t* __restrict__ token_to_seq, int32_t* __restrict__ slot_mapping,
    int32_t* __restrict__ d_err) {
  if (blockIdx.x == 0) {
    scan_lengths<kFillThreads>(query_lens, seq_lens, S, T, qsl, ssl, stats, d_err);
    return;
  }
  __shared__ int64_t lds_w[kFillThreads / 64];
  const int32_t s = static_cast<int32_t>(blockIdx.x) - 1;
  int64_t part = 0;
  for (int32_t i = threadIdx.x; i < s; i += kFillThreads) {
    const int32_t q = query_lens[i];
    part += q < 0 ? 0 : q;
  }
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
  if ((threadIdx.x & 63) == 0) lds_w[threadIdx.x >> 6] = part;
  __syncthreads();
  int64_t start = 0;
#pragma unroll
  for (int w = 0; w < kFillThreads / 64; ++w) start += lds_w[w];
  fill_sequence(s, static_cast<int32_t>(start > INT32_MAX ? INT32_MAX : start), query_lens, seq_lens, T,
                block_tables, MB, bs, NB, positions, token_to_seq, slot_mapping, d_err);
}

}  // namespace

hipError_t launch_metadata(const int32_t* query_lens, const int32_t* seq_lens, int32_t S, int32_t T,
                           const int32_t* block_tables, int32_t MB, int32_t bs, int32_t NB,
                           int32_t* qsl, int32_t* ssl, int32_t* positions, int32_t* token_to_seq,
                           int32_t* slot_mapping, int32_t* stats, int32_t* d_err, hipStream_t stream) {
  if (S <= kFusedMaxSeqs) {
    launch_mark("meta_fused_kernel", stream);
    meta_fused_kernel<<<1 + S, kFillThreads, 0, stream>>>(query_lens, seq_lens, S, T, qsl, ssl, stats,
                                                          block_tables, MB, bs, NB, positions, token_to_seq,
                                                          slot_mapping, d_err);
    launch_done(stream);
    return hipGetLastError();
  }
  launch_mark("meta_scan_kernel", stream);
  meta_scan_kernel<<<1, kScanThreads, 0, stream>>>(query_lens, seq_lens, S, T, qsl, ssl, stats, d_err);
  launch_done(stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int grid = S < 2048 ? S : 2048;
  launch_mark("meta_fill_kernel", stream);
  meta_fill_kernel<<<grid, 256, 0, stream>>>(query_lens, seq_lens, S, T, qsl, block_tables, MB, bs, NB,
                                             positions, token_to_seq, slot_mapping, d_err);
  launch_done(stream);
  return hipGetLastError();
}

}  // namespace pa

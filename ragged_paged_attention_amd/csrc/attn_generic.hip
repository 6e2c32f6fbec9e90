// Generic ragged paged attention: any dtype, head_dim <= 256, any block size.
//
// "vLLM Continuous Batching：从 Forward Shape 理解两个核心参数" §2.3 and
// §2.3补充 第二步: a query row of sequence s at position p reads positions
// 0..p of s through s's block table (logical block j / bs -> physical block,
// offset j % bs) and nothing else.  Online softmax over key chunks follows the
// running-max / rescaled-sum form of "LLM 推理引擎 Continuous Batching 与
// PagedAttention" §3.3.
//
// One wave64 per (flat row t, query head h).  Keys are taken 64 at a time, one
// per lane: each lane forms its key's dot product in fp32 from q staged in
// LDS, the wave agrees on the chunk max, and then all lanes accumulate
// p_j * V[j] over the chunk with lane = head-dim element, so the V reads of one
// key are coalesced across the wave.  This is the correctness path (fp32
// inputs, odd shapes, tiny batches, scale <= 0); the MFMA kernels handle
// bf16/f16 at head_dim 64, 128 and 256 with block sizes that are multiples or
// divisors of 16.
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kMaxD = 256;
constexpr int kPerLane = kMaxD / 64;

// Sequence owning flat row t: the s with qsl[s] <= t < qsl[s+1], found by
// binary search (sequences with query_len 0 own no rows).  Returns -1 when t
// is not covered.
__device__ __forceinline__ int32_t owner_of(const int32_t* qsl, int32_t S, int32_t t) {
  if (S <= 0 || qsl[0] > t || qsl[S] <= t) return -1;
  int32_t lo = 0, hi = S;  // qsl[lo] <= t < qsl[hi]
  while (hi - lo > 1) {
    const int32_t mid = (lo + hi) >> 1;
    if (qsl[mid] <= t) lo = mid;
    else hi = mid;
  }
  return lo;
}

template <class F>
__global__ __launch_bounds__(64) void attn_generic_kernel(
    const typename F::T* __restrict__ q, const typename F::T* __restrict__ k_cache,
    const typename F::T* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ seq_lens, int32_t S, int32_t Hq,
    int32_t Hkv, int32_t D, int32_t bs, int32_t NB, int32_t MB, float scale,
    typename F::T* __restrict__ out, int32_t* __restrict__ d_err, int32_t skip_rows_le, int32_t max_q) {
  using T = typename F::T;
  const int32_t t = blockIdx.x;
  const int32_t h = blockIdx.y;
  const int lane = threadIdx.x;
  __shared__ float qs[kMaxD];

  T* orow = out + (static_cast<int64_t>(t) * Hq + h) * D;
  const int32_t s = owner_of(qsl, S, t);
  int32_t err = 0;
  int32_t qlen = 0, L = 0;
  if (s < 0) {
    err = PA_DERR_TOKEN_SUM;
  } else {
    qlen = qsl[s + 1] - qsl[s];
    // rows of sequences with query_len * G <= skip_rows_le belong to another kernel
    if (qlen * (Hq / Hkv) <= skip_rows_le) return;
    if (qlen > max_q && t == qsl[s] && h == 0 && lane == 0) flag(d_err, PA_DERR_HINT);
    L = seq_lens[s];
    if (L < 0 || qlen > L) err = PA_DERR_QLEN_GT_SEQLEN;
    else if (ceil_div(L, bs) > MB) err = PA_DERR_BLOCK_OOB;
  }
  if (err) {
    if (lane == 0) flag(d_err, err);
    for (int d = lane; d < D; d += 64) orow[d] = F::store(0.f);
    return;
  }
  const int32_t p = L - qlen + (t - qsl[s]);  // last visible position
  const int32_t g = h / (Hq / Hkv);
  const int32_t* bt = block_tables + static_cast<int64_t>(s) * MB;
  const T* qrow = q + (static_cast<int64_t>(t) * Hq + h) * D;
  for (int d = lane; d < D; d += 64) qs[d] = F::load(qrow[d]);
  __syncthreads();

  const int64_t row_elems = static_cast<int64_t>(Hkv) * D;  // one slot, all heads
  float m = -INFINITY, l = 0.f;
  float acc[kPerLane];
#pragma unroll
  for (int r = 0; r < kPerLane; ++r) acc[r] = 0.f;

  for (int32_t j0 = 0; j0 <= p; j0 += 64) {
    const int32_t j = j0 + lane;
    bool valid = j <= p;
    int64_t base = 0;  // element offset of row j, head g
    float x = -INFINITY;
    if (valid) {
      const int32_t b = bt[j / bs];
      if (b < 0 || b >= NB) {
        err |= PA_DERR_BLOCK_OOB;
        valid = false;
      } else {
        base = (static_cast<int64_t>(b) * bs + j % bs) * row_elems + static_cast<int64_t>(g) * D;
        const T* krow = k_cache + base;
        float dot = 0.f;
        for (int d = 0; d < D; ++d) dot = fmaf(qs[d], F::load(krow[d]), dot);
        x = dot * scale;
      }
    }
    const float m_new = fmaxf(m, wave_max(x));
    const float pj = valid ? expf(x - m_new) : 0.f;
    const float alpha = (m == m_new) ? 1.f : expf(m - m_new);
    l = l * alpha + wave_sum(pj);
#pragma unroll
    for (int r = 0; r < kPerLane; ++r) acc[r] *= alpha;
    m = m_new;
    const int32_t n = (p - j0 + 1) < 64 ? (p - j0 + 1) : 64;
    const int32_t base_lo = static_cast<int32_t>(base & 0xffffffff);
    const int32_t base_hi = static_cast<int32_t>(base >> 32);
    for (int32_t kk = 0; kk < n; ++kk) {
      const float pk = __shfl(pj, kk, 64);
      if (pk == 0.f) continue;  // wave-uniform: masked or underflowed key
      const uint32_t lo = static_cast<uint32_t>(__shfl(base_lo, kk, 64));
      const int64_t hi = __shfl(base_hi, kk, 64);
      const T* vrow = v_cache + ((hi << 32) | lo);
#pragma unroll
      for (int r = 0; r < kPerLane; ++r) {
        const int d = lane + 64 * r;
        if (d < D) acc[r] = fmaf(pk, F::load(vrow[d]), acc[r]);
      }
    }
  }
  if (err && lane == 0) flag(d_err, err);
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int r = 0; r < kPerLane; ++r) {
    const int d = lane + 64 * r;
    if (d < D) orow[d] = F::store(acc[r] * inv);
  }
}

}  // namespace

hipError_t launch_attn_generic(const AttnArgs& a, hipStream_t stream) {
  return launch_attn_generic_rows(a, 0, stream);
}

hipError_t launch_attn_generic_rows(const AttnArgs& a, int32_t skip_rows_le, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  const dim3 grid(a.T, a.Hq);
#define PA_GENERIC(F)                                                                              \
  attn_generic_kernel<F><<<grid, 64, 0, stream>>>(                                                 \
      static_cast<const F::T*>(a.q), static_cast<const F::T*>(a.k_cache),                          \
      static_cast<const F::T*>(a.v_cache), a.block_tables, a.qsl, a.seq_lens, a.S, a.Hq, a.Hkv,   \
      a.D, a.bs, a.NB, a.MB, a.scale, static_cast<F::T*>(a.out), a.d_err, skip_rows_le, a.max_qlen)
  launch_mark("attn_generic_kernel", stream);
  switch (a.dtype) {
    case PA_F32: PA_GENERIC(F32); break;
    case PA_BF16: PA_GENERIC(BF16); break;
    case PA_F16: PA_GENERIC(F16); break;
    default: return hipErrorInvalidValue;
  }
  launch_done(stream);
#undef PA_GENERIC
  return hipGetLastError();
}

}  // namespace pa

// MFMA fast paths for pa_attention: bf16/f16 storage, head_dim 128, block
// size a multiple of 16 (so every 16-token chunk lies inside one block).
//
// What is computed is the same as the generic kernel: for each new row of a
// sequence, causal softmax attention over its own cached K/V read through its
// block table ("vLLM Continuous Batching：从 Forward Shape 理解两个核心参数"
// §2.3, §2.3补充 第二步), with the online-softmax running max / rescaled sum of
// "LLM 推理引擎 Continuous Batching 与 PagedAttention" §3.3, and split-K parts
// combined by the same rescaling.
//
// Decode kernel (sequences with query_len * G <= 16, G = Hq / Hkv)
// -----------------------------------------------------------------
// Work item = (sequence s, KV head g, part of the context).  One wave64 per
// item.  All G query heads of the group (times query_len rows) form the 16
// columns of one MFMA tile, so every K/V byte is read once per (s, g):
//   S^T[16 tok][16 rows] = K[16 tok][128] . Q^T[128][16 rows]
//       4 x v_mfma_f32_16x16x32 (A = K rows straight from HBM, 16 B per lane)
//   O^T[128][16 rows]   += V^T[128][16 tok] . P^T[16 tok][16 rows]
//       8 x v_mfma_f32_16x16x16 (B = P^T is exactly the S^T accumulator
//       layout, so P never moves; A = V^T comes from a V tile staged in LDS
//       and read back transposed with ds_read_b64_tr_b16).
// The chunk loop keeps the next chunk's K and V loads in flight while the
// current chunk computes.  Block ids of the part are fetched 64 at a time into
// one VGPR and picked per chunk with readlane.  Work items are remapped so
// that consecutive items (same part and head, consecutive sequences) land on
// the same XCD: sequences that share prefix blocks then hit the same L2.
// A part writes (m, l, O) partials to the workspace; a merge kernel combines
// parts with the rescaling algebra.  A sequence with one part writes out
// directly.
#include "mfma_common.h"
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kPartFloats = 132;    // per partial row: O[128], m, l, pad
constexpr int kMaxRows = 16;        // query rows of one decode item
constexpr int kTargetItems = 8192;  // decode work items wanted to fill 256 CUs
constexpr int kMinChunks = 16;      // do not split contexts below 256 tokens per part

// Split of a context of `nchunks` 16-token chunks into parts: at most P parts,
// none below kMinChunks chunks unless the whole context is, none empty.
__host__ __device__ __forceinline__ void plan_parts(int32_t nchunks, int32_t P, int32_t* nparts,
                                                    int32_t* cpp) {
  int32_t np = (nchunks + kMinChunks - 1) / kMinChunks;
  if (np > P) np = P;
  if (np < 1) np = 1;
  int32_t c = (nchunks + np - 1) / np;
  if (c < 1) c = 1;
  *cpp = c;
  *nparts = (nchunks + c - 1) / c;
}

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_tables;
  const int32_t* qsl;
  const int32_t* seq_lens;
  int32_t S, Hq, Hkv, G, NB, MB, bs, P, n_items;
  float scale_log2e;
  uint16_t* out;
  float* ws;
  int32_t* d_err;
};

template <class F>
__global__ __launch_bounds__(64) void decode_kernel(DecodeArgs a) {
  using M = Mma<F>;
  __shared__ __attribute__((aligned(16))) uint8_t vlds[kChunk * kVRowBytes];
  const int lane = threadIdx.x;
  const int r = lane & 15;    // MFMA column = query row of the item
  const int grp = lane >> 4;  // 16-lane group

  // XCD-aware mapping: workgroup b runs on XCD b % 8; give each XCD a
  // contiguous range of items.
  const int32_t bid = blockIdx.x;
  const int32_t per = a.n_items >> 3, rem = a.n_items & 7, xcd = bid & 7, loc = bid >> 3;
  const int32_t item = xcd * per + (xcd < rem ? xcd : rem) + loc;
  const int32_t s = item % a.S;
  const int32_t tmp = item / a.S;
  const int32_t g = tmp % a.Hkv;
  const int32_t part = tmp / a.Hkv;

  const int32_t q0 = a.qsl[s];
  const int32_t qlen = a.qsl[s + 1] - q0;
  if (qlen <= 0 || qlen * a.G > kMaxRows) return;  // nothing here, or a prefill item
  const int32_t L = a.seq_lens[s];
  const int32_t rows = qlen * a.G;
  const int32_t i_row = r / a.G;
  const int32_t hg = r - i_row * a.G;
  const bool rvalid = r < rows;
  const int32_t t = q0 + i_row;
  const int32_t h = g * a.G + hg;
  uint16_t* orow = a.out + (static_cast<int64_t>(t) * a.Hq + h) * kD;

  if (L < qlen || ceil_div(L, a.bs) > a.MB) {
    if (part == 0) {
      if (lane == 0) flag(a.d_err, L < qlen ? PA_DERR_QLEN_GT_SEQLEN : PA_DERR_BLOCK_OOB);
      if (rvalid)
        for (int d = 4 * grp; d < kD; d += 16) *reinterpret_cast<uint2*>(orow + d) = make_uint2(0, 0);
    }
    return;
  }
  const int32_t nchunks = ceil_div(L, kChunk);
  int32_t np, cpp;
  plan_parts(nchunks, a.P, &np, &cpp);
  if (part >= np) return;
  const int32_t c0 = part * cpp;
  const int32_t c1 = min(nchunks, c0 + cpp);

  // Q^T fragments (B operand): lane holds Q[row r][32kk + 8grp .. +8]
  uint4 qf[4];
  const uint16_t* qrow = a.q + (static_cast<int64_t>(t) * a.Hq + h) * kD + 8 * grp;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) qf[kk] = rvalid ? ld16(qrow + 32 * kk) : make_uint4(0, 0, 0, 0);
  const int32_t qpos = rvalid ? L - qlen + i_row : -1;  // last visible position of this row

  const int64_t slot_stride = static_cast<int64_t>(a.Hkv) * kD;  // elements between slots
  const uint16_t* kbase = a.k_cache + static_cast<int64_t>(g) * kD;
  const uint16_t* vbase = a.v_cache + static_cast<int64_t>(g) * kD;
  const int32_t* btrow = a.block_tables + static_cast<int64_t>(s) * a.MB;
  const int32_t cpb = a.bs / kChunk;  // chunks per block
  const int32_t nblk = ceil_div(L, a.bs);

  // block ids of 64 consecutive logical blocks, one per lane
  int32_t ids_base = -(1 << 30);
  int32_t ids = 0;
  auto slot_of_chunk = [&](int32_t c) -> int64_t {
    const int32_t lb = c / cpb;
    if (lb - ids_base >= 64 || lb < ids_base) {
      ids_base = lb;
      int32_t v = (lb + lane < nblk) ? btrow[lb + lane] : 0;
      if (v < 0 || v >= a.NB) {
        flag(a.d_err, PA_DERR_BLOCK_OOB);
        v = 0;
      }
      ids = v;
    }
    const int32_t b = __builtin_amdgcn_readlane(ids, lb - ids_base);
    return static_cast<int64_t>(b) * a.bs + (c - lb * cpb) * kChunk;
  };

  uint4 kf[4], vf[4];
  auto load_chunk = [&](int32_t c) {
    const int64_t slot0 = slot_of_chunk(c);
    const uint16_t* kp = kbase + (slot0 + r) * slot_stride + 8 * grp;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) kf[kk] = ld16(kp + 32 * kk);
    const uint16_t* vp = vbase + (slot0 + grp) * slot_stride + 8 * r;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) vf[r4] = ld16(vp + 4 * r4 * slot_stride);
  };

  float m = -INFINITY, lsum = 0.f;
  f32x4_t o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  load_chunk(c0);
  for (int32_t c = c0; c < c1; ++c) {
    uint4 kc[4], vc[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      kc[x] = kf[x];
      vc[x] = vf[x];
    }
    if (c + 1 < c1) load_chunk(c + 1);
    const int32_t tok0 = c * kChunk;

    // scores: S^T[tok 4grp + j][row r]
    f32x4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) st = M::qk(kc[kk], qf[kk], st);
    float x[4];
    const int32_t tb = tok0 + 4 * grp;
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = (tb + j <= qpos) ? st[j] * a.scale_log2e : -INFINITY;
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = xor_max(mx, 16);
    mx = xor_max(mx, 32);
    const float m_new = fmaxf(m, mx);
    float p[4];
    float alpha = 1.f;
    if (m_new == -INFINITY) {
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = 0.f;
    } else {
      alpha = __builtin_amdgcn_exp2f(m - m_new);
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = __builtin_amdgcn_exp2f(x[j] - m_new);
    }
    m = m_new;
    lsum = lsum * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    if (__any(alpha != 1.f)) {  // wave-uniform: skip the rescale when no row's max moved
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
    }
    i16x4_t pb;
#pragma unroll
    for (int j = 0; j < 4; ++j) pb[j] = static_cast<short>(M::cvt(p[j]));

    // stage V (rows past the context are zeroed: garbage there could be NaN)
    if (tok0 + kChunk > L) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        if (tok0 + 4 * r4 + grp >= L) vc[r4] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      *reinterpret_cast<uint4*>(vlds + (4 * r4 + grp) * kVRowBytes + 16 * r) = vc[r4];
    __asm__ volatile("" ::: "memory");
    // A = V^T: lane r of group grp gets V[4grp + j][16dt + r] (j = 0..3)
    const int rd_off = (4 * grp + (r >> 2)) * kVRowBytes + 8 * (r & 3);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const i16x4_t va = lds_read_tr16(vlds + rd_off + 32 * dt);
      o[dt] = M::pv(va, pb, o[dt]);
    }
    __asm__ volatile("" ::: "memory");
  }

  lsum = xor_sum(lsum, 16);
  lsum = xor_sum(lsum, 32);
  if (np == 1) {
    if (rvalid) {
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        uint2 w;
        w.x = static_cast<uint32_t>(M::cvt(o[dt][0] * inv)) | (static_cast<uint32_t>(M::cvt(o[dt][1] * inv)) << 16);
        w.y = static_cast<uint32_t>(M::cvt(o[dt][2] * inv)) | (static_cast<uint32_t>(M::cvt(o[dt][3] * inv)) << 16);
        *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * grp) = w;
      }
    }
  } else if (rvalid) {
    float* e = a.ws + ((static_cast<int64_t>(s) * a.Hkv + g) * a.P + part) * (kMaxRows * kPartFloats) +
               r * kPartFloats;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<float4*>(e + 16 * dt + 4 * grp) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    if (grp == 0) {
      e[kD] = m;
      e[kD + 1] = lsum;
    }
  }
}

// Combine the parts of every split decode item: with m = max_p m_p,
//   o = sum_p 2^(m_p - m) O_p / sum_p 2^(m_p - m) l_p.
template <class F>
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a) {
  const int32_t s = blockIdx.x, g = blockIdx.y;
  const int32_t q0 = a.qsl[s];
  const int32_t qlen = a.qsl[s + 1] - q0;
  if (qlen <= 0 || qlen * a.G > kMaxRows) return;
  const int32_t L = a.seq_lens[s];
  if (L < qlen || ceil_div(L, a.bs) > a.MB) return;
  int32_t np, cpp;
  plan_parts(ceil_div(L, kChunk), a.P, &np, &cpp);
  if (np == 1) return;
  const int32_t rows = qlen * a.G;
  const float* base = a.ws + (static_cast<int64_t>(s) * a.Hkv + g) * a.P * (kMaxRows * kPartFloats);
  for (int idx = threadIdx.x; idx < rows * kD; idx += blockDim.x) {
    const int r = idx / kD, d = idx - r * kD;
    float mm = -INFINITY;
    for (int p = 0; p < np; ++p) mm = fmaxf(mm, base[(p * kMaxRows + r) * kPartFloats + kD]);
    float num = 0.f, den = 0.f;
    if (mm != -INFINITY) {
      for (int p = 0; p < np; ++p) {
        const float* e = base + (p * kMaxRows + r) * kPartFloats;
        const float w = __builtin_amdgcn_exp2f(e[kD] - mm);
        num = fmaf(w, e[d], num);
        den = fmaf(w, e[kD + 1], den);
      }
    }
    const int32_t i_row = r / a.G, hg = r - i_row * a.G;
    const int64_t t = q0 + i_row;
    a.out[(t * a.Hq + g * a.G + hg) * kD + d] = Mma<F>::cvt(den > 0.f ? num / den : 0.f);
  }
}

int32_t decode_parts(int32_t S, int32_t Hkv, int32_t max_seqlen) {
  const int64_t units = static_cast<int64_t>(S) * Hkv;
  int64_t P = (kTargetItems + units - 1) / (units > 0 ? units : 1);
  const int64_t max_useful = (ceil_div(max_seqlen > 0 ? max_seqlen : 1, kChunk) + kMinChunks - 1) / kMinChunks;
  if (P > max_useful) P = max_useful;
  if (P < 1) P = 1;
  if (P > 64) P = 64;
  return static_cast<int32_t>(P);
}

}  // namespace

bool fast_path_supported(const AttnArgs& a) {
  return (a.dtype == PA_BF16 || a.dtype == PA_F16) && a.D == kD && a.bs % kChunk == 0 &&
         a.Hq / a.Hkv <= kMaxRows;
}

size_t fast_workspace_bytes(int32_t S, int32_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t max_seqlen) {
  (void)T;
  (void)Hq;
  if (D != kD) return 0;
  const int32_t P = decode_parts(S, Hkv, max_seqlen);
  if (P <= 1) return 0;
  return static_cast<size_t>(S) * Hkv * P * kMaxRows * kPartFloats * sizeof(float);
}

hipError_t launch_attn_fast(const AttnArgs& a, hipStream_t stream) {
  DecodeArgs d;
  d.q = static_cast<const uint16_t*>(a.q);
  d.k_cache = static_cast<const uint16_t*>(a.k_cache);
  d.v_cache = static_cast<const uint16_t*>(a.v_cache);
  d.block_tables = a.block_tables;
  d.qsl = a.qsl;
  d.seq_lens = a.seq_lens;
  d.S = a.S;
  d.Hq = a.Hq;
  d.Hkv = a.Hkv;
  d.G = a.Hq / a.Hkv;
  d.NB = a.NB;
  d.MB = a.MB;
  d.bs = a.bs;
  d.P = decode_parts(a.S, a.Hkv, a.max_seqlen);
  d.scale_log2e = a.scale * 1.4426950408889634f;
  d.out = static_cast<uint16_t*>(a.out);
  d.ws = static_cast<float*>(a.workspace);
  d.d_err = a.d_err;
  const int64_t items = static_cast<int64_t>(a.S) * a.Hkv * d.P;
  if (items > INT32_MAX) return hipErrorInvalidValue;
  d.n_items = static_cast<int32_t>(items);

  // prefill-class rows (query_len * G > 16): MFMA prefill kernel
  hipError_t e = launch_attn_prefill(a, kMaxRows, stream);
  if (e != hipSuccess) return e;
  if (a.dtype == PA_BF16) {
    decode_kernel<BF16><<<d.n_items, 64, 0, stream>>>(d);
    if (d.P > 1) merge_kernel<BF16><<<dim3(a.S, a.Hkv), 256, 0, stream>>>(d);
  } else {
    decode_kernel<F16><<<d.n_items, 64, 0, stream>>>(d);
    if (d.P > 1) merge_kernel<F16><<<dim3(a.S, a.Hkv), 256, 0, stream>>>(d);
  }
  return hipGetLastError();
}

}  // namespace pa

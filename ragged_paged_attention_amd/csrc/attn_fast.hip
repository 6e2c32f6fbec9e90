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
// Compile-time tuning of the decode work split (measured on MI355X).
constexpr int kPartChunks = 48;     // a context part is at most 48 chunks = 768 tokens
constexpr int kMaxParts = 64;       // parts per sequence (longer parts past 48k tokens)
constexpr int kXcdRun = 16;         // consecutive decode items kept on one XCD
constexpr int kGroupHeadsBelow = 16;  // item order: head-grouped when Hkv < this

// Split of a context of `nchunks` 16-token chunks into parts of about
// kPartChunks chunks: at most P parts, none empty.  Equal-sized parts keep the
// tail of the launch short however uneven the context lengths are.
__host__ __device__ __forceinline__ void plan_parts(int32_t nchunks, int32_t P, int32_t* nparts,
                                                    int32_t* cpp) {
  int32_t np = (nchunks + kPartChunks - 1) / kPartChunks;
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
  int32_t S, Hq, Hkv, G, NB, MB, bs, P, n_items, grouped;
  float scale_log2e;
  uint16_t* out;
  float* ws;
  int32_t* d_err;
};

template <class F>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3, 8))) void decode_kernel(DecodeArgs a) {
  using M = Mma<F>;
  __shared__ __attribute__((aligned(16))) uint8_t vlds[2 * kChunk * kVRowBytes];
  const int lane = threadIdx.x;
  const int r = lane & 15;    // MFMA column = query row of the item
  const int grp = lane >> 4;  // 16-lane group

  // XCD-aware mapping: workgroup b runs on XCD b % 8.  Items go out in runs of
  // kXcdRun consecutive items per XCD, the runs rotating over the 8 XCDs: every
  // XCD gets an even share of every part index (balance), and a run of
  // neighbouring items lives on one XCD's L2.  The grid is a multiple of
  // 8 * kXcdRun.
  const int32_t bid = blockIdx.x;
  const int32_t xcd = bid & 7, j = bid >> 3;
  const int32_t item = ((j / kXcdRun) * 8 + xcd) * kXcdRun + (j % kXcdRun);
  if (item >= a.n_items) return;
  // item = (part, sequence, KV head), head fastest: the Hkv waves reading the
  // same token rows (all heads of a slot are one contiguous row of the cache)
  // run side by side.
  int32_t s, g, part;
  if (a.grouped) {
    // (part, block of kXcdRun sequences, head, sequence in block): a run is the
    // same (part, head) of kXcdRun neighbouring sequences on one XCD (shared
    // prefix blocks stay in its L2); the runs in flight on the other XCDs are
    // the other heads of the same sequences, so each token row -- all heads of
    // a slot, contiguous -- is read by all heads at about the same time.
    const int32_t si = item % kXcdRun;
    const int32_t tmp = item / kXcdRun;
    g = tmp % a.Hkv;
    const int32_t tmp2 = tmp / a.Hkv;
    const int32_t sblocks = (a.S + kXcdRun - 1) / kXcdRun;
    s = (tmp2 % sblocks) * kXcdRun + si;
    part = tmp2 / sblocks;
    if (s >= a.S) return;
  } else {
    // (part, head, sequence): with many KV heads a token row is long, and
    // spreading the concurrent reads over many sequences' randomly placed
    // blocks keeps more HBM channels busy than reading whole rows at once.
    s = item % a.S;
    const int32_t tmp = item / a.S;
    g = tmp % a.Hkv;
    part = tmp / a.Hkv;
  }

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

  // Chunks are taken two at a time (32 tokens, 16 KB of K+V per wave in
  // flight).  One register buffer per pair: the next pair's K loads are issued
  // as soon as the QK MFMAs have read the current K, the next V loads as soon
  // as the current V is in LDS.  A pair's second chunk may lie past the part
  // (odd chunk counts): it is then neither loaded nor counted.
  uint4 kf[2][4], vf[2][4];
  // K/V read once are streamed past the caches (6.0 vs 5.6 TB/s measured on
  // the decode batch).  A part whose first block is also mapped by a
  // neighbouring sequence (a shared prefix) keeps cacheable loads, so the
  // sequences sharing it hit in L2.
  bool stream = true;
  if (a.grouped) {
    const int32_t lb0 = c0 / cpb;
    const int32_t mine = btrow[lb0];
    bool shared = false;
    if (s > 0) shared |= a.block_tables[static_cast<int64_t>(s - 1) * a.MB + lb0] == mine;
    if (s + 1 < a.S) shared |= a.block_tables[static_cast<int64_t>(s + 1) * a.MB + lb0] == mine;
    stream = !shared;
  }
  auto load_pair = [&](int32_t c, bool do_k, bool do_v) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      if (c + h2 < c1) {
        const int64_t slot0 = slot_of_chunk(c + h2);
        if (do_k) {
          const uint16_t* kp = kbase + (slot0 + r) * slot_stride + 8 * grp;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) kf[h2][kk] = stream ? ld16_nt(kp + 32 * kk) : ld16(kp + 32 * kk);
        }
        if (do_v) {
          const uint16_t* vp = vbase + (slot0 + grp) * slot_stride + 8 * r;
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4)
            vf[h2][r4] = stream ? ld16_nt(vp + 4 * r4 * slot_stride) : ld16(vp + 4 * r4 * slot_stride);
        }
      } else {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          if (do_k) kf[h2][x] = make_uint4(0, 0, 0, 0);
          if (do_v) vf[h2][x] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  };

  float m = -INFINITY, lsum = 0.f;
  f32x4_t o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  load_pair(c0, true, true);
  const int rd_off = (4 * grp + (r >> 2)) * kVRowBytes + 8 * (r & 3);
  for (int32_t c = c0; c < c1; c += 2) {
    const int32_t tok0 = c * kChunk;
    const bool more = c + 2 < c1;

    // scores: S^T[tok0 + 16 h2 + 4grp + j][row r]
    f32x4_t st[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) st[h2] = M::qk(kf[h2][kk], qf[kk], st[h2]);
    if (more) load_pair(c + 2, true, false);

    // stage V; rows past the context or the part are zeroed (unwritten slots
    // may hold NaN, and the second chunk may not have been loaded)
    const int32_t tok_end = min(L, c1 * kChunk);
    if (tok0 + 2 * kChunk > tok_end) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          if (tok0 + 16 * h2 + 4 * r4 + grp >= tok_end) vf[h2][r4] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<uint4*>(vlds + (16 * h2 + 4 * r4 + grp) * kVRowBytes + 16 * r) = vf[h2][r4];
    __asm__ volatile("" ::: "memory");
    if (more) load_pair(c + 2, false, true);

    float x[2][4];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int32_t tb = tok0 + 16 * h2 + 4 * grp;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        x[h2][j] = (tb + j <= qpos && tb + j < tok_end) ? st[h2][j] * a.scale_log2e : -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                     fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
    mx = group_max4(mx);
    const float m_new = fmaxf(m, mx);
    float p[2][4];
    float alpha = 1.f;
    if (m_new == -INFINITY) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int j = 0; j < 4; ++j) p[h2][j] = 0.f;
    } else {
      alpha = __builtin_amdgcn_exp2f(m - m_new);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int j = 0; j < 4; ++j) p[h2][j] = __builtin_amdgcn_exp2f(x[h2][j] - m_new);
    }
    m = m_new;
    lsum = lsum * alpha + (((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) + ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3])));
    if (__any(alpha != 1.f)) {  // wave-uniform: skip the rescale when no row's max moved
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
    }
    // B = P^T for 32 tokens: k = 8grp + j holds token 4grp + j (j < 4) and
    // 16 + 4grp + (j - 4); A = V^T uses the same token order.
    const uint4 pb = make_uint4(M::pk(p[0][0], p[0][1]), M::pk(p[0][2], p[0][3]),
                                M::pk(p[1][0], p[1][1]), M::pk(p[1][2], p[1][3]));
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const i16x4_t lo = lds_read_tr16(vlds + rd_off + 32 * dt);
      const i16x4_t hi = lds_read_tr16(vlds + rd_off + 16 * kVRowBytes + 32 * dt);
      const uint4 va = __builtin_bit_cast(uint4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      o[dt] = M::qk(va, pb, o[dt]);
    }
    __asm__ volatile("" ::: "memory");
  }

  lsum = group_sum4(lsum);
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
// One workgroup per (sequence, KV head); the per-(row, part) weights are
// computed once into LDS, then each thread produces output elements.
template <class F>
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a) {
  __shared__ float wts[kMaxRows][kMaxParts];
  __shared__ float inv_den[kMaxRows];
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
  if (threadIdx.x < rows) {
    const int r = threadIdx.x;
    float mm = -INFINITY;
    for (int p = 0; p < np; ++p) mm = fmaxf(mm, base[(p * kMaxRows + r) * kPartFloats + kD]);
    float den = 0.f;
    for (int p = 0; p < np; ++p) {
      const float* e = base + (p * kMaxRows + r) * kPartFloats;
      const float w = mm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(e[kD] - mm);
      wts[r][p] = w;
      den = fmaf(w, e[kD + 1], den);
    }
    inv_den[r] = den > 0.f ? 1.f / den : 0.f;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < rows * kD; idx += blockDim.x) {
    const int r = idx / kD, d = idx - r * kD;
    float num = 0.f;
    for (int p = 0; p < np; ++p) num = fmaf(wts[r][p], base[(p * kMaxRows + r) * kPartFloats + d], num);
    const int32_t i_row = r / a.G, hg = r - i_row * a.G;
    const int64_t t = q0 + i_row;
    a.out[(t * a.Hq + g * a.G + hg) * kD + d] = Mma<F>::cvt(num * inv_den[r]);
  }
}

// Parts per sequence the launch provides for: enough for max_seq_len.  A
// longer sequence than the hint still works (its parts just get longer).
int32_t decode_parts(int32_t S, int32_t Hkv, int32_t max_seqlen) {
  (void)S;
  (void)Hkv;
  int32_t P = (ceil_div(max_seqlen > 0 ? max_seqlen : 1, kChunk) + kPartChunks - 1) / kPartChunks;
  if (P < 1) P = 1;
  if (P > kMaxParts) P = kMaxParts;
  return P;
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
  d.grouped = a.Hkv < kGroupHeadsBelow ? 1 : 0;
  const int64_t s_pad = d.grouped ? (a.S + kXcdRun - 1) / kXcdRun * kXcdRun : a.S;
  const int64_t items = s_pad * a.Hkv * d.P;
  const int64_t grid = (items + 8 * kXcdRun - 1) / (8 * kXcdRun) * (8 * kXcdRun);
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  d.n_items = static_cast<int32_t>(items);

  // prefill-class rows (query_len * G > 16): MFMA prefill kernel
  hipError_t e = launch_attn_prefill(a, kMaxRows, stream);
  if (e != hipSuccess) return e;
  launch_mark("decode_kernel", stream);
  if (a.dtype == PA_BF16) decode_kernel<BF16><<<static_cast<uint32_t>(grid), 64, 0, stream>>>(d);
  else decode_kernel<F16><<<static_cast<uint32_t>(grid), 64, 0, stream>>>(d);
  launch_done(stream);
  if (d.P > 1) {
    launch_mark("merge_kernel", stream);
    if (a.dtype == PA_BF16) merge_kernel<BF16><<<dim3(a.S, a.Hkv), 256, 0, stream>>>(d);
    else merge_kernel<F16><<<dim3(a.S, a.Hkv), 256, 0, stream>>>(d);
    launch_done(stream);
  }
  return hipGetLastError();
}

}  // namespace pa

// MFMA fast paths for pa_attention: bf16/f16 storage, head_dim 64, 128 or
// 256, and a block size that is a multiple of 16 (a 16-token chunk lies
// inside one block) or divides 16 (each lane finds its own token's block);
// query tiles of longer chunks go to the prefill kernel (attn_prefill.hip).
//
// What is computed is the same as the generic kernel: for each new row of a
// sequence, causal softmax attention over its own cached K/V read through its
// block table ("vLLM Continuous Batching：从 Forward Shape 理解两个核心参数"
// §2.3, §2.3补充 第二步), with the online-softmax running max / rescaled sum of
// "LLM 推理引擎 Continuous Batching 与 PagedAttention" §3.3, and split-K parts
// combined by the same rescaling.
//
// Decode kernel (sequences with query_len * G <= 32, G = Hq / Hkv)
// -----------------------------------------------------------------
// Work item = (sequence s, KV head g, part of the context).  One wave64 per
// item.  All G query heads of the group (times query_len rows) form the
// columns of one or two 16-column MFMA tiles (NT = 1 for up to 16 rows, NT = 2
// for 17..32: a verify step of a few draft tokens), so every K/V byte is read
// once per (s, g) whatever the row count:
//   S^T[16 tok][16 rows] = K[16 tok][D] . Q^T[D][16 rows]
//       D/32 x v_mfma_f32_16x16x32 (A = K rows straight from HBM, 16 B per lane)
//   O^T[D][16 rows]     += V^T[D][32 tok] . P^T[32 tok][16 rows]
//       D/16 x v_mfma_f32_16x16x32 per 32 tokens (B = P^T is exactly the S^T
//       accumulator layout, so P never moves; A = V^T comes from a V tile
//       staged in LDS and read back transposed with ds_read_b64_tr_b16).
// The chunk loop keeps the next chunk's K and V loads in flight while the
// current chunk computes.  Block ids of the part are fetched 64 at a time into
// one VGPR and picked per chunk with readlane.  Work items are remapped so
// that consecutive items (same part and head, consecutive sequences) land on
// the same XCD: sequences that share prefix blocks then hit the same L2.
// A part writes (m, l, O) partials to the workspace; a merge kernel combines
// parts with the rescaling algebra.  A sequence with one part writes out
// directly.
#include <algorithm>
#include <cstdio>
#include <mutex>
#include <vector>

#include "mfma_common.h"
#include "pa_common.h"
#include "pa_internal.h"


namespace pa {
namespace {

constexpr int kTileRows = 16;       // query rows per MFMA column tile
constexpr int kMaxRows = 32;        // query rows of one decode item (two tiles)
// Compile-time tuning of the decode work order (measured on MI355X); the
// part split (kPartChunks, plan_parts) is in pa_internal.h.
constexpr int kXcdRun = 16;         // consecutive decode items kept on one XCD
constexpr int kSimds = 1024;        // 256 CUs x 4 SIMDs
constexpr int kGroupHeadsBelow = 16;  // item order: head-grouped when Hkv < this

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_tables;
  const int32_t* qsl;
  const int32_t* seq_lens;
  int32_t S, Hq, Hkv, G, NB, MB, bs, P, n_items, grouped;
  int32_t rows_cap;    // 16 or 32: larger items go to the prefill kernel
  const int4* seq_prefix;  // cascade prefix of each sequence (layout in pa_internal.h); null without cascade
  const float* ws_pre;     // cascade prefix partials
  int32_t prefill_on;  // the prefill kernel runs in this call
  int32_t max_q;       // the caller's max_query_len hint
  // Decode work lists of the plan (one-tile, two-tile items; null without a
  // plan): entries (sequence, part), heaviest first; counts in dec_n[0..1],
  // chunks per part of each list in dec_n[2..3].
  const int2* dec_list[2];
  const int32_t* dec_n;
  float scale_log2e;
  uint16_t* out;
  float* ws;
  int32_t* d_err;
};

// NT = row tiles: the instance with NT tiles takes items with
// 16 (NT - 1) < rows <= 16 NT.  The one-tile instance also checks the
// max_query_len hint and zero-fills the rows of items no kernel of this call
// covers (rows above rows_cap while the prefill kernel does not run).
// D = head_dim (64, 128, 256).  kBlk16: the block size is a multiple of 16;
// otherwise it divides 16 and each lane looks up its own token's block.
// Waves per SIMD the register budget is set for: the pair-buffered K/V
// fragments and the O accumulators of head_dim 256 need about twice the
// registers (and head_dim 256 items take one row tile only).
template <int NT, int D, bool kBeside>
constexpr int decode_min_waves() {
  return kBeside || D == 256 ? 1 : (NT == 1 ? 3 : 2);
}

// kBeside: the instance that runs beside the prefill kernel on a mixed batch
// (launch_attn_fast): each of its waves holds more than half of a SIMD's
// registers (168 VGPRs and AGPRs up to a100, 272 in all), so at most one of
// them sits on a SIMD, next to one prefill wave (208 registers); the two
// kernels then share every CU at a fixed split (one prefill workgroup and
// four decode waves) instead of taking each other's slots as they free up.
template <class F, int NT, int D, bool kBlk16, bool kBeside = false>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(decode_min_waves<NT, D, kBeside>(), 8))) void decode_kernel(
    DecodeArgs a) {
  if constexpr (kBeside) __asm__ volatile("" ::: "a100");  // register footprint only; no instruction
  using M = Mma<F>;
  constexpr int kKK = D / 32;       // 16x16x32 K steps of QK; also V loads per 16-row chunk
  constexpr int kDT = D / 16;       // 16-wide output tiles of PV
  constexpr int kVRow = 2 * D + 32;  // LDS row pitch of the staged V tile (32 B of padding)
  constexpr int kLpr = D / 8;       // lanes per V row in a load (16 B each)
  constexpr int kRpi = 64 / kLpr;   // V rows per load instruction
  constexpr int kPF = D + 4;        // floats of one partial row: O[D], m, l, pad
  __shared__ __attribute__((aligned(16))) uint8_t vlds[2 * kChunk * kVRow];
  const int lane = threadIdx.x;
  const int r = lane & 15;    // MFMA column = query row of the item (within its tile)
  const int grp = lane >> 4;  // 16-lane group

  // XCD-aware mapping: workgroup b runs on XCD b % 8.  Items go out in runs of
  // kXcdRun consecutive items per XCD (a run of neighbouring items lives on
  // one XCD's L2).  The k-th run an XCD takes is run 8k + ((xcd + k) mod 8):
  // the XCD of a run moves on every block of 8 runs, so no stride in the item
  // order (a layer of S x Hkv items, say, when S is a multiple of 128) can pin
  // a sequence or a head to one XCD and leave the XCDs' loads uneven.  The
  // grid is a multiple of 8 * kXcdRun.
  const int32_t bid = blockIdx.x;
  int32_t s, g, part;
  if (a.dec_list[0]) {
    // the plan's list in XCD runs: (block of kXcdRun entries, KV head, entry
    // in block), the k-th run an XCD takes being run 8k + ((xcd + k) mod 8).
    // Entries are the real (sequence, part) items of this instance, heaviest
    // first, so neighbouring entries weigh about the same and the grid's empty
    // workgroups all come after the real ones (measured against the mapping
    // below on the mixed batch: decode 419 -> 389 us; verify batch 0.51 ->
    // 0.46 ms; ordering the list head-fastest instead of in runs was slower
    // than either)
    const int32_t xcd = bid & 7, j = bid >> 3;
    const int32_t k = j / kXcdRun;
    const int32_t item = (k * 8 + ((xcd + k) & 7)) * kXcdRun + (j % kXcdRun);
    const int32_t tmp = item / kXcdRun;
    g = tmp % a.Hkv;
    const int32_t e = (tmp / a.Hkv) * kXcdRun + item % kXcdRun;
    if (e >= a.dec_n[NT - 1]) return;
    const int2 en = a.dec_list[NT - 1][e];
    s = en.x;
    part = en.y;
  } else {
  const int32_t xcd = bid & 7, j = bid >> 3;
  const int32_t k = j / kXcdRun;
  const int32_t item = (k * 8 + ((xcd + k) & 7)) * kXcdRun + (j % kXcdRun);
  if (item >= a.n_items) return;
  // item = (part, sequence, KV head), head fastest: the Hkv waves reading the
  // same token rows (all heads of a slot are one contiguous row of the cache)
  // run side by side.
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
  }

  const int32_t q0 = a.qsl[s];
  const int32_t qlen = a.qsl[s + 1] - q0;
  if (qlen <= 0) return;
  const int32_t rows = qlen * a.G;
  if (NT == 1 && part == 0) {
    if (qlen > a.max_q && g == 0 && lane == 0) flag(a.d_err, PA_DERR_HINT);
    if (rows > a.rows_cap && !a.prefill_on) {  // not covered by this call: zeros
      for (int32_t idx = lane; idx < rows * (D / 4); idx += 64) {
        const int32_t rr = idx / (D / 4), d4 = idx - rr * (D / 4);
        const int32_t tt = q0 + rr / a.G, hh = g * a.G + rr % a.G;
        *reinterpret_cast<uint2*>(a.out + (static_cast<int64_t>(tt) * a.Hq + hh) * D + 4 * d4) = make_uint2(0, 0);
      }
      return;
    }
  }
  if (rows <= kTileRows * (NT - 1) || rows > kTileRows * NT || rows > a.rows_cap) return;  // another kernel's
  const int32_t L = a.seq_lens[s];
  // per tile: this lane's query row, its flat row and head, its output row
  int32_t rt_row[NT], qpos[NT];
  bool rvalid[NT];
  uint16_t* orow[NT];
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    rt_row[rt] = kTileRows * rt + r;
    const int32_t i_row = rt_row[rt] / a.G;
    const int32_t hg = rt_row[rt] - i_row * a.G;
    rvalid[rt] = rt_row[rt] < rows;
    orow[rt] = a.out + (static_cast<int64_t>(q0 + i_row) * a.Hq + g * a.G + hg) * D;
    qpos[rt] = rvalid[rt] ? L - qlen + i_row : -1;  // last visible position of this row
  }

  if (L < qlen || ceil_div(L, a.bs) > a.MB) {
    if (part == 0) {
      if (lane == 0) flag(a.d_err, L < qlen ? PA_DERR_QLEN_GT_SEQLEN : PA_DERR_BLOCK_OOB);
#pragma unroll
      for (int rt = 0; rt < NT; ++rt)
        if (rvalid[rt])
          for (int d = 4 * grp; d < D; d += 16) *reinterpret_cast<uint2*>(orow[rt] + d) = make_uint2(0, 0);
    }
    return;
  }
  // A cascade member reads only its own suffix: the shared prefix is done once
  // for its group by the prefill kernel, which leaves npp partials for the
  // merge.
  int32_t pre = 0, npp = 0;
  if (a.seq_prefix) {
    const int4 sp = a.seq_prefix[s];
    pre = sp.x;
    npp = sp.y;
  }
  const int32_t nchunks = ceil_div(L, kChunk);
  const int32_t cbeg = pre / kChunk;
  int32_t np, cpp;
  plan_parts(nchunks - cbeg, a.P, &np, &cpp, a.dec_list[0] ? a.dec_n[2 + NT - 1] : kPartChunks);
  if (part >= np) return;
  const int32_t c0 = cbeg + part * cpp;
  const int32_t c1 = min(nchunks, c0 + cpp);

  // Q^T fragments (B operand): lane holds Q[row][32kk + 8grp .. +8] of its
  // row in each tile (the q row sits at the same offset as the output row)
  uint4 qf[NT][kKK];
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    const uint16_t* qrow = a.q + (orow[rt] - a.out) + 8 * grp;
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) qf[rt][kk] = rvalid[rt] ? ld16(qrow + 32 * kk) : make_uint4(0, 0, 0, 0);
  }

  const int64_t slot_stride = static_cast<int64_t>(a.Hkv) * D;  // elements between slots
  const uint16_t* kbase = a.k_cache + static_cast<int64_t>(g) * D;
  const uint16_t* vbase = a.v_cache + static_cast<int64_t>(g) * D;
  const int32_t* btrow = a.block_tables + static_cast<int64_t>(s) * a.MB;
  const int32_t nblk = ceil_div(L, a.bs);

  // block ids of 64 consecutive logical blocks, one per lane
  int32_t ids_base = -(1 << 30);
  int32_t ids = 0;
  auto fetch_ids = [&](int32_t lb) {  // wave-uniform lb
    ids_base = lb;
    int32_t v = (lb + lane < nblk) ? btrow[lb + lane] : 0;
    if (v < 0 || v >= a.NB) {
      flag(a.d_err, PA_DERR_BLOCK_OOB);
      v = 0;
    }
    ids = v;
  };
  // kBlk16: first slot of 16-token chunk c (the chunk lies in one block)
  auto slot_of_chunk = [&](int32_t c) -> int64_t {
    const int32_t cpb = a.bs / kChunk;  // chunks per block
    const int32_t lb = c / cpb;
    if (lb - ids_base >= 64 || lb < ids_base) fetch_ids(lb);
    const int32_t b = __builtin_amdgcn_readlane(ids, lb - ids_base);
    return static_cast<int64_t>(b) * a.bs + (c - lb * cpb) * kChunk;
  };
  // !kBlk16: make the id window cover chunks c, c + 1 (32 tokens, at most 32
  // blocks), then each lane's slot of token t of that range
  auto window_for = [&](int32_t c) {
    const int32_t lb0 = (c * kChunk) / a.bs, lb1 = (c * kChunk + 2 * kChunk - 1) / a.bs;
    if (lb0 < ids_base || lb1 - ids_base >= 64) fetch_ids(lb0);
  };
  auto slot_of_token = [&](int32_t t) -> int64_t {
    const int32_t lb = t / a.bs;
    const int32_t b = __shfl(ids, lb - ids_base, 64);
    return static_cast<int64_t>(b) * a.bs + (t - lb * a.bs);
  };

  // Chunks are taken two at a time (32 tokens, 16 KB of K+V per wave in
  // flight).  One register buffer per pair: the next pair's K loads are issued
  // as soon as the QK MFMAs have read the current K, the next V loads as soon
  // as the current V is in LDS.  A pair's second chunk may lie past the part
  // (odd chunk counts): it is then neither loaded nor counted.
  uint4 kf[2][kKK], vf[2][kKK];
  // K/V read once are streamed past the caches (6.0 vs 5.6 TB/s measured on
  // the decode batch).  A part whose first block is also mapped by a
  // neighbouring sequence (a shared prefix) keeps cacheable loads, so the
  // sequences sharing it hit in L2.
  bool stream = true;
  {
    const int32_t lb0 = (c0 * kChunk) / a.bs;
    const int32_t mine = btrow[lb0];
    bool shared = false;
    if (s > 0) shared |= a.block_tables[static_cast<int64_t>(s - 1) * a.MB + lb0] == mine;
    if (s + 1 < a.S) shared |= a.block_tables[static_cast<int64_t>(s + 1) * a.MB + lb0] == mine;
    stream = !shared;
  }
  // K: lane holds row r of the chunk, columns 32 kk + 8 grp .. + 8.  V: load
  // r4 brings rows kRpi r4 + vrow, columns 8 vcol .. + 8.
  const int vrow = lane / kLpr, vcol = lane % kLpr;
  auto load_pair = [&](int32_t c, bool do_k, bool do_v) {
    if (!kBlk16) window_for(c);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      if (c + h2 < c1) {
        const int32_t tok = (c + h2) * kChunk;
        const int64_t slot0 = kBlk16 ? slot_of_chunk(c + h2) : 0;
        if (do_k) {
          const int64_t sl = kBlk16 ? slot0 + r : slot_of_token(tok + r);
          const uint16_t* kp = kbase + sl * slot_stride + 8 * grp;
#pragma unroll
          for (int kk = 0; kk < kKK; ++kk) kf[h2][kk] = stream ? ld16_nt(kp + 32 * kk) : ld16(kp + 32 * kk);
        }
        if (do_v) {
#pragma unroll
          for (int r4 = 0; r4 < kKK; ++r4) {
            const int32_t row = kRpi * r4 + vrow;
            const int64_t sl = kBlk16 ? slot0 + row : slot_of_token(tok + row);
            const uint16_t* vp = vbase + sl * slot_stride + 8 * vcol;
            vf[h2][r4] = stream ? ld16_nt(vp) : ld16(vp);
          }
        }
      } else {
#pragma unroll
        for (int x = 0; x < kKK; ++x) {
          if (do_k) kf[h2][x] = make_uint4(0, 0, 0, 0);
          if (do_v) vf[h2][x] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  };

  float m[NT], lsum[NT];
  f32x4_t o[NT][kDT];
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    m[rt] = -INFINITY;
    lsum[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) o[rt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  load_pair(c0, true, true);
  const int rd_off = (4 * grp + (r >> 2)) * kVRow + 8 * (r & 3);
  for (int32_t c = c0; c < c1; c += 2) {
    const int32_t tok0 = c * kChunk;
    const bool more = c + 2 < c1;

    // scores: S^T[tok0 + 16 h2 + 4grp + j][row r of tile rt]
    f32x4_t st[NT][2];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) st[rt][0] = st[rt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) st[rt][h2] = M::qk(kf[h2][kk], qf[rt][kk], st[rt][h2]);
    if (more) load_pair(c + 2, true, false);

    // stage V; rows past the context or the part are zeroed (unwritten slots
    // may hold NaN, and the second chunk may not have been loaded)
    const int32_t tok_end = min(L, c1 * kChunk);
    if (tok0 + 2 * kChunk > tok_end) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int r4 = 0; r4 < kKK; ++r4)
          if (tok0 + 16 * h2 + kRpi * r4 + vrow >= tok_end) vf[h2][r4] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int r4 = 0; r4 < kKK; ++r4)
        *reinterpret_cast<uint4*>(vlds + (16 * h2 + kRpi * r4 + vrow) * kVRow + 16 * vcol) = vf[h2][r4];
    __asm__ volatile("" ::: "memory");
    if (more) load_pair(c + 2, false, true);

    uint4 pb[NT];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      float x[2][4];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int32_t tb = tok0 + 16 * h2 + 4 * grp;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          x[h2][j] = (tb + j <= qpos[rt] && tb + j < tok_end) ? st[rt][h2][j] * a.scale_log2e : -INFINITY;
      }
      float mx = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                       fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
      mx = group_max4(mx);
      const float m_new = fmaxf(m[rt], mx);
      float p[2][4];
      float alpha = 1.f;
      if (m_new == -INFINITY) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int j = 0; j < 4; ++j) p[h2][j] = 0.f;
      } else {
        alpha = __builtin_amdgcn_exp2f(m[rt] - m_new);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int j = 0; j < 4; ++j) p[h2][j] = __builtin_amdgcn_exp2f(x[h2][j] - m_new);
      }
      m[rt] = m_new;
      lsum[rt] = lsum[rt] * alpha +
                 (((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) + ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3])));
      if (__any(alpha != 1.f)) {  // wave-uniform: skip the rescale when no row's max moved
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) o[rt][dt] *= alpha;
      }
      // B = P^T for 32 tokens: k = 8grp + j holds token 4grp + j (j < 4) and
      // 16 + 4grp + (j - 4); A = V^T uses the same token order.
      pb[rt] = make_uint4(M::pk(p[0][0], p[0][1]), M::pk(p[0][2], p[0][3]), M::pk(p[1][0], p[1][1]),
                          M::pk(p[1][2], p[1][3]));
    }
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) {
      const i16x4_t lo = lds_read_tr16(vlds + rd_off + 32 * dt);
      const i16x4_t hi = lds_read_tr16(vlds + rd_off + 16 * kVRow + 32 * dt);
      const uint4 va = __builtin_bit_cast(uint4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) o[rt][dt] = M::qk(va, pb[rt], o[rt][dt]);
    }
    __asm__ volatile("" ::: "memory");
  }

#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    const float ls = group_sum4(lsum[rt]);
    if (!rvalid[rt]) continue;
    if (np == 1 && npp == 0) {
      const float inv = ls > 0.f ? 1.f / ls : 0.f;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) {
        uint2 w;
        w.x = static_cast<uint32_t>(M::cvt(o[rt][dt][0] * inv)) |
              (static_cast<uint32_t>(M::cvt(o[rt][dt][1] * inv)) << 16);
        w.y = static_cast<uint32_t>(M::cvt(o[rt][dt][2] * inv)) |
              (static_cast<uint32_t>(M::cvt(o[rt][dt][3] * inv)) << 16);
        *reinterpret_cast<uint2*>(orow[rt] + 16 * dt + 4 * grp) = w;
      }
    } else {
      float* e = a.ws + ((static_cast<int64_t>(s) * a.Hkv + g) * a.P + part) * (a.rows_cap * kPF) +
                 rt_row[rt] * kPF;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt)
        *reinterpret_cast<float4*>(e + 16 * dt + 4 * grp) =
            make_float4(o[rt][dt][0], o[rt][dt][1], o[rt][dt][2], o[rt][dt][3]);
      if (grp == 0) {
        e[D] = m[rt];
        e[D + 1] = ls;
      }
    }
  }
}

// Combine the parts of every split decode item: with m = max_p m_p,
//   o = sum_p 2^(m_p - m) O_p / sum_p 2^(m_p - m) l_p.
// One workgroup per (sequence, KV head, slice of kMergeRows rows).  Each wave
// first forms the part weights of two rows (lane = part, one load each, wave
// reductions) into LDS; then every thread produces four consecutive outputs
// of one row from float4 partial loads, several parts in flight at once.
constexpr int kMergeRows = 8;  // rows per merge workgroup (256 threads = 8 rows x 32 float4)

template <class F, int D>
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a) {
  constexpr int kMaxMerge = kMaxParts + kCascadeMaxParts;  // decode parts + cascade prefix parts
  constexpr int kPF = D + 4;  // floats of one decode partial row
  __shared__ float wts[kMergeRows][kMaxMerge];
  __shared__ float inv_den[kMergeRows];
  const int32_t s = blockIdx.x, g = blockIdx.y;
  const int32_t r0 = blockIdx.z * kMergeRows;
  const int32_t q0 = a.qsl[s];
  const int32_t qlen = a.qsl[s + 1] - q0;
  const int32_t rows = qlen * a.G;
  if (qlen <= 0 || rows > a.rows_cap || r0 >= rows) return;
  const int32_t L = a.seq_lens[s];
  if (L < qlen || ceil_div(L, a.bs) > a.MB) return;
  int32_t pre = 0, npp = 0, pslot = 0, prow = 0;
  if (a.seq_prefix) {
    const int4 sp = a.seq_prefix[s];
    pre = sp.x;
    npp = sp.y;
    pslot = sp.z;
    prow = sp.w;
  }
  int32_t np, cpp;
  plan_parts(ceil_div(L, kChunk) - pre / kChunk, a.P, &np, &cpp,
             a.dec_list[0] ? a.dec_n[2 + (rows > kTileRows ? 1 : 0)] : kPartChunks);
  if (np == 1 && npp == 0) return;  // written directly by the decode kernel
  const int32_t ntot = np + npp;
  const int32_t stride = a.rows_cap * kPF;  // one decode part's partials
  const float* base = a.ws + (static_cast<int64_t>(s) * a.Hkv + g) * a.P * stride;
  // partial row r of the k-th part: decode parts 0..np-1, then the group's
  // prefix parts (slot pslot + j, this sequence's rows from prow; head_dim
  // 128 only)
  auto part_row = [&](int32_t k, int32_t r) -> const float* {
    return k < np ? base + k * stride + r * kPF
                  : a.ws_pre + ((static_cast<int64_t>(pslot + k - np) * a.Hkv + g) * kCascadeRows + prow + r) *
                                   kPartFloats;
  };
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    const int rl = 2 * wave + k2;  // row within the slice
    const int32_t r = r0 + rl;
    if (r >= rows) break;          // wave-uniform
    float mp[2], lp[2], mm = -INFINITY;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int32_t k = 64 * c + lane;
      const float* e = k < ntot ? part_row(k, r) : nullptr;
      mp[c] = k < ntot ? e[D] : -INFINITY;
      lp[c] = k < ntot ? e[D + 1] : 0.f;
      mm = fmaxf(mm, mp[c]);
    }
    mm = wave_max(mm);
    float den = 0.f;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int32_t k = 64 * c + lane;
      const float w = (k < ntot && mm != -INFINITY) ? __builtin_amdgcn_exp2f(mp[c] - mm) : 0.f;
      if (k < kMaxMerge) wts[rl][k] = w;
      den += w * lp[c];
    }
    den = wave_sum(den);
    if (lane == 0) inv_den[rl] = den > 0.f ? 1.f / den : 0.f;
  }
  __syncthreads();
  const int rl = threadIdx.x >> 5;
  const int32_t r = r0 + rl;
  if (r >= rows) return;
  const float inv = inv_den[rl];
  const int32_t i_row = r / a.G, hg = r - i_row * a.G;
  // 32 threads per row, D / 4 float4 columns
  for (int d4 = threadIdx.x & 31; d4 < D / 4; d4 += 32) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    int32_t k = 0;
    for (; k + 4 <= ntot; k += 4) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const float4*>(part_row(k + u, r) + 4 * d4);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float wu = wts[rl][k + u];
        acc.x = fmaf(wu, v[u].x, acc.x);
        acc.y = fmaf(wu, v[u].y, acc.y);
        acc.z = fmaf(wu, v[u].z, acc.z);
        acc.w = fmaf(wu, v[u].w, acc.w);
      }
    }
    for (; k < ntot; ++k) {
      const float4 v = *reinterpret_cast<const float4*>(part_row(k, r) + 4 * d4);
      const float wu = wts[rl][k];
      acc.x = fmaf(wu, v.x, acc.x);
      acc.y = fmaf(wu, v.y, acc.y);
      acc.z = fmaf(wu, v.z, acc.z);
      acc.w = fmaf(wu, v.w, acc.w);
    }
    uint2 o;
    o.x = static_cast<uint32_t>(Mma<F>::cvt(acc.x * inv)) | (static_cast<uint32_t>(Mma<F>::cvt(acc.y * inv)) << 16);
    o.y = static_cast<uint32_t>(Mma<F>::cvt(acc.z * inv)) | (static_cast<uint32_t>(Mma<F>::cvt(acc.w * inv)) << 16);
    *reinterpret_cast<uint2*>(a.out + ((static_cast<int64_t>(q0) + i_row) * a.Hq + g * a.G + hg) * D + 4 * d4) = o;
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
  // 16-byte vector loads and stores of q, the caches, out and the workspace
  const uintptr_t align = reinterpret_cast<uintptr_t>(a.q) | reinterpret_cast<uintptr_t>(a.k_cache) |
                          reinterpret_cast<uintptr_t>(a.v_cache) | reinterpret_cast<uintptr_t>(a.out) |
                          reinterpret_cast<uintptr_t>(a.workspace);
  // scale > 0: the prefill kernel takes a tile's row maximum on the raw
  // scores and scales it afterwards, which needs a positive scale
  return (a.dtype == PA_BF16 || a.dtype == PA_F16) && (a.D == 64 || a.D == 128 || a.D == 256) && a.scale > 0.f &&
         (a.bs % kChunk == 0 || kChunk % a.bs == 0) && a.Hq / a.Hkv <= kTileRows && align % 16 == 0;
}

// Rows of the largest item the decode kernels take in a call: two tiles when
// the max_query_len hint allows items of more than one tile (head_dim 256:
// always one), else one.
static int32_t decode_rows_cap(int32_t G, int32_t max_q, int32_t D) {
  return D != 256 && static_cast<int64_t>(max_q) * G > kTileRows ? kMaxRows : kTileRows;
}

// Work split of one call, from the sizes and hints alone (the same numbers
// give the workspace size and the launches).
// prefill_on: rows above rows_cap may come (the prefill kernel takes them);
// mfma_prefill: the planned MFMA prefill kernel runs (prefill query tiles or
// cascade prefix parts).
struct FastPlan {
  int32_t G, P, rows_cap;
  bool prefill_on, cascade_on, mfma_prefill;
  size_t dec_bytes, pre_off, plan_off, bytes;
};

static FastPlan fast_plan(int32_t S, int32_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t max_q,
                          int32_t max_seqlen) {
  FastPlan f;
  f.G = Hq / Hkv;
  f.P = decode_parts(S, Hkv, max_seqlen);
  f.rows_cap = decode_rows_cap(f.G, max_q, D);
  f.prefill_on = static_cast<int64_t>(max_q) * f.G > f.rows_cap;
  f.cascade_on = D == kD && cascade_possible(S, max_seqlen);
  f.mfma_prefill = f.prefill_on || f.cascade_on;
  // Workspace: split-K partials of the decode kernels (when a context can take
  // more than one part, or a cascade prefix makes even one part a partial),
  // the cascade prefix partials, then the work plan, each 256-byte aligned.
  const size_t align = 255;
  f.dec_bytes = (f.P > 1 || f.cascade_on)
                    ? (static_cast<size_t>(S) * Hkv * f.P * f.rows_cap * (D + 4) * sizeof(float) + align) & ~align
                    : 0;
  f.pre_off = f.dec_bytes;
  f.plan_off = f.pre_off + (f.cascade_on ? (static_cast<size_t>(kCascadeEntries) * Hkv * kCascadeRows * kPartFloats *
                                                    sizeof(float) + align) & ~align
                                         : 0);
  f.bytes = f.plan_off + (f.mfma_prefill ? plan_layout(S, T, f.G, f.P, f.prefill_on, f.cascade_on).bytes : 0);
  return f;
}

size_t fast_workspace_bytes(int32_t S, int32_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t max_q,
                            int32_t max_seqlen) {
  if ((D != 64 && D != 128 && D != 256) || Hkv < 1 || Hq % Hkv) return 0;
  return fast_plan(S, T, Hq, Hkv, D, max_q, max_seqlen).bytes;
}

// One decode launch for the call's head_dim and block-size class.  beside:
// the one-tile head_dim-128 instance that runs next to the prefill kernel.
template <class F, int NT>
static void launch_decode(const DecodeArgs& d, int32_t D, bool blk16, uint32_t grid, hipStream_t stream,
                          bool beside = false) {
  if constexpr (NT == 1) {
    if (beside) {
      decode_kernel<F, 1, 128, true, true><<<grid, 64, 0, stream>>>(d);
      return;
    }
  }
#define PA_DECODE_D(DD)                                                          \
  if (blk16) decode_kernel<F, NT, DD, true><<<grid, 64, 0, stream>>>(d);        \
  else decode_kernel<F, NT, DD, false><<<grid, 64, 0, stream>>>(d);
  if (D == 64) {
    PA_DECODE_D(64)
  } else if (D == 128) {
    PA_DECODE_D(128)
  } else if constexpr (NT == 1) {
    PA_DECODE_D(256)
  }
#undef PA_DECODE_D
}

template <class F>
static void launch_merge(const DecodeArgs& d, int32_t D, dim3 grid, hipStream_t stream) {
  if (D == 64) merge_kernel<F, 64><<<grid, 256, 0, stream>>>(d);
  else if (D == 256) merge_kernel<F, 256><<<grid, 256, 0, stream>>>(d);
  else merge_kernel<F, 128><<<grid, 256, 0, stream>>>(d);
}

// A side stream per device for the prefill kernel of a large mixed batch,
// which runs beside the decode launches (launch_attn_fast).  Created on first
// use, default priority, never destroyed; the fork and join events are
// recorded and waited on under one lock, so concurrent calls cannot
// interleave them.
namespace {
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool ok = false, tried = false;
};
constexpr int kMaxDevices = 64;
SideStream g_side[kMaxDevices];
std::mutex g_side_mu;

SideStream* side_stream_locked() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  SideStream& ss = g_side[dev];
  if (!ss.tried) {
    ss.tried = true;
    ss.ok = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) == hipSuccess &&
            hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) == hipSuccess &&
            hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) == hipSuccess;
  }
  return ss.ok ? &ss : nullptr;
}
}  // namespace

bool decode_beside_prefill(const AttnArgs& a) {
  const FastPlan f = fast_plan(a.S, a.T, a.Hq, a.Hkv, a.D, a.max_qlen, a.max_seqlen);
  return f.prefill_on && a.D == kD && a.bs % kChunk == 0 && a.S >= kBesideMinSeqs &&
         static_cast<int64_t>(a.T) <= static_cast<int64_t>(kBesideMaxMeanQuery) * a.S;
}

hipError_t launch_attn_fast(const AttnArgs& a, hipStream_t stream, bool side_stream_ok, const WriteJob* w) {
  const FastPlan f = fast_plan(a.S, a.T, a.Hq, a.Hkv, a.D, a.max_qlen, a.max_seqlen);
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
  d.G = f.G;
  d.NB = a.NB;
  d.MB = a.MB;
  d.bs = a.bs;
  d.P = f.P;
  d.rows_cap = f.rows_cap;
  d.prefill_on = f.prefill_on ? 1 : 0;
  d.max_q = a.max_qlen;
  d.scale_log2e = a.scale * 1.4426950408889634f;
  d.out = static_cast<uint16_t*>(a.out);
  d.ws = static_cast<float*>(a.workspace);
  d.d_err = a.d_err;
  d.grouped = a.Hkv < kGroupHeadsBelow ? 1 : 0;
  d.seq_prefix = nullptr;
  d.dec_list[0] = d.dec_list[1] = nullptr;
  d.dec_n = nullptr;
  d.ws_pre = reinterpret_cast<const float*>(static_cast<const uint8_t*>(a.workspace) + f.pre_off);
  const int64_t s_pad = d.grouped ? (a.S + kXcdRun - 1) / kXcdRun * kXcdRun : a.S;
  const int64_t items = s_pad * a.Hkv * d.P;
  // with the plan's lists: whole blocks of kXcdRun entries for every head
  const int64_t list_items = (static_cast<int64_t>(a.S) * d.P + kXcdRun - 1) / kXcdRun * kXcdRun * a.Hkv;
  const int64_t grid_items = f.mfma_prefill ? std::max(items, list_items) : items;
  const int64_t grid = (grid_items + 8 * kXcdRun - 1) / (8 * kXcdRun) * (8 * kXcdRun);
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  d.n_items = static_cast<int32_t>(items);

  // A large mixed batch (many decode sequences next to a few prefill
  // chunks) runs its decode launches and its prefill kernel side by side,
  // the prefill kernel on a side stream: the prefill kernel takes one
  // workgroup per CU (its launch asks
  // for kBesideLdsPad more bytes of LDS) and the decode kernel one wave per
  // SIMD (its kBeside instance), so the HBM-bound decode and the MFMA-bound
  // prefill share every CU (mixed batch: 0.715 -> 0.68 ms per step; the same
  // two launches side by side without the split: 0.721 ms, the decode waves
  // taking every slot a prefill workgroup frees).  Other calls run their
  // launches one after the other on `stream`.
  const bool beside = side_stream_ok && decode_beside_prefill(a);
  // A KV write that comes with the call (pa_write_kv_attention) goes into the
  // planning launch as workgroups of its own: planning reads only lengths and
  // block tables, and everything that reads the cache follows that launch.
  // (On the side stream beside the planning launches instead, the two event
  // waits it needs cost as much as the overlap gained: mixed batch 0.677 ms
  // per step either way.)  Without a plan it goes first on `stream`.
  const bool write_in_plan = w && f.mfma_prefill && write_in_plan_ok(*w);
  if (w && !write_in_plan) {
    const hipError_t e = launch_write_kv(w->k, w->v, w->slot_mapping, w->T, w->row_bytes, w->k_cache, w->v_cache,
                                         w->num_slots, w->d_err, w->validate, stream);
    if (e != hipSuccess) return e;
  }
  std::unique_lock<std::mutex> side_lock(g_side_mu, std::defer_lock);
  SideStream* ss = nullptr;
  if (beside) {
    side_lock.lock();
    ss = side_stream_locked();
  }
  SideStream* side = nullptr;  // the side stream when the prefill kernel runs on it
  const hipStream_t ds = stream;  // the one-tile decode launch's stream
  if (f.mfma_prefill) {
    int32_t* plan = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(a.workspace) + f.plan_off);
    // list entries one wave of each decode launch holds: waves per SIMD x
    // 1024 SIMDs, one wave per KV head of an entry
    const int32_t dec_slots[2] = {kSimds * (beside || a.D == 256 ? 1 : 3) / a.Hkv, kSimds * 2 / a.Hkv};
    hipError_t e = launch_attn_plan(a, f.rows_cap, f.P, f.prefill_on, f.cascade_on, dec_slots, plan,
                                    write_in_plan ? w : nullptr, stream);
    if (e != hipSuccess) return e;
    // Beside the decode launches the prefill kernel runs on the side stream,
    // behind the planning launch (and the write in it); the one-tile decode
    // launch, the longer of the two chains, starts on `stream` without the
    // wait for the fork.
    hipStream_t ps = stream;  // the prefill kernel's stream
    if (beside && ss) {
      if (hipEventRecord(ss->fork, stream) == hipSuccess && hipStreamWaitEvent(ss->s, ss->fork, 0) == hipSuccess) {
        side = ss;
        ps = ss->s;
      }
    }
    e = launch_attn_prefill(a, f.rows_cap, f.P, f.prefill_on, f.cascade_on, plan,
                            reinterpret_cast<float*>(static_cast<uint8_t*>(a.workspace) + f.pre_off),
                            side ? kBesideLdsPad : 0, ps);
    if (e != hipSuccess) {
      if (side) {  // rejoin, so `stream` still orders after the side stream
        (void)hipEventRecord(side->join, side->s);
        (void)hipStreamWaitEvent(stream, side->join, 0);
      }
      return e;
    }
    const PlanLayout l = plan_layout(a.S, a.T, f.G, f.P, f.prefill_on, f.cascade_on);
    if (f.cascade_on) d.seq_prefix = reinterpret_cast<const int4*>(reinterpret_cast<const uint8_t*>(plan) + l.seqpre_off);
    const int2* dec = reinterpret_cast<const int2*>(reinterpret_cast<const uint8_t*>(plan) + l.dec_off);
    d.dec_list[0] = dec;
    d.dec_list[1] = dec + l.cap_dec;
    d.dec_n = plan + 2;
  }
  // The one-tile and two-tile instances one after the other.  Running the
  // two-tile launch on a second stream beside the one-tile launch (both
  // HBM-bound, each filling the machine only partly) measured slower once the
  // plan's sorted work lists were in place: verify batch 0.459 ms side by
  // side, 0.437 ms one after the other (either order).
  const bool blk16 = a.bs % kChunk == 0;
  launch_mark("decode_kernel", ds);
  if (a.dtype == PA_BF16) launch_decode<BF16, 1>(d, a.D, blk16, static_cast<uint32_t>(grid), ds, side != nullptr);
  else launch_decode<F16, 1>(d, a.D, blk16, static_cast<uint32_t>(grid), ds, side != nullptr);
  launch_done(ds);
  if (d.rows_cap > kTileRows) {
    // Beside the prefill kernel the two-tile launch follows it on the side
    // stream.  With the prefill waves at a higher issue priority the prefill
    // chain is the shorter one, and it takes the (often empty) two-tile
    // launch: mixed step 0.662 -> 0.654 ms (the move alone, at equal
    // priorities: 0.668 ms).  The one-tile launch, now the longer chain,
    // stays on `stream` and starts without the wait for the fork (cold
    // median 0.626-0.629 -> 0.620-0.625 ms).
    const hipStream_t ds2 = side ? side->s : ds;
    launch_mark("decode_kernel_2t", ds2);
    if (a.dtype == PA_BF16) launch_decode<BF16, 2>(d, a.D, blk16, static_cast<uint32_t>(grid), ds2);
    else launch_decode<F16, 2>(d, a.D, blk16, static_cast<uint32_t>(grid), ds2);
    launch_done(ds2);
  }
  if (side) {  // join: the merge and everything after it wait for the side stream's launches
    hipError_t e = hipEventRecord(side->join, side->s);
    if (e == hipSuccess) e = hipStreamWaitEvent(stream, side->join, 0);
    side_lock.unlock();
    if (e != hipSuccess) return e;
  }
  if (d.P > 1 || f.cascade_on) {
    launch_mark("merge_kernel", stream);
    const dim3 mgrid(a.S, a.Hkv, d.rows_cap / kMergeRows);
    if (a.dtype == PA_BF16) launch_merge<BF16>(d, a.D, mgrid, stream);
    else launch_merge<F16>(d, a.D, mgrid, stream);
    launch_done(stream);
  }
  return hipGetLastError();
}

static void trace_header(const AttnArgs& a, const char* path) {
  std::fprintf(stderr,
               "[pa_trace] pa_attention S=%d T=%d Hq=%d Hkv=%d D=%d block_size=%d max_query_len=%d "
               "max_seq_len=%d scale=%g path=%s\n",
               a.S, a.T, a.Hq, a.Hkv, a.D, a.bs, a.max_qlen, a.max_seqlen, static_cast<double>(a.scale), path);
}

void trace_attn_generic(const AttnArgs& a) { trace_header(a, "generic"); }

static hipError_t trace_d_err(const AttnArgs& a, hipStream_t stream) {
  if (!a.d_err) return hipSuccess;
  int32_t e = 0;
  const hipError_t r = hipMemcpyAsync(&e, a.d_err, sizeof(e), hipMemcpyDeviceToHost, stream);
  if (r == hipSuccess && hipStreamSynchronize(stream) == hipSuccess)
    std::fprintf(stderr, "[pa_trace]   d_err=0x%x\n", static_cast<unsigned>(e));
  return r;
}

// Waits for the call, copies its plan to the host and prints it.  w: the KV
// write the call also did (in the planning launch, or first), or null.
hipError_t trace_attn_fast(const AttnArgs& a, hipStream_t stream, const WriteJob* w) {
  const FastPlan f = fast_plan(a.S, a.T, a.Hq, a.Hkv, a.D, a.max_qlen, a.max_seqlen);
  trace_header(a, "fast");
  std::fprintf(stderr,
               "[pa_trace]   split: G=%d decode_parts<=%d rows_per_decode_item<=%d "
               "prefill_rows=%d shared_prefix=%d decode_beside_prefill=%d kv_write=%s workspace_bytes=%zu\n",
               f.G, f.P, f.rows_cap, f.prefill_on ? 1 : 0, f.cascade_on ? 1 : 0, decode_beside_prefill(a) ? 1 : 0,
               !w ? "none" : f.mfma_prefill && write_in_plan_ok(*w) ? "in_plan" : "first", f.bytes);
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return e;
  if (!f.mfma_prefill) {
    std::fprintf(stderr, "[pa_trace]   plan: none (decode items mapped directly: %d sequences x %d heads x %d parts)\n",
                 a.S, a.Hkv, f.P);
    return trace_d_err(a, stream);
  }
  const PlanLayout l = plan_layout(a.S, a.T, f.G, f.P, f.prefill_on, f.cascade_on);
  std::vector<uint8_t> h(l.bytes);
  e = hipMemcpy(h.data(), static_cast<const uint8_t*>(a.workspace) + f.plan_off, l.bytes, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  const int32_t* hdr = reinterpret_cast<const int32_t*>(h.data());
  const int2* entries = reinterpret_cast<const int2*>(hdr + kPlanHeader);
  const int32_t n_entries = std::min(hdr[0], l.cap_entries), n_groups = std::min(hdr[1], l.cap_groups);
  const int64_t n_dec[2] = {std::min<int64_t>(hdr[2], l.cap_dec), std::min<int64_t>(hdr[3], l.cap_dec)};
  int32_t n_tiles = 0, n_parts = 0;
  for (int32_t i = 0; i < n_entries; ++i) (entries[i].x >= 0 ? n_tiles : n_parts)++;
  std::fprintf(stderr,
               "[pa_trace]   plan: %d prefill-kernel entries (%d query tiles, %d shared-prefix parts), %d "
               "shared-prefix groups, decode items %lld one-tile, %lld two-tile (parts of at most %d, %d "
               "tokens)\n",
               n_entries, n_tiles, n_parts, n_groups, static_cast<long long>(n_dec[0]),
               static_cast<long long>(n_dec[1]), hdr[4] * kChunk, hdr[5] * kChunk);
  const int4* groups = reinterpret_cast<const int4*>(h.data() + l.groups_off);
  const int32_t* members = reinterpret_cast<const int32_t*>(h.data() + l.members_off);
  for (int32_t g = 0; g < n_groups; ++g) {
    const int4 gr = groups[g];
    std::fprintf(stderr, "[pa_trace]   group %d: prefix_tokens=%d parts=%d first_prefix_slot=%d members=%d [", g,
                 gr.z, gr.w & 255, gr.w >> 8, gr.y);
    for (int32_t k = 0; k < gr.y && gr.x + k < a.S; ++k) std::fprintf(stderr, "%s%d", k ? " " : "", members[gr.x + k]);
    std::fprintf(stderr, "]\n");
  }
  constexpr int32_t kShow = 32;
  std::fprintf(stderr, "[pa_trace]   prefill list (sequence, query tile) or (-(group + 1), part), heaviest first:");
  for (int32_t i = 0; i < std::min(n_entries, kShow); ++i) std::fprintf(stderr, " (%d,%d)", entries[i].x, entries[i].y);
  std::fprintf(stderr, "%s\n", n_entries > kShow ? " ..." : "");
  const int2* dec = reinterpret_cast<const int2*>(h.data() + l.dec_off);
  for (int c = 0; c < 2; ++c) {
    std::fprintf(stderr, "[pa_trace]   %s decode list (sequence, part), heaviest first:", c ? "two-tile" : "one-tile");
    for (int64_t i = 0; i < std::min<int64_t>(n_dec[c], kShow); ++i)
      std::fprintf(stderr, " (%d,%d)", dec[c * l.cap_dec + i].x, dec[c * l.cap_dec + i].y);
    std::fprintf(stderr, "%s\n", n_dec[c] > kShow ? " ..." : "");
  }
  return trace_d_err(a, stream);
}

}  // namespace pa

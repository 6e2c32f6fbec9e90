// MFMA prefill / chunk kernel for pa_attention (bf16/f16, head_dim 64, 128
// or 256, block size a multiple or a divisor of 16): sequences with
// query_len * G above the decode kernels' rows, and the shared-prefix parts of
// cascade groups.
//
// "vLLM Continuous Batching：从 Forward Shape 理解两个核心参数" §2.3: the rows of
// a prefill chunk at positions p = seq_len - query_len + i each see positions
// 0..p of their own sequence (history and this step's rows, already written
// to the cache); "LLM 推理引擎 Continuous Batching 与 PagedAttention" §1.1:
// prefill is the compute-bound O(n^2) side, so this kernel is built around the
// matrix cores.  Online softmax as in that page's §3.3 kernel.
//
// Work item = (sequence, 128 query rows, KV head g); the rows are the
// (query i, head hg) pairs of the group, i-major, so the G query heads that
// share KV head g share every K/V tile.  Workgroup = 4 waves x 32 rows.
// KV is walked in 64-token tiles gathered through the block table (each
// 16-token group lies in one block) straight from HBM into LDS with
// global_load_lds_dwordx4 (no register staging); two LDS stages, so the next
// tile's loads are in flight while the current tile computes, one barrier per
// tile.
//   S^T[64 tok][32 rows] = K . Q^T : 2 token blocks x D/16 steps of
//                                    v_mfma_f32_32x32x16, A = K rows from LDS
//                                    (ds_read_b128), B = the wave's Q^T
//                                    fragments held in registers
//   O^T[D][32 rows]     += V^T . P^T : D/32 output blocks x 4 steps of 16
//                                    tokens; P^T is 8 consecutive S^T results
//                                    of a lane, converted in place; V^T comes
//                                    from two transposed LDS reads per operand.
// Each lane holds one row of its wave, so the softmax of a tile is in-lane
// work plus one lane swap.  Only tiles that cross a wave's diagonal are masked.
//
// Work list: a one-workgroup planning kernel lists every (sequence, query
// tile) of the prefill class, sorted by its number of K/V tiles, heaviest
// first; the attention kernel's workgroups take the list in that order.  So
// the longest items start first (the launch tail is short), and the grid,
// sized from the batch's bound, only ever has empty items at its end: the
// workgroup dispatcher is in order, and empty items mixed among real ones were
// measured to hold back the real ones behind them.
#include "mfma_common.h"
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kRowsPerWG = 128;                    // query rows per workgroup
constexpr int kRowsPerWave = 32;                    // the 32 columns of a wave's MFMA tiles
constexpr int kWaves = kRowsPerWG / kRowsPerWave;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 64;                          // KV tokens per tile
constexpr float kRescaleSlack = 8.f;               // log2 units the running max may lag
constexpr int kQtRun = 4;                          // query tiles of one (sequence, head) per XCD run

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_tables;
  const int32_t* qsl;
  const int32_t* seq_lens;
  int32_t S, Hq, Hkv, G, NB, MB, bs, min_rows;
  float scale_log2e;
  uint16_t* out;
  int32_t* d_err;
  const int32_t* plan;  // work list (layout in pa_internal.h)
  const int4* groups;   // cascade groups
  const int32_t* members;  // cascade members (a group's x is its first position)
  float* ws_pre;        // cascade prefix partials: (slot, KV head, group row)
  int32_t prio;         // 1: raise the waves' issue priority (launched beside the decode kernel)
};

constexpr int kPlanThreads = 1024;
constexpr int kPlanBuckets = 2048;  // K/V tile counts; larger ones share the top bucket
constexpr int kMatchThreads = 256;  // matching kernel: one workgroup per sequence
constexpr int kMatchU = 8;          // block ids per thread and compare step (2048 per step)

struct PlanArgs {
  const int32_t* qsl;
  const int32_t* seq_lens;
  const int32_t* block_tables;
  int32_t S, T, G, MB, bs, rows_cap, prefill_on, cascade_on, cap_entries, cap_groups;
  int32_t P, max_q;  // decode parts per sequence at most; the max_query_len hint
  int32_t dec_slots[2];  // list entries one wave of the one-tile / two-tile decode launch holds
  int64_t cap_dec;   // entries of each decode list
  int32_t* plan;
  int4* groups;
  int4* seq_prefix;
  int32_t* members;  // cascade members, each leader's stretch in rank order
  const int2* match; // per sequence: (leader, blocks shared with it), from cascade_match_kernel
  int2* dec;         // decode lists: one-tile at dec, two-tile at dec + cap_dec
  int32_t* d_err;
  // a KV write done by workgroups 1.. of the launch, 16 token rows each
  // (write_kv_row; 16-byte rows and pointers); wT = 0: none
  const char* wk;
  const char* wv;
  const int32_t* wslot;
  char* wk_cache;
  char* wv_cache;
  int64_t w_row_bytes, w_num_slots;
  int32_t* w_err;
  int32_t wT;
};

struct MatchArgs {
  const int32_t* qsl;
  const int32_t* seq_lens;
  const int32_t* block_tables;
  int32_t S, MB, bs, thr_blocks;
  int2* match;
};

constexpr int kDecBuckets = 1024;  // decode list weights: chunks of a part, larger ones share the top bucket

// KV heads per run slot of the prefill item order: 4 when they divide Hkv.
__host__ __device__ __forceinline__ int32_t prefill_head_group(int32_t Hkv) {
  return (Hkv & 3) == 0 ? 4 : ((Hkv & 1) == 0 ? 2 : 1);
}

// K/V tiles query tile qt of a sequence reads (its last row's causal limit).
__device__ __forceinline__ int32_t plan_weight(int32_t L, int32_t qlen, int32_t rows, int32_t G, int32_t qt) {
  if (L < qlen) return 1;  // invalid: the kernel only writes zeros
  const int32_t last_row = min(qt * kRowsPerWG + kRowsPerWG - 1, rows - 1);
  return min((L - qlen + last_row / G) / kTile + 1, kPlanBuckets - 1);
}

// Exclusive scan over the kPlanThreads threads of the plan workgroup (sum or
// max, with `id` the identity); wbuf holds one value per wave.  Every thread
// must call it.
template <bool kMax>
__device__ int32_t plan_block_scan(int32_t v, int32_t id, int32_t* wbuf) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t incl = v;
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t y = __shfl_up(incl, off, 64);
    if (lane >= off) incl = kMax ? max(incl, y) : incl + y;
  }
  int32_t excl = __shfl_up(incl, 1, 64);
  if (lane == 0) excl = id;
  __syncthreads();
  if (lane == 63) wbuf[wave] = incl;
  __syncthreads();
  int32_t before = id;
  for (int w = 0; w < wave; ++w) before = kMax ? max(before, wbuf[w]) : before + wbuf[w];
  return kMax ? max(before, excl) : before + excl;
}

// A cascade candidate: a single-token decode sequence with at least
// thr_blocks full blocks and a valid first block id (its key).  The four
// loads are unconditional (s < S, and the caller checks MB >= 1), so a
// thread's loads for two sequences are all in flight together.
struct Candidate {
  int32_t key, full;
  bool ok;
};
__device__ __forceinline__ Candidate cascade_candidate(const MatchArgs& a, int32_t s) {
  const int32_t q0 = a.qsl[s], q1 = a.qsl[s + 1], L = a.seq_lens[s];
  const int32_t key = a.block_tables[static_cast<int64_t>(s) * a.MB];
  Candidate c;
  c.key = key;
  c.full = L / a.bs;
  c.ok = q1 - q0 == 1 && L >= 1 && ceil_div(L, a.bs) <= a.MB && c.full >= a.thr_blocks && key >= 0;
  return c;
}

// Smallest value any thread of the workgroup offers (INT32_MAX if none);
// every thread must call it.
__device__ __forceinline__ int32_t match_block_min(int32_t v, int32_t* cell) {
  if (threadIdx.x == 0) *cell = INT32_MAX;
  __syncthreads();
  if (v != INT32_MAX) atomicMin(cell, v);
  __syncthreads();
  const int32_t m = *cell;
  __syncthreads();  // the cell is reused by the next call
  return m;
}

// Cascade matching, one workgroup per sequence s ("vLLM 原理" §2.1, and the
// shared prefixes of "LLM 推理引擎 Continuous Batching 与 PagedAttention"
// §4.1, §4.2: sequences whose tables map the same physical block at the same
// logical position share that block's contents).  A candidate's leader is
// the smallest candidate with the same first block id (itself if there is
// none before it), so the grouping depends only on which tables share
// blocks, not on where the sequences sit in the batch.  A follower compares
// its table with its leader's from the start; match[s] = (leader, full
// blocks the two agree on from the start), (s, full blocks) for a leader and
// (-1, 0) for a sequence that is no candidate.
__global__ __launch_bounds__(kMatchThreads) void cascade_match_kernel(MatchArgs a) {
  __shared__ int32_t cell, leader_full;
  const int32_t s = blockIdx.x;
  const int tid = threadIdx.x;
  if (a.MB < 1) {  // no table entries: no candidates (and no row to read)
    if (tid == 0) a.match[s] = make_int2(-1, 0);
    return;
  }
  // this sequence and the first kMatchThreads sequences, loads in flight together
  const Candidate me = cascade_candidate(a, s);
  Candidate other = cascade_candidate(a, min(tid, s));
  if (!me.ok) {
    if (tid == 0) a.match[s] = make_int2(-1, 0);
    return;
  }
  int32_t ld = s;
  for (int32_t t0 = 0; t0 < s; t0 += kMatchThreads) {
    const int32_t t = t0 + tid;
    if (t0 > 0) other = cascade_candidate(a, min(t, s));
    const bool hit = t < s && other.ok && other.key == me.key;
    const int32_t m = match_block_min(hit ? t : INT32_MAX, &cell);
    if (m != INT32_MAX) {
      if (t == m) leader_full = other.full;
      __syncthreads();
      ld = m;
      break;
    }
  }
  int32_t first = me.full;
  if (ld != s) {
    const int32_t n = min(me.full, leader_full);
    const int32_t* b0 = a.block_tables + static_cast<int64_t>(ld) * a.MB;
    const int32_t* b1 = a.block_tables + static_cast<int64_t>(s) * a.MB;
    first = n;
    for (int32_t j0 = 0; j0 < n; j0 += kMatchThreads * kMatchU) {
      // all loads first (indices clamped into the row), then the compares
      int32_t x0[kMatchU], x1[kMatchU];
#pragma unroll
      for (int u = 0; u < kMatchU; ++u) {
        const int32_t j = min(j0 + kMatchThreads * u + tid, n - 1);
        x0[u] = b0[j];
        x1[u] = b1[j];
      }
      int32_t mn = INT32_MAX;
#pragma unroll
      for (int u = 0; u < kMatchU; ++u) {
        const int32_t j = j0 + kMatchThreads * u + tid;
        if (j < n && x0[u] != x1[u]) mn = min(mn, j);
      }
      const int32_t m = match_block_min(mn, &cell);
      if (m != INT32_MAX) {
        first = m;
        break;
      }
    }
  }
  if (tid == 0) a.match[s] = make_int2(ld, first);
}

// One workgroup plans the call.
//
// Cascade groups, from cascade_match_kernel's (leader, shared blocks) of each
// candidate: a follower that agrees with its leader on at least
// kCascadeMinTiles tiles joins it; the group's shared prefix is the fewest
// blocks any joined member shares with the leader, rounded down to whole
// tiles (members agree pairwise there), read once for all members in up to
// kCascadeMaxParts parts.  A leader's members are listed in the plan (rank
// order) and cut into groups of at most kCascadeRows / G; groups take their
// indices in leader order, and the first kCascadeEntries are cascaded.
//
// Work list: every prefill-class (sequence, query tile) and every cascade
// prefix part, counting-sorted by the K/V tiles it reads, heaviest first.
// Entries of equal weight land in any order (which workgroup computes an
// entry does not change its result).  At most cap_entries entries are written
// (more can only come from inconsistent query_start_loc, which other kernels
// flag); a query_len outside 1..T is not planned.
__global__ __launch_bounds__(kPlanThreads) void attn_plan_kernel(PlanArgs a) {
  __shared__ int32_t hist[kPlanBuckets];
  __shared__ int32_t cursor[kPlanBuckets];
  __shared__ int32_t wave_tot[kPlanThreads / 64];
  __shared__ int32_t gbase_of[kCascadeMaxSeqs];  // leader with members: its first group index, else -1
  __shared__ int32_t mbase_of[kCascadeMaxSeqs];  // leader with members: its first member-list position
  __shared__ int32_t hcnt[kCascadeMaxSeqs];      // leader: joined followers, later the rank counter
  __shared__ int32_t hpre[kCascadeMaxSeqs];      // leader: fewest blocks a joined follower shares with it
  __shared__ int32_t n_groups;
  __shared__ int32_t dhist[2][2][kDecBuckets];  // [default, doubled part length][list][weight]
  __shared__ int32_t dcur[2][kDecBuckets];
  __shared__ int32_t dcount[2];  // decode list entries at the default part length
  if (blockIdx.x > 0) {  // the KV write's workgroups: one wave per token row
    const int64_t t = static_cast<int64_t>(blockIdx.x - 1) * (kPlanThreads / 64) +
                      __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (t < a.wT)
      write_kv_row<16>(a.wk, a.wv, a.wslot, t, a.w_row_bytes, a.wk_cache, a.wv_cache, a.w_num_slots, a.w_err,
                       threadIdx.x & 63);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kPlanBuckets; i += kPlanThreads) hist[i] = 0;
  for (int i = tid; i < kDecBuckets; i += kPlanThreads) {
    dhist[0][0][i] = 0;
    dhist[0][1][i] = 0;
    dhist[1][0][i] = 0;
    dhist[1][1][i] = 0;
  }
  if (tid == 0) n_groups = 0;
  if (tid < 2) dcount[tid] = 0;

  // Barriers order global stores too (each waits for this workgroup's stores
  // to complete), so the stores are placed where little follows them: the
  // per-sequence prefix records are zeroed up front only when a group is
  // possible at all, else once at the very end.
  bool prefix_zero_late = false;
  if (a.cascade_on) {
    static_assert(kCascadeMaxSeqs == kPlanThreads, "one sequence per thread in the cascade phases");
    const int32_t thr_blocks = ceil_div(kCascadeMinTiles * kTile, a.bs);
    const int32_t max_members = max(2, kCascadeRows / a.G);
    const int32_t s = tid;
    int2 m = make_int2(-1, 0);
    if (s < a.S) m = a.match[s];
    gbase_of[s] = -1;
    hcnt[s] = 0;
    hpre[s] = INT32_MAX;
    __syncthreads();
    // followers sharing at least thr_blocks with their leader join it
    const bool joins = m.x >= 0 && m.x != s && m.y >= thr_blocks;
    if (joins) {
      atomicAdd(&hcnt[m.x], 1);
      atomicMin(&hpre[m.x], m.y);
    }
    if (!__syncthreads_or(joins)) {  // no follower joined: no group
      prefix_zero_late = true;
      if (tid == 0) a.plan[1] = 0;
    } else {
      if (s < a.S) a.seq_prefix[s] = make_int4(0, 0, 0, 0);
      // groups in leader order: a leader with members heads ceil(members /
      // max_members) groups over its stretch of the member list
      {
        int32_t ngs = 0, nms = 0;
        if (m.x == s && hcnt[s] > 0) {
          nms = hcnt[s] + 1;  // the followers and the leader
          ngs = ceil_div(nms, max_members);
        }
        const int32_t gb = plan_block_scan<false>(ngs, 0, wave_tot);
        const int32_t mb = plan_block_scan<false>(nms, 0, wave_tot);
        if (ngs > 0) {
          gbase_of[s] = gb;
          mbase_of[s] = mb;
          hcnt[s] = 0;  // from here on the leader's rank counter
          const int32_t pre_tokens = hpre[s] * a.bs / kTile * kTile;
          for (int32_t c = 0; c < ngs && gb + c < a.cap_groups; ++c)
            a.groups[gb + c] = make_int4(mb + c * max_members, min(max_members, nms - c * max_members), pre_tokens, 0);
        }
        if (tid == kPlanThreads - 1) n_groups = min(gb + ngs, a.cap_groups);
      }
      __syncthreads();
      // parts (up to kCascadeMaxParts of at least kCascadeMinTiles tiles,
      // kCascadeEntries over all groups) and each group's first prefix slot
      const int32_t ngr = n_groups;
      if (wave == 0) {
        int32_t parts = 0;
        int4 gr = make_int4(0, 0, 0, 0);
        if (lane < ngr) {
          gr = a.groups[lane];
          parts = max(1, min(min(kCascadeMaxParts, gr.z / kTile / kCascadeMinTiles), kCascadeEntries / ngr));
        }
        int32_t base = parts;
        for (int off = 1; off < 64; off <<= 1) {
          const int32_t y = __shfl_up(base, off, 64);
          if (lane >= off) base += y;
        }
        base -= parts;
        if (lane < ngr) {
          gr.w = parts | (base << 8);
          a.groups[lane] = gr;
        }
      }
      __syncthreads();
      // members: the leader and each joined follower take a rank in the
      // leader's stretch of the member list (any order: a member's rows give
      // the same values wherever they sit in the group), and a member of a
      // cascaded group gets its prefix record
      const int32_t ld = m.x;
      if (ld >= 0 && gbase_of[ld] >= 0 && (ld == s || joins)) {
        const int32_t r = atomicAdd(&hcnt[ld], 1);
        a.members[mbase_of[ld] + r] = s;
        const int32_t gi = gbase_of[ld] + r / max_members;
        if (gi < ngr) {
          const int4 gr = a.groups[gi];
          a.seq_prefix[s] = make_int4(gr.z, gr.w & 255, gr.w >> 8, (r % max_members) * a.G);
        }
      }
      if (tid == 0) a.plan[1] = ngr;
    }
  }
  __syncthreads();
  const int32_t ng = n_groups;

  // A decode-class sequence's item: list c (one-tile 0, two-tile 1) and the
  // chunks its parts cover (nch, the cascade prefix removed); special: the
  // decode kernels only zero-fill it (one weight-0 part).  False: no decode item.
  auto dec_item = [&](int32_t s, int32_t& c, int32_t& nch, bool& special) -> bool {
    const int32_t qlen = a.qsl[s + 1] - a.qsl[s];
    if (qlen <= 0 || qlen > a.T) return false;
    const int32_t rows = qlen * a.G;
    c = 0;
    nch = 0;
    special = true;
    if (rows > a.rows_cap) return !a.prefill_on;
    c = rows > 16 ? 1 : 0;
    const int32_t L = a.seq_lens[s];
    if (L < qlen || ceil_div(L, a.bs) > a.MB) return true;
    const int32_t pre = a.cascade_on && !prefix_zero_late ? a.seq_prefix[s].x : 0;
    nch = ceil_div(L, 16) - pre / 16;
    special = false;
    return true;
  };

  // Histogram by the weight of each sequence's heaviest query tile (its
  // last) and of each group's prefix parts.  A sequence's query tiles stay
  // together in the list, heaviest first, so the tiles of one (sequence, KV
  // head), which read the same K/V, run side by side on one XCD and share it
  // through L2 (sorting single tiles by weight mixed sequences and doubled the
  // mixed batch's HBM reads); the order stays longest-first by sequence.
  if (a.prefill_on) {
    for (int32_t s = tid; s < a.S; s += kPlanThreads) {
      const int32_t qlen = a.qsl[s + 1] - a.qsl[s];
      if (qlen <= 0 || qlen > a.T || qlen * a.G <= a.rows_cap) continue;
      const int32_t rows = qlen * a.G, L = a.seq_lens[s], nq = ceil_div(rows, kRowsPerWG);
      atomicAdd(&hist[plan_weight(L, qlen, rows, a.G, nq - 1)], nq);
    }
  }
  for (int32_t gi = tid; gi < ng; gi += kPlanThreads) {
    const int4 gr = a.groups[gi];
    const int32_t parts = gr.w & 255;
    atomicAdd(&hist[min(ceil_div(gr.z / kTile, parts), kPlanBuckets - 1)], parts);
  }
  __syncthreads();
  // exclusive scan in descending weight: thread t owns reversed buckets
  constexpr int kPer = kPlanBuckets / kPlanThreads;
  int32_t v[kPer], sum = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    v[j] = hist[kPlanBuckets - 1 - (kPer * tid + j)];
    sum += v[j];
  }
  int32_t incl = sum;
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int32_t before = 0;
  for (int w = 0; w < wave; ++w) before += wave_tot[w];
  int32_t run = before + incl - sum;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int w = kPlanBuckets - 1 - (kPer * tid + j);
    cursor[w] = run;  // first position of bucket w
    run += v[j];
  }
  if (tid == kPlanThreads - 1) a.plan[0] = min(run, a.cap_entries);  // total entries
  __syncthreads();
  int2* entries = reinterpret_cast<int2*>(a.plan + kPlanHeader);
  if (a.prefill_on) {
    for (int32_t s = tid; s < a.S; s += kPlanThreads) {
      const int32_t qlen = a.qsl[s + 1] - a.qsl[s];
      if (qlen <= 0 || qlen > a.T || qlen * a.G <= a.rows_cap) continue;
      const int32_t rows = qlen * a.G, L = a.seq_lens[s], nq = ceil_div(rows, kRowsPerWG);
      const int32_t pos = atomicAdd(&cursor[plan_weight(L, qlen, rows, a.G, nq - 1)], nq);
      for (int32_t k = 0; k < nq && pos + k < a.cap_entries; ++k) entries[pos + k] = make_int2(s, nq - 1 - k);
    }
  }
  for (int32_t gi = tid; gi < ng; gi += kPlanThreads) {
    const int4 gr = a.groups[gi];
    const int32_t parts = gr.w & 255;
    const int32_t pos = atomicAdd(&cursor[min(ceil_div(gr.z / kTile, parts), kPlanBuckets - 1)], parts);
    for (int32_t pp = 0; pp < parts && pos + pp < a.cap_entries; ++pp) entries[pos + pp] = make_int2(-(gi + 1), pp);
  }

  // Decode work lists: every (sequence, part) item of the one-tile and of the
  // two-tile decode instance, each list counting-sorted by the chunks the part
  // reads, heaviest first, so the decode grids hold no empty item before a
  // real one.  A sequence the decode kernels only zero-fill (a violated hint,
  // an invalid length or table) gets one part-0 entry in the one-tile list,
  // last.  The max_query_len hint is checked here for every sequence.
  // (dhist was cleared at the start; no barrier here, so the list entries'
  // stores above need not complete before the decode histogram is built)
  auto item_parts = [&](int32_t nch, bool special, int32_t pc, int32_t& np, int32_t& cpp) {
    np = 1;
    cpp = 0;
    if (!special) plan_parts(nch, a.P, &np, &cpp, pc);
  };
  auto part_weight = [&](int32_t p, int32_t cpp, int32_t nch, bool special) {
    return special ? 0 : min(min(cpp, nch - p * cpp), kDecBuckets - 1);
  };
  // Part length of each list: a list whose items at the default length would
  // fill between one and two waves of its launch's slots gets parts twice as
  // long, so it runs as one wave (the same time per slot by a count of
  // rounds, with half the item starts and no second round behind the first:
  // verify batch 0.436 -> 0.413 ms).  Other lists keep kPartChunks.  The
  // histogram is built for both lengths at once; the counts decide which
  // one the scan takes.
  for (int32_t s = tid; s < a.S; s += kPlanThreads) {
    const int32_t qlen = a.qsl[s + 1] - a.qsl[s];
    if (qlen > a.max_q) flag(a.d_err, PA_DERR_HINT);
    int32_t c, np, cpp, nch;
    bool special;
    if (!dec_item(s, c, nch, special)) continue;
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      item_parts(nch, special, (d + 1) * kPartChunks, np, cpp);
      if (d == 0) atomicAdd(&dcount[c], np);
      for (int32_t p = 0; p < np; ++p) atomicAdd(&dhist[d][c][part_weight(p, cpp, nch, special)], 1);
    }
  }
  __syncthreads();
  int32_t dbl[2];  // 1: the list takes the doubled part length
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int32_t n = dcount[c];
    dbl[c] = n > a.dec_slots[c] && n < 2 * a.dec_slots[c] ? 1 : 0;
  }
  static_assert(kDecBuckets == kPlanThreads, "one bucket per thread in the scan");
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int32_t v = dhist[dbl[c]][c][kDecBuckets - 1 - tid];  // descending weight
    const int32_t excl = plan_block_scan<false>(v, 0, wave_tot);
    dcur[c][kDecBuckets - 1 - tid] = excl;
    if (tid == kPlanThreads - 1) {
      const int64_t total = static_cast<int64_t>(excl) + v;
      a.plan[2 + c] = static_cast<int32_t>(total < a.cap_dec ? total : a.cap_dec);
      a.plan[4 + c] = (dbl[c] + 1) * kPartChunks;
    }
  }
  __syncthreads();
  for (int32_t s = tid; s < a.S; s += kPlanThreads) {
    int32_t c, np, cpp, nch;
    bool special;
    if (!dec_item(s, c, nch, special)) continue;
    item_parts(nch, special, (dbl[c] + 1) * kPartChunks, np, cpp);
    int2* list = a.dec + c * a.cap_dec;
    for (int32_t p = 0; p < np; ++p) {
      const int32_t pos = atomicAdd(&dcur[c][part_weight(p, cpp, nch, special)], 1);
      if (pos < a.cap_dec) list[pos] = make_int2(s, p);
    }
  }
  if (prefix_zero_late)
    for (int32_t s = tid; s < a.S; s += kPlanThreads) a.seq_prefix[s] = make_int4(0, 0, 0, 0);
}


// LDS tile geometry for head_dim D: a token row of one head is 2D bytes =
// D/8 chunks of 16 bytes, 64 rows per tile, stored without padding.  Chunk c
// of row R sits in slot c ^ swz(R):
//   K: swz = R & min(D/8 - 1, 15) -> at head_dim 128 the 16 rows one K
//      fragment read touches use 16 different slots, i.e. all 64 banks once;
//   V: swz = (R & 3) << 2 (<< 1 at head_dim 64) -> a transposed read takes
//      4 consecutive rows x 32 bytes per 16 lanes (x 64 bytes per 32 lanes),
//      and the XOR moves the 4 rows' chunks onto different banks.
template <int D>
struct Geom {
  static constexpr int kRowBytes = 2 * D;                 // one token row of one head
  static constexpr int kChunks = D / 8;                   // 16-byte chunks per row
  static constexpr int kTileBytes = kTile * kRowBytes;    // one K or V tile
  static constexpr int kStageBytes = 2 * kTileBytes;      // K tile then V tile
  static constexpr int kSwzK = (kChunks < 16 ? kChunks : 16) - 1;
  static constexpr int kVSh = D >= 128 ? 2 : 1;           // V swizzle: chunk ^ ((row & 3) << kVSh)
  static constexpr int kKK = D / 16;                      // 32x32x16 K steps of QK
  static constexpr int kDB = D / 32;                      // 32-wide output blocks of PV
  static constexpr int kRpi = 512 / D;                    // tile rows per DMA instruction
  // K rows: 8 (16) consecutive rows read one chunk each, so their chunks are
  // spread over the banks by XOR with the row's low bits.
  static __device__ __forceinline__ int k_slot(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ (row & kSwzK)) << 4);
  }
  // V rows: a transposed read takes 4 consecutive rows x 32 (or 64) bytes, so
  // the 4 rows' chunks are moved apart by XOR with (row & 3) times 2 (4) chunks.
  static __device__ __forceinline__ int v_swz(int row) { return (row & 3) << kVSh; }
  static __device__ __forceinline__ int v_slot(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ v_swz(row)) << 4);
  }
};

// Waves per SIMD the register budget is set for: head_dim 256 (O of 32 rows
// x 256 columns, twice the Q fragments) runs one wave per SIMD, and one
// workgroup per CU (its two LDS stages take 128 KB).
constexpr int kWavesPerEU = kWaves / 2;  // two workgroups per CU
template <int D>
constexpr int prefill_waves_per_eu() {
  return D == 256 ? 1 : kWavesPerEU;
}

// kBlk16: the block size is a multiple of 16 (a wave's 16-row group lies in
// one block); otherwise it divides 16 and each row finds its own block.
// D: head_dim (64, 128, 256).
template <class F, bool kBlk16, int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(prefill_waves_per_eu<D>(), kWavesPerEU))) void prefill_kernel(PrefillArgs a) {
  using M = Mma<F>;
  using Gm = Geom<D>;
  constexpr int kRowBytes = Gm::kRowBytes, kTileBytes = Gm::kTileBytes, kStageBytes = Gm::kStageBytes;
  constexpr int kKK = Gm::kKK, kDB = Gm::kDB, kRpi = Gm::kRpi;
  // Two stages as two arrays: the tile loop below is unrolled by two so every
  // LDS read and every DMA names its stage statically, and the compiler can
  // see that the DMA into one stage does not touch the stage being read (with
  // one array indexed by kt & 1 it waited for the next tile's DMA before the
  // first read of the current tile, exposing every load's latency).
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h = lane >> 5;  // the lane's row of the wave, and its half
  // Beside the decode kernel's waves (one of each per SIMD) the prefill waves
  // issue first: mixed step's prefill launch 578 -> 540-549 us, its decode
  // launch 542 -> 558-564 us, so the two chains end closer together (the
  // two-tile decode launch then follows the prefill kernel; launch_attn_fast)
  if (a.prio) __builtin_amdgcn_s_setprio(1);

  // Items.  Workgroup b runs on XCD b % 8, and an XCD hands its workgroups
  // in order, round-robin, to its 4 shader engines, each waiting for a free
  // slot on its own engine.  A run is kQtRun consecutive list entries (often
  // query tiles of one sequence, which share every K/V tile through the XCD's
  // L2) times a group of hg KV heads, ordered entry-major: consecutive
  // workgroups are the same entry for different heads, equal in weight, so
  // the engines stay evenly loaded (entry-minor order gave one engine every
  // block's heaviest tile and stalled the others behind it).  The k-th run an
  // XCD takes is run 8k + ((xcd + k) mod 8); runs go by (entry block, head
  // group), heaviest first.
  const int32_t bid = blockIdx.x;
  const int32_t hg = prefill_head_group(a.Hkv), run_len = kQtRun * hg;
  const int32_t xcd = bid & 7, jj = bid >> 3;
  const int32_t kr = jj / run_len, within = jj - kr * run_len;
  const int32_t run = kr * 8 + ((xcd + kr) & 7);
  const int32_t n_hg = a.Hkv / hg;
  const int32_t e = (run / n_hg) * kQtRun + within / hg;
  const int32_t g = (run % n_hg) * hg + within % hg;
  if (e >= a.plan[0]) return;
  const int2 ent = reinterpret_cast<const int2*>(a.plan + kPlanHeader)[e];
  // A prefill entry is one query tile of sequence s.  A cascade entry is one
  // part of a group's shared prefix: its rows are (member, query head) pairs,
  // one decode row per member, all of the prefix is visible to them, K/V come
  // through the first member's table (the same blocks as every member's), and
  // the result is a split-K partial per row for the decode merge.
  const bool cascade = ent.x < 0;
  int32_t s, qt_first, q0, qlen, rows_total, L, pp = 0, slot = 0, kt_begin = 0, kt_end = 0, mbeg = 0;
  if (!cascade) {
    s = ent.x;
    qt_first = ent.y;
    q0 = a.qsl[s];
    qlen = a.qsl[s + 1] - q0;
    rows_total = qlen * a.G;
    L = a.seq_lens[s];
  } else {
    const int4 gr = a.groups[-ent.x - 1];
    s = a.members[gr.x];  // any member's table holds the shared prefix
    mbeg = gr.x;
    qt_first = 0;
    q0 = 0;
    qlen = 1;
    rows_total = gr.y * a.G;
    L = gr.z;  // the prefix: every tile read lies inside it
    pp = ent.y;
    slot = (gr.w >> 8) + pp;
    const int32_t per = ceil_div(gr.z / kTile, gr.w & 255);
    kt_begin = pp * per;
    kt_end = min(gr.z / kTile, kt_begin + per);
  }

  if (!cascade && (L < qlen || ceil_div(L, a.bs) > a.MB)) {
    if (tid == 0) flag(a.d_err, L < qlen ? PA_DERR_QLEN_GT_SEQLEN : PA_DERR_BLOCK_OOB);
    const int32_t r0 = qt_first * kRowsPerWG, r1 = min(r0 + kRowsPerWG, rows_total);
    for (int32_t idx = tid; idx < (r1 - r0) * D; idx += kThreads) {
      const int32_t rho = r0 + idx / D;
      const int32_t i = rho / a.G, hg = rho - (rho / a.G) * a.G;
      a.out[((static_cast<int64_t>(q0) + i) * a.Hq + g * a.G + hg) * D + idx % D] = 0;
    }
    return;
  }

  const int32_t* btrow = a.block_tables + static_cast<int64_t>(s) * a.MB;
  const int64_t slot_stride = static_cast<int64_t>(a.Hkv) * D;  // elements between slots
  const uint16_t* kbase = a.k_cache + static_cast<int64_t>(g) * D;
  const uint16_t* vbase = a.v_cache + static_cast<int64_t>(g) * D;

  // DMA of one tile: wave w fills rows kDmaRows*w .. (inside one 16-token
  // group, so one block id) of the K and V tiles, kRpi rows per instruction,
  // lane -> 16 bytes (row lane / (D/8), slot lane % (D/8)).  Rows at or past
  // the context end re-read the last valid row, so nothing unwritten
  // (possibly NaN) ever reaches LDS; such rows are masked anyway.
  constexpr int kDmaRows = kTile / kWaves;     // tile rows each wave fills
  constexpr int kDmaInst = kDmaRows / kRpi;    // DMA instructions per wave and tile
  static_assert(16 % kDmaRows == 0 || kDmaRows % 16 == 0, "a wave's rows stay inside 16-token groups");
  static_assert(kDmaRows % kRpi == 0, "whole DMA instructions per wave");
  const int row_base = kDmaRows * __builtin_amdgcn_readfirstlane(wave);  // wave-uniform
  const int dma_row = lane / Gm::kChunks, dma_slot = lane % Gm::kChunks;
  // Byte offsets of this lane's K and V sources from the first slot of the
  // wave's rows; the same for every tile whose rows are all inside the context.
  // (at most 15 slot rows of Hkv x 2D bytes: fits 32 bits for any Hkv the
  // grid allows).  Unsigned, so a DMA address is a scalar base plus a
  // zero-extended lane offset, which the instruction takes as is.
  uint32_t k_src_off[kDmaInst], v_src_off[kDmaInst];
#pragma unroll
  for (int u = 0; u < kDmaInst; ++u) {
    const int row = row_base + kRpi * u + dma_row;
    const uint32_t rowoff = static_cast<uint32_t>((row & 15) * a.Hkv * kRowBytes);
    k_src_off[u] = rowoff + 16 * (dma_slot ^ (row & Gm::kSwzK));
    v_src_off[u] = rowoff + 16 * (dma_slot ^ Gm::v_swz(row));
  }
  // Block id of the wave's 16-token group in tile kt when the group lies
  // inside the context (loaded one tile ahead of its DMA, so the DMA never
  // waits for the block table); 0 otherwise (the DMA then takes the per-row
  // path).
  // The table is read-only here and the index wave-uniform: read it through
  // the constant address space, which makes it a scalar load (counted apart
  // from the tile DMAs, so using it never waits for them).
  constexpr bool blk16 = kBlk16;
  const __attribute__((address_space(4))) int32_t* btrow_c =
      (const __attribute__((address_space(4))) int32_t*)(btrow);
  auto load_bid = [&](int32_t kt) -> int32_t {
    const int32_t t16 = kt * kTile + (row_base & ~15);
    return t16 + 16 <= L ? btrow_c[t16 / a.bs] : 0;
  };
  auto issue_tile = [&](int32_t kt, uint8_t* stage_lds, int32_t b) {
    const int32_t t16 = kt * kTile + (row_base & ~15);
    uint8_t* kdst = stage_lds + row_base * kRowBytes;
    uint8_t* vdst = kdst + kTileBytes;
    if (blk16 && t16 + 16 <= L) {  // all of the wave's rows inside the context: one block, fixed offsets
      const int32_t lb = t16 / a.bs;
      if (b < 0 || b >= a.NB) {
        flag(a.d_err, PA_DERR_BLOCK_OOB);
        b = 0;
      }
      const int64_t slot0 = static_cast<int64_t>(b) * a.bs + (t16 - lb * a.bs);  // first slot of the group
      const uint8_t* ksrc = reinterpret_cast<const uint8_t*>(kbase + slot0 * slot_stride);
      const uint8_t* vsrc = reinterpret_cast<const uint8_t*>(vbase + slot0 * slot_stride);
#pragma unroll
      for (int u = 0; u < kDmaInst; ++u) {
        __builtin_amdgcn_global_load_lds((const void*)(ksrc + k_src_off[u]),
                                         (__attribute__((address_space(3))) void*)(kdst + kRpi * u * kRowBytes),
                                         16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(vsrc + v_src_off[u]),
                                         (__attribute__((address_space(3))) void*)(vdst + kRpi * u * kRowBytes),
                                         16, 0, 0);
      }
      return;
    }
    const int32_t lb = (t16 < L ? t16 : L - 1) / a.bs;
    b = btrow_c[lb];
    if (b < 0 || b >= a.NB) {
      flag(a.d_err, PA_DERR_BLOCK_OOB);
      b = 0;
    }
    const int64_t slot0 = static_cast<int64_t>(b) * a.bs + (t16 < L ? t16 - lb * a.bs : 0);
#pragma unroll
    for (int u = 0; u < kDmaInst; ++u) {
      const int row = row_base + kRpi * u + dma_row;  // tile row this lane fills
      const int32_t tok = kt * kTile + row;
      int64_t slot;
      if (tok < L && blk16) slot = slot0 + (row & 15);
      else if (tok < L) {  // a block size dividing 16: this row's own block
        const int32_t lbr = tok / a.bs;
        int32_t br = btrow[lbr];
        if (br < 0 || br >= a.NB) {
          flag(a.d_err, PA_DERR_BLOCK_OOB);
          br = 0;
        }
        slot = static_cast<int64_t>(br) * a.bs + (tok - lbr * a.bs);
      } else {  // past the end: last valid token of the sequence
        const int32_t lb2 = (L - 1) / a.bs;
        int32_t b2 = btrow_c[lb2];
        b2 = (b2 < 0 || b2 >= a.NB) ? 0 : b2;
        slot = static_cast<int64_t>(b2) * a.bs + (L - 1 - lb2 * a.bs);
      }
      const int kc = dma_slot ^ (row & Gm::kSwzK);  // chunk whose data lands in slot dma_slot
      const int vc = dma_slot ^ Gm::v_swz(row);
      __builtin_amdgcn_global_load_lds((const void*)(kbase + slot * slot_stride + 8 * kc),
                                       (__attribute__((address_space(3))) void*)(kdst + kRpi * u * kRowBytes),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vbase + slot * slot_stride + 8 * vc),
                                       (__attribute__((address_space(3))) void*)(vdst + kRpi * u * kRowBytes),
                                       16, 0, 0);
    }
  };

  {
    const int32_t qt = qt_first;
    const int32_t row0 = qt * kRowsPerWG;
    const int32_t last_row = min(row0 + kRowsPerWG, rows_total) - 1;
    if (!cascade) kt_end = (L - qlen + last_row / a.G) / kTile + 1;
    // flat token index of row rho (its query head is rho mod G)
    auto row_token = [&](int32_t rho) -> int32_t {
      return cascade ? a.qsl[a.members[mbeg + rho / a.G]] : q0 + rho / a.G;
    };
    issue_tile(kt_begin, lds0, load_bid(kt_begin));
    int32_t bid_next = load_bid(kt_begin + 1);

    // The wave's 32 rows are the columns of its MFMA tiles: lane (n, h) works
    // on row n, and the two halves h hold different tokens (S^T, P^T) or head
    // dims (O^T) of it.  Q^T fragment kk: head dims 16 kk + 8 h .. + 7 of row n.
    const int32_t wave_row0 = row0 + wave * kRowsPerWave;
    const bool wave_active = wave_row0 < rows_total;
    const int32_t qpos_min_wave = cascade ? INT32_MAX : L - qlen + wave_row0 / a.G;
    const int32_t rho_n = wave_row0 + n;
    const bool row_valid = rho_n < rows_total;
    const int32_t qpos = cascade ? INT32_MAX : (row_valid ? L - qlen + rho_n / a.G : -1);
    uint4 qf[kKK];
    {
      const int32_t hg = rho_n - (rho_n / a.G) * a.G;
      const int32_t t = row_valid ? row_token(rho_n) : 0;
      const uint16_t* qp = a.q + (static_cast<int64_t>(t) * a.Hq + g * a.G + hg) * D + 8 * h;
#pragma unroll
      for (int kk = 0; kk < kKK; ++kk) qf[kk] = row_valid ? ld16(qp + 16 * kk) : make_uint4(0, 0, 0, 0);
    }

    // Running max of row n in log2 units.  It is only moved when a tile's max
    // exceeds it by more than kRescaleSlack, so p = 2^(x - m) stays <= 2^8 and
    // the O rescale is rare; numerator and denominator always share the same
    // m, so the result is unchanged.  lsum: this half's share of the row sum
    // of P (the halves are added at the end).
    float m = -INFINITY, lsum = 0.f;
    f32x16_t o[kDB];
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[db][v] = 0.f;
    // Per-lane LDS byte offsets inside a stage.  K fragment kk: row n, chunk
    // 2 kk + h (+ 32 rows for the second token block).  Transposed V read for
    // output block db: the lane supplies 4 head dims (chunk 4 db + 2 dhalf +
    // c/2, half c%2) of row 4 h + jrow, where (dhalf, jrow, c) are lane bits
    // 4, 3-2 and 1-0 (+ 32 b + 16 s and + 8 rows per read).  Row offsets that
    // are multiples of 16 (K) or 4 (V) leave the swizzle unchanged, so they
    // fold into constants.
    int koff[kKK], voff[kDB];
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) koff[kk] = Gm::k_slot(n, 2 * kk + h);
    {
      const int dhalf = (lane >> 4) & 1, jrow = (lane >> 2) & 3, c = lane & 3;
#pragma unroll
      for (int db = 0; db < kDB; ++db) voff[db] = Gm::v_slot(4 * h + jrow, 4 * db + 2 * dhalf + (c >> 1)) + 8 * (c & 1);
    }

    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    auto tile = [&](int32_t kt, const uint8_t* kt_lds, uint8_t* next_lds) {
      if (kt + 1 < kt_end) {
        issue_tile(kt + 1, next_lds, bid_next);
        bid_next = load_bid(kt + 2);
      }
      const uint8_t* vt_lds = kt_lds + kTileBytes;
      if (wave_active) {
        // S^T of token block b (tile tokens 32 b .. 32 b + 31): result e holds
        // token 32 b + 8 (v / 4) + 4 h + v % 4 of row n.
        f32x16_t st[2];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v) st[b][v] = 0.f;
#pragma unroll
        for (int kk = 0; kk < kKK; ++kk) {
          uint4 ka[2];
#pragma unroll
          for (int b = 0; b < 2; ++b) ka[b] = *reinterpret_cast<const uint4*>(kt_lds + koff[kk] + 32 * b * kRowBytes);
#pragma unroll
          for (int b = 0; b < 2; ++b) st[b] = M::mm32(ka[b], qf[kk], st[b]);
        }

        float x[2][16];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v) x[b][v] = st[b][v];
        if (kt * kTile + kTile - 1 > qpos_min_wave) {  // the tile crosses the wave's diagonal
          const int32_t lim = qpos - (kt * kTile + 4 * h);  // visible iff 32 b + 8 (v / 4) + v % 4 <= lim
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v)
              if (32 * b + 8 * (v >> 2) + (v & 3) > lim) x[b][v] = -INFINITY;
        }
        float mx[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          mx[u] = fmaxf(fmaxf(x[u >> 2][4 * (u & 3)], x[u >> 2][4 * (u & 3) + 1]),
                        fmaxf(x[u >> 2][4 * (u & 3) + 2], x[u >> 2][4 * (u & 3) + 3]));
        float tmax = fmaxf(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3])), fmaxf(fmaxf(mx[4], mx[5]), fmaxf(mx[6], mx[7])));
        {
          const uint32_t u = __float_as_uint(tmax);
          const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);  // the other half's max
          tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * a.scale_log2e;
        }
        float alpha = 1.f;
        if (tmax > m + kRescaleSlack) {
          alpha = __builtin_amdgcn_exp2f(m - tmax);  // 0 on the first visible tile
          m = tmax;
        }
        const float msub = m == -INFINITY ? 0.f : m;
        // P^T operand of PV step (b, s): tile tokens 32 b + 16 s .. + 15, the
        // lane's 8 being results 8 s .. 8 s + 7 of S^T block b.
        uint4 pb[2][2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          float p[16];
#pragma unroll
          for (int v = 0; v < 16; ++v) p[v] = __builtin_amdgcn_exp2f(fmaf(x[b][v], a.scale_log2e, -msub));
#pragma unroll
          for (int sq = 0; sq < 2; ++sq)
            pb[b][sq] = make_uint4(M::pk(p[8 * sq], p[8 * sq + 1]), M::pk(p[8 * sq + 2], p[8 * sq + 3]),
                                   M::pk(p[8 * sq + 4], p[8 * sq + 5]), M::pk(p[8 * sq + 6], p[8 * sq + 7]));
        }
        if (__any(alpha != 1.f)) {  // wave-uniform, rare after the first tiles
          lsum *= alpha;
#pragma unroll
          for (int db = 0; db < kDB; ++db) o[db] *= alpha;
        }
        // the row sum of the rounded P that enters PV
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int sq = 0; sq < 2; ++sq) {
            lsum = M::dot1(pb[b][sq].x, lsum);
            lsum = M::dot1(pb[b][sq].y, lsum);
            lsum = M::dot1(pb[b][sq].z, lsum);
            lsum = M::dot1(pb[b][sq].w, lsum);
          }

        // O^T += V^T . P^T: for step (b, s) the lane's V^T operand is head dim
        // 32 db + n of tokens 32 b + 16 s + 4 h + 0..3 and + 8 (two transposed reads).
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int sq = 0; sq < 2; ++sq)
#pragma unroll
            for (int db = 0; db < kDB; ++db) {
              const i16x4_t lo = lds_read_tr16(vt_lds + voff[db] + (32 * b + 16 * sq) * kRowBytes);
              const i16x4_t hi = lds_read_tr16(vt_lds + voff[db] + (32 * b + 16 * sq + 8) * kRowBytes);
              const uint4 va = __builtin_bit_cast(uint4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
              o[db] = M::mm32(va, pb[b][sq], o[db]);
            }
      }
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // next tile landed everywhere; this stage is free again
    };
    for (int32_t kt = kt_begin; kt < kt_end; kt += 2) {
      tile(kt, lds0, lds1);
      if (kt + 1 < kt_end) tile(kt + 1, lds1, lds0);
    }
    if (!wave_active) return;

    // O^T block db result v: head dim 32 db + 8 (v / 4) + 4 h + v % 4 of row n
    const uint32_t lu = __float_as_uint(lsum);
    const auto lsw = __builtin_amdgcn_permlane32_swap(lu, lu, false, false);
    const float l = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
    if (!row_valid) return;
    if (cascade) {  // split-K partials (O unnormalised, m in log2 units, l) of every member row
      if constexpr (D == kD) {  // cascades run at head_dim 128 only
        float* pe = a.ws_pre + ((static_cast<int64_t>(slot) * a.Hkv + g) * kCascadeRows + rho_n) * kPartFloats;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            *reinterpret_cast<float4*>(pe + 32 * db + 8 * i + 4 * h) =
                make_float4(o[db][4 * i], o[db][4 * i + 1], o[db][4 * i + 2], o[db][4 * i + 3]);
        if (h == 0) {
          pe[D] = m;
          pe[D + 1] = l;
        }
      }
      return;
    }
    const int32_t i_q = rho_n / a.G, hg = rho_n - (rho_n / a.G) * a.G;
    uint16_t* orow = a.out + ((static_cast<int64_t>(q0) + i_q) * a.Hq + g * a.G + hg) * D;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint2*>(orow + 32 * db + 8 * i + 4 * h) =
            make_uint2(M::pk(o[db][4 * i] * inv, o[db][4 * i + 1] * inv),
                       M::pk(o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv));
  }
}

}  // namespace

static int64_t prefill_entries_cap(int32_t S, int32_t T, int32_t G) {
  return (static_cast<int64_t>(T) * G + kRowsPerWG - 1) / kRowsPerWG + S;
}

PlanLayout plan_layout(int32_t S, int32_t T, int32_t G, int32_t P, bool prefill_on, bool cascade_on) {
  PlanLayout l;
  l.cap_groups = cascade_on ? kCascadeEntries : 0;
  const int64_t cap = (prefill_on ? prefill_entries_cap(S, T, G) : 0) + (cascade_on ? kCascadeEntries : 0);
  l.cap_entries = static_cast<int32_t>(cap > INT32_MAX ? INT32_MAX : cap);
  l.groups_off = (static_cast<size_t>(kPlanHeader) * 4 + static_cast<size_t>(cap) * 8 + 15) & ~static_cast<size_t>(15);
  l.seqpre_off = l.groups_off + static_cast<size_t>(l.cap_groups) * 16;
  l.members_off = l.seqpre_off + (cascade_on ? static_cast<size_t>(S) * 16 : 0);
  l.match_off = (l.members_off + (cascade_on ? static_cast<size_t>(S) * 4 : 0) + 7) & ~static_cast<size_t>(7);
  l.dec_off = (l.match_off + (cascade_on ? static_cast<size_t>(S) * 8 : 0) + 15) & ~static_cast<size_t>(15);
  l.cap_dec = static_cast<int64_t>(S) * P;
  l.bytes = l.dec_off + static_cast<size_t>(2 * l.cap_dec) * 8;
  return l;
}

bool cascade_possible(int32_t S, int32_t max_seqlen) {
  return S >= 2 && S <= kCascadeMaxSeqs && max_seqlen >= 2 * kCascadeMinTiles * kTile;
}

hipError_t launch_attn_plan(const AttnArgs& a, int32_t rows_cap, int32_t P, bool prefill_on, bool cascade_on,
                            const int32_t dec_slots[2], int32_t* plan, const WriteJob* w, hipStream_t stream) {
  const int32_t G = a.Hq / a.Hkv;
  const PlanLayout l = plan_layout(a.S, a.T, G, P, prefill_on, cascade_on);
  PlanArgs p;
  p.qsl = a.qsl;
  p.seq_lens = a.seq_lens;
  p.block_tables = a.block_tables;
  p.S = a.S;
  p.T = a.T;
  p.G = G;
  p.MB = a.MB;
  p.bs = a.bs;
  p.rows_cap = rows_cap;
  p.prefill_on = prefill_on;
  p.cascade_on = cascade_on;
  p.cap_entries = l.cap_entries;
  p.cap_groups = l.cap_groups;
  p.plan = plan;
  p.groups = reinterpret_cast<int4*>(reinterpret_cast<uint8_t*>(plan) + l.groups_off);
  p.seq_prefix = reinterpret_cast<int4*>(reinterpret_cast<uint8_t*>(plan) + l.seqpre_off);
  p.members = reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(plan) + l.members_off);
  int2* match = reinterpret_cast<int2*>(reinterpret_cast<uint8_t*>(plan) + l.match_off);
  p.match = match;
  p.P = P;
  p.max_q = a.max_qlen;
  p.dec_slots[0] = dec_slots[0];
  p.dec_slots[1] = dec_slots[1];
  p.cap_dec = l.cap_dec;
  p.dec = reinterpret_cast<int2*>(reinterpret_cast<uint8_t*>(plan) + l.dec_off);
  p.d_err = a.d_err;
  p.wk = w ? static_cast<const char*>(w->k) : nullptr;
  p.wv = w ? static_cast<const char*>(w->v) : nullptr;
  p.wslot = w ? w->slot_mapping : nullptr;
  p.wk_cache = w ? static_cast<char*>(w->k_cache) : nullptr;
  p.wv_cache = w ? static_cast<char*>(w->v_cache) : nullptr;
  p.w_row_bytes = w ? w->row_bytes : 0;
  p.w_num_slots = w ? w->num_slots : 0;
  p.w_err = w ? w->d_err : nullptr;
  p.wT = w && w->row_bytes > 0 ? w->T : 0;
  if (cascade_on) {
    MatchArgs m;
    m.qsl = a.qsl;
    m.seq_lens = a.seq_lens;
    m.block_tables = a.block_tables;
    m.S = a.S;
    m.MB = a.MB;
    m.bs = a.bs;
    m.thr_blocks = ceil_div(kCascadeMinTiles * kTile, a.bs);
    m.match = match;
    launch_mark("cascade_match_kernel", stream);
    cascade_match_kernel<<<static_cast<uint32_t>(a.S), kMatchThreads, 0, stream>>>(m);
    launch_done(stream);
  }
  const int64_t wgs = 1 + (static_cast<int64_t>(p.wT) + kPlanThreads / 64 - 1) / (kPlanThreads / 64);
  launch_mark("attn_plan_kernel", stream);
  attn_plan_kernel<<<static_cast<uint32_t>(wgs), kPlanThreads, 0, stream>>>(p);
  launch_done(stream);
  return hipGetLastError();
}

hipError_t launch_attn_prefill(const AttnArgs& a, int32_t rows_cap, int32_t P, bool prefill_on, bool cascade_on,
                               const int32_t* plan, float* ws_pre, size_t lds_pad, hipStream_t stream) {
  PrefillArgs p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k_cache = static_cast<const uint16_t*>(a.k_cache);
  p.v_cache = static_cast<const uint16_t*>(a.v_cache);
  p.block_tables = a.block_tables;
  p.qsl = a.qsl;
  p.seq_lens = a.seq_lens;
  p.S = a.S;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.G = a.Hq / a.Hkv;
  p.NB = a.NB;
  p.MB = a.MB;
  p.bs = a.bs;
  p.min_rows = rows_cap;
  p.scale_log2e = a.scale * 1.4426950408889634f;
  p.out = static_cast<uint16_t*>(a.out);
  p.d_err = a.d_err;
  const PlanLayout l = plan_layout(a.S, a.T, p.G, P, prefill_on, cascade_on);
  p.plan = plan;
  p.groups = reinterpret_cast<const int4*>(reinterpret_cast<const uint8_t*>(plan) + l.groups_off);
  p.members = reinterpret_cast<const int32_t*>(reinterpret_cast<const uint8_t*>(plan) + l.members_off);
  p.ws_pre = ws_pre;
  p.prio = lds_pad > 0 ? 1 : 0;
  const int64_t n_eb = (static_cast<int64_t>(l.cap_entries) + kQtRun - 1) / kQtRun;
  const int64_t items_raw = n_eb * kQtRun * a.Hkv;
  const int64_t run_len = static_cast<int64_t>(kQtRun) * prefill_head_group(a.Hkv);
  const int64_t items = (items_raw + 8 * run_len - 1) / (8 * run_len) * (8 * run_len);
  if (items > INT32_MAX) return hipErrorInvalidValue;
  if (items == 0) return hipSuccess;
  launch_mark("prefill_kernel", stream);
  const uint32_t grid = static_cast<uint32_t>(items);
  const bool blk16 = a.bs % 16 == 0;
#define PA_PREFILL_D(DD)                                                                             \
  if (blk16) {                                                                                       \
    if (a.dtype == PA_BF16) prefill_kernel<BF16, true, DD><<<grid, kThreads, lds_pad, stream>>>(p);        \
    else prefill_kernel<F16, true, DD><<<grid, kThreads, lds_pad, stream>>>(p);                            \
  } else {                                                                                           \
    if (a.dtype == PA_BF16) prefill_kernel<BF16, false, DD><<<grid, kThreads, lds_pad, stream>>>(p);       \
    else prefill_kernel<F16, false, DD><<<grid, kThreads, lds_pad, stream>>>(p);                           \
  }
  if (a.D == 64) {
    PA_PREFILL_D(64)
  } else if (a.D == 256) {
    PA_PREFILL_D(256)
  } else {
    PA_PREFILL_D(128)
  }
#undef PA_PREFILL_D
  launch_done(stream);
  return hipGetLastError();
}

}  // namespace pa

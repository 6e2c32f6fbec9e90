"""CPU oracle for ragged paged attention.  TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may
import or call this module.  The product path (the HIP library and its Python
binding) never does, and this module imports nothing from it.

It is the plain definition of what the hot path computes, in float64 NumPy,
written for a reader to check against the pages by eye.  Page references:

  [FS]  "vLLM Continuous Batching：从 Forward Shape 理解两个核心参数"
  [VP]  "vLLM 原理"
  [CB]  "LLM 推理引擎 Continuous Batching 与 PagedAttention：从 vLLM 原理到生产级部署实战"
  [BN]  "vLLM 学习笔记（2）：从单请求到批处理"

Readings taken where the pages leave a point open (each is listed in the
design notes with its justification):
  * seq_lens[s] is the KV length of sequence s after this step's rows are
    written, new rows included ([FS] §2.1: B = 7 cached + b7 -> 8).
  * The i-th new row of a sequence with query_len q and seq_len L sits at
    position L - q + i and sees positions 0 .. L - q + i ([FS] §2.1 positions
    [7,2,0,1,2,3,4]; [FS] §2.3 causal rule; [VP] §3.7: seqlen_k is the whole
    sequence length).
  * Query head h reads KV head h // (Hq / Hkv) (grouped heads; the pages give
    only the shapes Q [T, n_q_heads, D], K/V [T, n_kv_heads, D], [FS] §2.2).
  * A slot is the integer block * block_size + offset ([VP] §3.7: the pool has
    num_blocks*block_size slots; [FS] §2.3 第一步 physical_slot(block=21,
    slot=3)); a negative slot means "do not write".
  * The cache of one layer is [num_blocks, block_size, num_kv_heads, head_dim],
    K and V separate ([VP] §3.6, kv_cache[0, layer] / kv_cache[1, layer]).
  * A sequence with query_len 0 contributes no rows; query_len > seq_len is
    invalid input.  Duplicate non-negative slots in one write are invalid.
  * Softmax scale is an argument (1/sqrt(head_dim) in every workload here).

Nothing here is parity-unpinned: tests/test_oracle_pins.py pins every
function against the pages' worked examples, closed forms, a library routine
(dense padded masked attention) and brute force; the 16-bit widening is
pinned on all 65,536 bit patterns against the bfloat16 / binary16 bit-field
definitions and torch's own conversions.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

INT32_MAX = 2**31 - 1


class OracleInputError(ValueError):
    """The batch violates a rule the method relies on."""


# ---------------------------------------------------------------------------
# dtype handling: stored values -> exact float64
# ---------------------------------------------------------------------------
def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact conversion of stored values to float64.

    f32 is stored as float32; bf16 and f16 as uint16 bit patterns.  A bf16
    value is the top half of the float32 with the same sign/exponent/mantissa
    bits, so shifting it left by 16 gives that float32 exactly."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(a, dtype=np.uint16).view(np.float16).astype(np.float64)
    raise OracleInputError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# metadata ([FS] §2.1, §2.3 第一步 and 第二步; [BN] query_start_loc example;
# [VP] §3.7 cu_seqlens and block_tables)
# ---------------------------------------------------------------------------
def prefix_offsets(lengths: Sequence[int]) -> np.ndarray:
    """Start offset of each entry in the flat array, with the total appended:
    entry s owns [out[s], out[s+1]).  ([BN]: lengths 3, 5, 2 -> [0, 3, 8, 10];
    the last value is the total, not a start.)"""
    out = np.zeros(len(lengths) + 1, dtype=np.int64)
    total = 0
    for s, n in enumerate(lengths):
        total += int(n)
        out[s + 1] = total
    if total > INT32_MAX:
        raise OracleInputError("offsets overflow int32")
    return out


def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head h: consecutive groups of Hq/Hkv query heads
    share one KV head."""
    return h // (num_q_heads // num_kv_heads)


def position_of(seq_len: int, query_len: int, i: int) -> int:
    """Position inside its sequence of the i-th new row ([FS] §2.1)."""
    return seq_len - query_len + i


def slot_of(block_table_row: np.ndarray, pos: int, block_size: int) -> int:
    """Paged address of a position ([FS] §2.3补充 第二步, the addressing chain):
    logical block pos // block_size -> physical block via the table ->
    slot physical * block_size + pos % block_size."""
    physical = int(block_table_row[pos // block_size])
    return physical * block_size + pos % block_size


@dataclass
class Metadata:
    query_start_loc: np.ndarray   # int32 [S+1]
    seq_start_loc: np.ndarray     # int32 [S+1]
    positions: np.ndarray         # int32 [T]
    token_to_seq: np.ndarray      # int32 [T]
    slot_mapping: Optional[np.ndarray]  # int32 [T] or None
    stats: np.ndarray             # int32 [6]: n_decode, n_prefill, n_decode_tokens,
                                  #            n_prefill_tokens, max_query_len, max_seq_len


def check_batch(query_lens, seq_lens, num_tokens, block_tables=None, block_size=None, num_blocks=None):
    """Raise OracleInputError unless the batch is well formed."""
    ql = np.asarray(query_lens, dtype=np.int64)
    sl = np.asarray(seq_lens, dtype=np.int64)
    if ql.shape != sl.shape or ql.ndim != 1:
        raise OracleInputError("query_lens and seq_lens must be 1-D and equal length")
    if (ql < 0).any() or (sl < 0).any():
        raise OracleInputError("negative length")
    if (ql > sl).any():
        raise OracleInputError("query_len exceeds seq_len")
    if int(ql.sum()) != int(num_tokens):
        raise OracleInputError("query_lens do not sum to num_tokens")
    if block_tables is not None:
        bt = np.asarray(block_tables)
        if bt.shape[0] != ql.shape[0]:
            raise OracleInputError("block_tables rows != num_seqs")
        for s in range(len(sl)):
            used = -(-int(sl[s]) // block_size)
            if used > bt.shape[1]:
                raise OracleInputError(f"sequence {s} needs {used} blocks, table has {bt.shape[1]}")
            row = bt[s, :used]
            if ((row < 0) | (row >= num_blocks)).any():
                raise OracleInputError(f"sequence {s} has an invalid physical block in its used range")


def build_metadata(query_lens, seq_lens, num_tokens, block_tables=None, block_size=None,
                   num_blocks=None) -> Metadata:
    """Flat-batch metadata for one step ([FS] §2.1 table of fields; §2.3)."""
    check_batch(query_lens, seq_lens, num_tokens, block_tables, block_size, num_blocks)
    ql = [int(x) for x in query_lens]
    sl = [int(x) for x in seq_lens]
    qsl = prefix_offsets(ql)
    ssl = prefix_offsets(sl)
    T = int(num_tokens)
    positions = np.zeros(T, dtype=np.int64)
    token_to_seq = np.zeros(T, dtype=np.int64)
    slots = np.zeros(T, dtype=np.int64) if block_tables is not None else None
    for s in range(len(ql)):
        for i in range(ql[s]):
            t = int(qsl[s]) + i
            pos = position_of(sl[s], ql[s], i)
            positions[t] = pos
            token_to_seq[t] = s
            if slots is not None:
                slots[t] = slot_of(np.asarray(block_tables)[s], pos, block_size)
    if slots is not None and len(slots) and slots.max() > INT32_MAX:
        raise OracleInputError("slot overflows int32")
    n_dec = sum(1 for q in ql if q == 1)
    n_pre = sum(1 for q in ql if q > 1)
    stats = np.array([
        n_dec, n_pre,
        sum(q for q in ql if q == 1), sum(q for q in ql if q > 1),
        max(ql, default=0), max(sl, default=0),
    ], dtype=np.int32)
    return Metadata(qsl.astype(np.int32), ssl.astype(np.int32), positions.astype(np.int32),
                    token_to_seq.astype(np.int32),
                    None if slots is None else slots.astype(np.int32), stats)


# ---------------------------------------------------------------------------
# KV write ([FS] §2.3 第一步; [VP] §3.7 store_kvcache before attention)
# ---------------------------------------------------------------------------
def write_kv(k_new: np.ndarray, v_new: np.ndarray, slot_mapping: np.ndarray,
             k_cache: np.ndarray, v_cache: np.ndarray) -> None:
    """In place: row t of k_new/v_new goes to slot slot_mapping[t] of the pool
    (block slot // block_size, offset slot % block_size).  Negative slots are
    skipped.  A pure copy: stored bits are moved unchanged."""
    num_blocks, block_size = k_cache.shape[0], k_cache.shape[1]
    sm = np.asarray(slot_mapping, dtype=np.int64)
    live = sm[sm >= 0]
    if (live >= num_blocks * block_size).any():
        raise OracleInputError("slot out of range")
    if len(np.unique(live)) != len(live):
        raise OracleInputError("duplicate slot in one write")
    for t in range(len(sm)):
        if sm[t] < 0:
            continue
        b, o = divmod(int(sm[t]), block_size)
        k_cache[b, o] = k_new[t]
        v_cache[b, o] = v_new[t]


# ---------------------------------------------------------------------------
# block copies ([VP] §2.1 copy-on-write; [CB] §4.4 swap)
# ---------------------------------------------------------------------------
def copy_blocks(src_k: np.ndarray, src_v: np.ndarray, dst_k: np.ndarray, dst_v: np.ndarray, pairs) -> None:
    """In place: for each (source, destination) pair, the destination block of
    both pools receives the source block's K and V, bit for bit.  A
    destination written twice, or used as a source too, is invalid."""
    pairs = [(int(a), int(b)) for a, b in np.asarray(pairs).reshape(-1, 2)]
    dsts = [d for _, d in pairs]
    if len(set(dsts)) != len(dsts):
        raise OracleInputError("a destination block appears twice")
    if src_k is dst_k and set(dsts) & {s for s, _ in pairs}:
        raise OracleInputError("a block is both a source and a destination")
    for s_, d_ in pairs:
        if not (0 <= s_ < src_k.shape[0]) or not (0 <= d_ < dst_k.shape[0]):
            raise OracleInputError("block id out of range")
    staged = [(d_, src_k[s_].copy(), src_v[s_].copy()) for s_, d_ in pairs]
    for d_, kb, vb in staged:
        dst_k[d_] = kb
        dst_v[d_] = vb


# ---------------------------------------------------------------------------
# attention ([FS] §2.3 and §2.3补充 第二步; [VP] §1.1 and §3.7)
# ---------------------------------------------------------------------------
def gather_sequence(cache: np.ndarray, block_table_row: np.ndarray, seq_len: int, dtype: str) -> np.ndarray:
    """Logical [seq_len, Hkv, D] rows of one sequence, read through its block
    table (position j lives in physical block table[j // bs], offset j % bs),
    widened exactly to float64."""
    block_size = cache.shape[1]
    rows = np.empty((seq_len,) + cache.shape[2:], dtype=cache.dtype)
    for j in range(seq_len):
        rows[j] = cache[int(block_table_row[j // block_size]), j % block_size]
    return widen(rows, dtype)


def softmax_weighted_sum(scores: np.ndarray, values: np.ndarray) -> np.ndarray:
    """sum_j e^{x_j - max x} v_j / sum_j e^{x_j - max x} over the last axis of
    `scores` ([G, n]) against values [n, D]."""
    m = scores.max(axis=-1, keepdims=True)
    w = np.exp(scores - m)
    return (w @ values) / w.sum(axis=-1, keepdims=True)


def attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_tables: np.ndarray,
              query_start_loc: np.ndarray, seq_lens: np.ndarray, num_kv_heads: int, scale: float,
              dtype: str, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Ragged causal paged attention, float64.

    For every sequence s (rows query_start_loc[s] .. query_start_loc[s+1]-1 of
    the flat batch), every new row i at position p = seq_len - query_len + i
    and every query head h with KV head g = kv_head_of(h):
        x_j = scale * <q[t, h], K_s[j, g]>   for j = 0 .. p
        o[t, h] = sum_j e^{x_j - max x} V_s[j, g] / sum_j e^{x_j - max x}
    where K_s, V_s are sequence s's logical rows read through its block
    table.  Attention never leaves the sequence ([FS] §0 item 4).

    `rows` limits the result to the listed flat rows (returned in that order);
    by default every row is computed.
    """
    T, Hq, D = q.shape
    if Hq % num_kv_heads:
        raise OracleInputError("num_q_heads must be a multiple of num_kv_heads")
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    sl = np.asarray(seq_lens, dtype=np.int64)
    S = len(sl)
    if qsl[S] != T:
        raise OracleInputError("query_start_loc does not end at num_tokens")
    wanted = list(range(T)) if rows is None else [int(r) for r in rows]
    out = np.zeros((len(wanted), Hq, D), dtype=np.float64)
    where = {}
    for n, t in enumerate(wanted):
        where.setdefault(t, []).append(n)
    for s in range(S):
        t0, t1 = int(qsl[s]), int(qsl[s + 1])
        mine = [t for t in range(t0, t1) if t in where]
        if not mine:
            continue
        L, qlen = int(sl[s]), t1 - t0
        if qlen > L:
            raise OracleInputError("query_len exceeds seq_len")
        K = gather_sequence(k_cache, block_tables[s], L, dtype)
        V = gather_sequence(v_cache, block_tables[s], L, dtype)
        for t in mine:
            p = position_of(L, qlen, t - t0)
            qt = widen(q[t], dtype)
            o = np.zeros((Hq, D), dtype=np.float64)
            for h in range(Hq):
                g = kv_head_of(h, Hq, num_kv_heads)
                x = scale * (K[:p + 1, g] @ qt[h])
                o[h] = softmax_weighted_sum(x[None, :], V[:p + 1, g])[0]
            for n in where[t]:
                out[n] = o
    return out


# ---------------------------------------------------------------------------
# a whole step, as the pages order it: metadata, write, then attend
# ([FS] §2.3: "it does two things"; [VP] §3.7 Attention.forward)
# ---------------------------------------------------------------------------
def empty_pool(shape, dtype: str, fill) -> np.ndarray:
    arr = np.empty(shape, dtype=np.float32 if dtype == "f32" else np.uint16)
    arr.fill(fill)
    return arr


def fill_history(hist, k_cache, v_cache, block_size: int) -> None:
    """Write rows cached before the step (a batch of writes) into the pool."""
    if hist.num_seqs == 0:
        return
    md = build_metadata(hist.query_lens, hist.seq_lens, hist.num_tokens, hist.block_tables,
                        block_size, k_cache.shape[0])
    write_kv(hist.k, hist.v, md.slot_mapping, k_cache, v_cache)


def run_step(w, rows: Optional[Sequence[int]] = None):
    """Oracle result for a workload: (metadata, k_cache, v_cache, out fp64)."""
    shape = w.pool_shape()
    k_cache = empty_pool(shape, w.dtype, w.pool_fill())
    v_cache = empty_pool(shape, w.dtype, w.pool_fill())
    fill_history(w.hist, k_cache, v_cache, w.block_size)
    st = w.step
    md = build_metadata(st.query_lens, st.seq_lens, st.num_tokens, st.block_tables,
                        w.block_size, w.num_blocks)
    write_kv(st.k, st.v, md.slot_mapping, k_cache, v_cache)
    out = attention(w.q, k_cache, v_cache, st.block_tables, md.query_start_loc, st.seq_lens,
                    w.num_kv_heads, w.scale, w.dtype, rows=rows)
    return md, k_cache, v_cache, out

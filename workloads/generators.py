"""Seeded synthetic inputs for ragged paged attention.

This module only *describes* a batch: lengths, which physical KV blocks each
sequence owns, and the random values of every K/V/Q row.  It performs none of
the method's arithmetic: no prefix sums, no position or slot computation, no
placement of rows into the paged pool and no attention.  Both the GPU path and
the CPU oracle consume the same `Workload` object and do that work themselves.

History (the K/V of tokens cached before the current step) is described as a
second batch of writes, `Workload.hist`, in the same vocabulary as the step
itself (query_lens / seq_lens / block_tables / k / v): "write these rows for
positions seq_len - query_len .. seq_len - 1 of this block table".  Each side
turns that into slots with its own metadata code and scatters it with its own
write code.  Shared prefixes (blocks with a reference count above one, as in
the prefix-sharing discussion of "vLLM 原理" §2.1 and §2.3) are written once,
by one history entry, and referenced by every block table of the group.

Value recipe: every Q/K/V element is an independent N(0, 1) draw in float32
from numpy's PCG64 generator seeded with `seed`, rounded once to the storage
dtype with round-to-nearest-even.  16-bit dtypes are stored as uint16 bit
patterns.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

DTYPES = ("f32", "bf16", "f16")


# --------------------------------------------------------------------------
# value generation
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Inputs here are finite normal draws, so no NaN/Inf handling is needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f16":
        return np.ascontiguousarray(x.astype(np.float16)).view(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def _normal(rng: np.random.Generator, shape, dtype: str, chunk_rows: int = 1 << 14) -> np.ndarray:
    """N(0,1) float32 draws rounded to `dtype`, generated in row chunks so that
    multi-GB history tensors never exist as float32 in full."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.float32 if dtype == "f32" else np.uint16)
    if shape[0] == 0:
        return out
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        out[r0:r1] = _store(rng.standard_normal((r1 - r0,) + shape[1:], dtype=np.float32), dtype)
    return out


def poison_value(dtype: str):
    """Bit pattern used to fill pool slots that no write reaches (a quiet NaN)."""
    if dtype == "f32":
        return np.float32(np.nan)
    if dtype == "bf16":
        return np.uint16(0x7FC0)
    if dtype == "f16":
        return np.uint16(0x7E00)
    raise ValueError(dtype)


def storage_dtype(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


# --------------------------------------------------------------------------
# batch description
# --------------------------------------------------------------------------
@dataclass
class Batch:
    """One batch of rows to attend or to write, in the pages' vocabulary."""
    query_lens: np.ndarray      # int32 [S]   new rows per sequence
    seq_lens: np.ndarray        # int32 [S]   KV length after the rows are in place
    block_tables: np.ndarray    # int32 [S, MB], -1 beyond the used blocks
    k: np.ndarray               # [sum(query_lens), Hkv, D] storage dtype
    v: np.ndarray               # [sum(query_lens), Hkv, D]

    @property
    def num_seqs(self) -> int:
        return int(self.query_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.k.shape[0])


@dataclass
class Workload:
    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    step: Batch                 # this step's new tokens (k/v are the new rows)
    q: np.ndarray               # [T, Hq, D] storage dtype
    hist: Batch                 # rows cached before the step
    # hist_segments[s] = indices of `hist` entries whose rows, concatenated in
    # order, are sequence s's history (positions 0 .. seq_len - query_len - 1).
    hist_segments: List[List[int]] = field(default_factory=list)
    seed: int = 0
    poison: bool = True
    notes: str = ""

    # --- convenience -----------------------------------------------------
    @property
    def num_seqs(self) -> int:
        return self.step.num_seqs

    @property
    def num_tokens(self) -> int:
        return self.step.num_tokens

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.step.block_tables.shape[1])

    @property
    def max_query_len(self) -> int:
        return int(self.step.query_lens.max(initial=0))

    @property
    def max_seq_len(self) -> int:
        return int(self.step.seq_lens.max(initial=0))

    def pool_shape(self):
        return (self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim)

    def pool_fill(self):
        return poison_value(self.dtype) if self.poison else storage_dtype(self.dtype)(0)

    def hist_row_offsets(self) -> np.ndarray:
        """Start row of each `hist` entry inside hist.k / hist.v (a plain running
        count over entries, used only to slice the generator's own arrays)."""
        return np.concatenate([[0], np.cumsum(self.hist.query_lens, dtype=np.int64)])

    def new_row_offsets(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.step.query_lens, dtype=np.int64)])

    def logical_kv(self, s: int):
        """Sequence s's full K and V in position order (history then new rows),
        straight from the generator's arrays, with no paging involved."""
        ho = self.hist_row_offsets()
        ks = [self.hist.k[ho[e]:ho[e + 1]] for e in self.hist_segments[s]]
        vs = [self.hist.v[ho[e]:ho[e + 1]] for e in self.hist_segments[s]]
        no = self.new_row_offsets()
        ks.append(self.step.k[no[s]:no[s + 1]])
        vs.append(self.step.v[no[s]:no[s + 1]])
        return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)

    def kv_bytes_logical(self) -> int:
        """Bytes of K and V one attention pass reads: every sequence's full
        context, once per KV head."""
        es = 4 if self.dtype == "f32" else 2
        return int(self.step.seq_lens.astype(np.int64).sum()) * 2 * self.num_kv_heads * self.head_dim * es

    def summary(self) -> dict:
        ql = self.step.query_lens
        return {
            "name": self.name, "dtype": self.dtype, "S": self.num_seqs, "T": self.num_tokens,
            "Hq": self.num_q_heads, "Hkv": self.num_kv_heads, "D": self.head_dim,
            "block_size": self.block_size, "num_blocks": self.num_blocks,
            "n_decode": int((ql == 1).sum()), "n_prefill": int((ql > 1).sum()),
            "max_seq_len": self.max_seq_len, "seed": self.seed,
        }


# --------------------------------------------------------------------------
# builders
# --------------------------------------------------------------------------
def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def _pad_tables(rows: Sequence[Sequence[int]], width: Optional[int] = None) -> np.ndarray:
    width = max([len(r) for r in rows] + [1]) if width is None else width
    bt = np.full((len(rows), width), -1, dtype=np.int32)
    for i, r in enumerate(rows):
        bt[i, :len(r)] = r
    return bt


def build_workload(name, dtype, Hq, Hkv, D, bs, NB, query_lens, seq_lens, tables,
                   seed, rng=None, shared=None, poison=True, notes="") -> Workload:
    """Generic builder.

    tables[s]   : physical block ids for sequence s's logical blocks (enough to
                  hold seq_lens[s] tokens).
    shared      : optional list of (member_seqs, prefix_tokens).  The first
                  `prefix_tokens` positions of every member are served by ONE
                  history entry (written once through the first member's table,
                  whose leading blocks all members share); members' remaining
                  history is private.
    """
    rng = np.random.default_rng(seed) if rng is None else rng
    S = len(query_lens)
    query_lens = np.asarray(query_lens, dtype=np.int32)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    assert (query_lens <= seq_lens).all() and (query_lens >= 0).all()
    bt = _pad_tables(tables)
    T = int(query_lens.sum())
    q = _normal(rng, (T, Hq, D), dtype)
    k_new = _normal(rng, (T, Hkv, D), dtype)
    v_new = _normal(rng, (T, Hkv, D), dtype)

    # history entries: (hist query_len, hist seq_len, table row)
    h_q, h_l, h_rows = [], [], []
    segments: List[List[int]] = [[] for _ in range(S)]
    prefix_of = {}
    for members, ptoks in (shared or []):
        e = len(h_q)
        h_q.append(ptoks); h_l.append(ptoks); h_rows.append(tables[members[0]])
        for m in members:
            prefix_of[m] = (e, ptoks)
    for s in range(S):
        ctx = int(seq_lens[s] - query_lens[s])
        start = 0
        if s in prefix_of:
            e, ptoks = prefix_of[s]
            assert ptoks <= ctx
            segments[s].append(e)
            start = ptoks
        if ctx > start:
            segments[s].append(len(h_q))
            h_q.append(ctx - start); h_l.append(ctx); h_rows.append(tables[s])
    Th = int(sum(h_q))
    hist = Batch(
        query_lens=np.asarray(h_q, dtype=np.int32),
        seq_lens=np.asarray(h_l, dtype=np.int32),
        block_tables=_pad_tables(h_rows, bt.shape[1]) if h_rows else np.full((0, bt.shape[1]), -1, np.int32),
        k=_normal(rng, (Th, Hkv, D), dtype),
        v=_normal(rng, (Th, Hkv, D), dtype),
    )
    step = Batch(query_lens=query_lens, seq_lens=seq_lens, block_tables=bt, k=k_new, v=v_new)
    return Workload(name=name, dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                    block_size=bs, num_blocks=NB, step=step, q=q, hist=hist,
                    hist_segments=segments, seed=seed, poison=poison, notes=notes)


def _shrunk_pool(NB, counts, f):
    """Pool size for a scaled-down config: 1/f of the full pool, never fewer
    than the blocks the batch needs plus a few spares."""
    return NB if f <= 1 else max(NB // f, int(sum(counts)) + 8)


def _place(rng, NB, counts):
    """Distinct physical ids drawn at random from the pool, handed out in order."""
    ids = rng.permutation(NB)[: int(sum(counts))]
    out, o = [], 0
    for c in counts:
        out.append([int(x) for x in ids[o:o + c]])
        o += c
    return out


CONFIG_NAMES = {
    1: "tiny_mixed",
    2: "ragged_prefill",
    3: "decode",
    4: "chunked_mixed",
    5: "shared_prefix_decode",
}


def config(n: int, seed: Optional[int] = None, dtype: Optional[str] = None, poison: bool = True,
           scale_down: int = 1, block_size: Optional[int] = None) -> Workload:
    """The five workloads (1-based).  `seed` defaults to the config number.

    `scale_down` > 1 shrinks lengths and counts of configs 2-5 (same structure,
    same head shapes) so the oracle finishes in seconds; 1 is the full size.
    `block_size` replaces config 4's 16 (the pool keeps its token capacity).
    """
    seed = n if seed is None else seed
    rng = np.random.default_rng(seed)
    f = int(scale_down)
    if n == 1:
        # Sequences B, C, A of the forward-shape walkthrough: B decodes position 7
        # (7 cached), C decodes position 2 (2 cached), A prefills 5 tokens.
        bs, NB = 4, 16
        ql, sl = [1, 1, 5], [8, 3, 5]
        tables = _place(rng, NB, [_ceil_div(L, bs) for L in sl])
        return build_workload("tiny_mixed", dtype or "f32", 2, 2, 16, bs, NB, ql, sl, tables,
                              seed, rng, poison=poison)
    if n == 2:
        bs, NB = 16, 1024
        lens = [16, 128, 1024, 2048]
        if f > 1:
            lens = [max(2, L // f) for L in lens]
        NB = _shrunk_pool(NB, [_ceil_div(L, bs) for L in lens], f)
        tables = _place(rng, NB, [_ceil_div(L, bs) for L in lens])
        return build_workload("ragged_prefill", dtype or "bf16", 32, 32, 128, bs, NB, lens, lens,
                              tables, seed, rng, poison=poison)
    if n == 3:
        bs, NB = 16, 20000
        S, hist_len = 100, 2000
        if f > 1:
            S, hist_len = max(2, S // f), max(1, hist_len // f)
        sl = [hist_len + 1] * S
        NB = _shrunk_pool(NB, [_ceil_div(L, bs) for L in sl], f)
        tables = _place(rng, NB, [_ceil_div(L, bs) for L in sl])
        return build_workload("decode", dtype or "bf16", 32, 32, 128, bs, NB, [1] * S, sl, tables,
                              seed, rng, poison=poison)
    if n == 4:
        bs = block_size or 16
        NB = 40000 * 16 // bs
        n_dec, n_chunk, budget = 240, 16, 8192
        lo, hi, ctx_hi = 128, 8192, 4096
        if f > 1:
            n_dec, n_chunk, budget = max(2, n_dec // f), max(1, n_chunk // f), max(8, budget // f)
            lo, hi, ctx_hi = max(2, lo // f), max(4, hi // f), max(1, ctx_hi // f)
        dec_ctx = np.rint(np.exp(rng.uniform(math.log(lo), math.log(hi), n_dec))).astype(np.int64)
        chunk = (budget - n_dec) // n_chunk
        early = rng.integers(0, ctx_hi + 1, n_chunk)
        ql = [1] * n_dec + [chunk] * n_chunk
        sl = [int(c) for c in dec_ctx] + [int(e) + chunk for e in early]
        NB = _shrunk_pool(NB, [_ceil_div(L, bs) for L in sl], f)
        tables = _place(rng, NB, [_ceil_div(L, bs) for L in sl])
        return build_workload("chunked_mixed", dtype or "bf16", 32, 8, 128, bs, NB, ql, sl, tables,
                              seed, rng, poison=poison,
                              notes=f"{n_dec} decodes + {n_chunk} chunks of {chunk}")
    if n == 5:
        bs, NB = 16, 8192
        groups, per_group, prefix, tail = 4, 16, 16384, 512
        if f > 1:
            per_group, prefix, tail = max(2, per_group // f), max(bs, (prefix // f) // bs * bs), max(2, tail // f)
        S = groups * per_group
        L = prefix + tail
        pb, tb = prefix // bs, _ceil_div(tail, bs)
        NB = _shrunk_pool(NB, [groups * pb + S * tb], f)
        ids = rng.permutation(NB)[: groups * pb + S * tb]
        tables, shared = [], []
        for gi in range(groups):
            pref = [int(x) for x in ids[gi * pb:(gi + 1) * pb]]
            members = []
            for j in range(per_group):
                s = gi * per_group + j
                o = groups * pb + s * tb
                tables.append(pref + [int(x) for x in ids[o:o + tb]])
                members.append(s)
            shared.append((members, prefix))
        return build_workload("shared_prefix_decode", dtype or "bf16", 64, 8, 128, bs, NB,
                              [1] * S, [L] * S, tables, seed, rng, shared=shared, poison=poison)
    raise ValueError(f"no config {n}")


def verify_batch(seed: int = 6, S: int = 64, q_lo: int = 2, q_hi: int = 8, ctx_lo: int = 2048,
                 ctx_hi: int = 16384, Hq: int = 32, Hkv: int = 8, dtype: Optional[str] = None,
                 poison: bool = True, scale_down: int = 1) -> Workload:
    """Speculative-decoding verify batch: each of S sequences feeds its last
    accepted token plus a few draft tokens (query_len uniform in q_lo..q_hi)
    over a cached context of log-uniform length in [ctx_lo, ctx_hi]; 32/8
    heads, head_dim 128, block_size 16, bf16 by default.  `scale_down` > 1
    shrinks S and the context range for oracle-sized runs."""
    rng = np.random.default_rng(seed)
    f = int(scale_down)
    bs, NB = 16, 40000
    if f > 1:
        S, ctx_lo, ctx_hi = max(2, S // f), max(1, ctx_lo // f), max(2, ctx_hi // f)
    ql = rng.integers(q_lo, q_hi + 1, S)
    ctx = np.rint(np.exp(rng.uniform(math.log(ctx_lo), math.log(ctx_hi), S))).astype(np.int64)
    sl = [int(c) + int(q) for c, q in zip(ctx, ql)]
    NB = _shrunk_pool(NB, [_ceil_div(L, bs) for L in sl], f)
    tables = _place(rng, NB, [_ceil_div(L, bs) for L in sl])
    return build_workload("spec_verify", dtype or "bf16", Hq, Hkv, 128, bs, NB, [int(q) for q in ql], sl, tables,
                          seed, rng, poison=poison, notes=f"query_len {q_lo}..{q_hi} over {ctx_lo}..{ctx_hi} tokens")


def decode_variant(D: int, bs: int, seed: int = 3, S: int = 100, hist_len: int = 2000, Hq: int = 32,
                   Hkv: int = 32, dtype: Optional[str] = None, poison: bool = True) -> Workload:
    """The decode batch (S sequences, one new token over `hist_len` cached
    ones, blocks placed at random) at another head_dim / block size: the
    head-dim and block-size variants of the decode path."""
    rng = np.random.default_rng(seed)
    sl = [hist_len + 1] * S
    counts = [_ceil_div(L, bs) for L in sl]
    NB = int(sum(counts)) * 8 // 5
    tables = _place(rng, NB, counts)
    return build_workload(f"decode_d{D}_bs{bs}", dtype or "bf16", Hq, Hkv, D, bs, NB, [1] * S, sl, tables,
                          seed, rng, poison=poison)


def prefill_variant(D: int, bs: int = 16, seed: int = 2, dtype: Optional[str] = None,
                    poison: bool = True) -> Workload:
    """The ragged prefill batch (prompts of 16/128/1024/2048 tokens, 32/32
    heads, blocks placed at random) at another head_dim / block size."""
    rng = np.random.default_rng(seed)
    lens = [16, 128, 1024, 2048]
    counts = [_ceil_div(L, bs) for L in lens]
    NB = int(sum(counts)) * 5
    tables = _place(rng, NB, counts)
    return build_workload(f"ragged_prefill_d{D}_bs{bs}", dtype or "bf16", 32, 32, D, bs, NB, lens, lens,
                          tables, seed, rng, poison=poison)


def random_batch(seed: int, S: int = 3, max_ctx: int = 12, max_q: int = 5, Hq: int = 4, Hkv: int = 2,
                 D: int = 16, bs: int = 4, dtype: str = "f32", extra_blocks: int = 4,
                 decode_frac: float = 0.4, poison: bool = True) -> Workload:
    """Small random ragged batch: mixed decodes (query_len 1) and chunks with
    history; blocks placed at random in a pool with spare blocks."""
    rng = np.random.default_rng(seed)
    ql, sl = [], []
    for _ in range(S):
        if rng.random() < decode_frac:
            q_ = 1
        else:
            q_ = int(rng.integers(1, max_q + 1))
        ctx = int(rng.integers(0, max_ctx + 1))
        ql.append(q_)
        sl.append(ctx + q_)
    counts = [_ceil_div(L, bs) for L in sl]
    NB = int(sum(counts)) + extra_blocks
    tables = _place(rng, NB, counts)
    return build_workload(f"random_{seed}", dtype, Hq, Hkv, D, bs, NB, ql, sl, tables, seed, rng,
                          poison=poison)


def relabel_blocks(w: Workload, perm: np.ndarray) -> Workload:
    """Same logical content, physical block b renamed perm[b] everywhere."""
    perm = np.asarray(perm, dtype=np.int32)

    def mp(bt):
        out = bt.copy()
        m = out >= 0
        out[m] = perm[out[m]]
        return out

    step = Batch(w.step.query_lens, w.step.seq_lens, mp(w.step.block_tables), w.step.k, w.step.v)
    hist = Batch(w.hist.query_lens, w.hist.seq_lens, mp(w.hist.block_tables), w.hist.k, w.hist.v)
    return Workload(w.name + "_relabeled", w.dtype, w.num_q_heads, w.num_kv_heads, w.head_dim,
                    w.block_size, w.num_blocks, step, w.q, hist, [list(x) for x in w.hist_segments],
                    w.seed, w.poison, w.notes)


def unshare(w: Workload, spare_ids: Sequence[int]) -> Workload:
    """Give every sequence a private copy of any block it shares with an earlier
    sequence (fresh ids from `spare_ids`), and write shared prefixes once per
    member instead of once per group.  Logical content is unchanged."""
    S = w.num_seqs
    bt = w.step.block_tables.copy()
    spare = list(int(x) for x in spare_ids)
    seen = set()
    for s in range(S):
        for j in range(bt.shape[1]):
            b = int(bt[s, j])
            if b < 0:
                continue
            if b in seen:
                bt[s, j] = spare.pop(0)
            seen.add(int(bt[s, j]))
    ho = w.hist_row_offsets()
    h_q, h_l, rows, ks, vs, segs = [], [], [], [], [], []
    for s in range(S):
        seg = []
        for e in w.hist_segments[s]:
            seg.append(len(h_q))
            h_q.append(int(w.hist.query_lens[e])); h_l.append(int(w.hist.seq_lens[e]))
            rows.append(bt[s])
            ks.append(w.hist.k[ho[e]:ho[e + 1]]); vs.append(w.hist.v[ho[e]:ho[e + 1]])
        segs.append(seg)
    sd = storage_dtype(w.dtype)
    hist = Batch(np.asarray(h_q, np.int32), np.asarray(h_l, np.int32),
                 np.stack(rows).astype(np.int32) if rows else np.zeros((0, bt.shape[1]), np.int32),
                 np.concatenate(ks) if ks else np.zeros((0, w.num_kv_heads, w.head_dim), sd),
                 np.concatenate(vs) if vs else np.zeros((0, w.num_kv_heads, w.head_dim), sd))
    step = Batch(w.step.query_lens, w.step.seq_lens, bt, w.step.k, w.step.v)
    return Workload(w.name + "_unshared", w.dtype, w.num_q_heads, w.num_kv_heads, w.head_dim,
                    w.block_size, w.num_blocks, step, w.q, hist, segs, w.seed, w.poison, w.notes)


def plant_needles(w: Workload, seed: int = 0, logit: float = 40.0) -> Workload:
    """A copy of `w` in which every (sequence, KV head) hides one dominant key.

    For sequence s and KV head g a position j is drawn at random among the
    positions every new row of s can see (0 .. seq_len - query_len), every
    query row of s at the G query heads of g is set to one fresh N(0, 1)
    vector u, and the K row of position j, head g, to c * u with
    c = logit / (scale * |u|^2): that key's score is about `logit` while the
    others score about N(0, 1), so each output row is, to many digits, the V
    row of the needle's position.  A read from a wrong block (or a block of
    another sequence) moves such an output by O(1) instead of by the
    O(1/sqrt(L)) of plain N(0, 1) data.  Positions are drawn so that no two
    needles land on the same stored row and head (shared prefix blocks are
    one stored row for the whole group).  V is unchanged."""
    rng = np.random.default_rng(seed)
    G = w.num_q_heads // w.num_kv_heads
    q = w.q.copy()
    hk = w.hist.k.copy()
    sk = w.step.k.copy()
    ho = w.hist_row_offsets()
    no = w.new_row_offsets()
    used = set()

    def stored_row(s: int, j: int):
        # the generator's own bookkeeping: which array and row holds position
        # j of sequence s (history entries cover seq_len - query_len .. seq_len - 1
        # of their own table, the step's rows come last)
        for e in w.hist_segments[s]:
            lo = int(w.hist.seq_lens[e] - w.hist.query_lens[e])
            if lo <= j < int(w.hist.seq_lens[e]):
                return "h", int(ho[e]) + j - lo
        L, ql = int(w.step.seq_lens[s]), int(w.step.query_lens[s])
        return "s", int(no[s]) + j - (L - ql)

    for s in range(w.num_seqs):
        L, ql = int(w.step.seq_lens[s]), int(w.step.query_lens[s])
        if ql == 0 or L == 0:
            continue
        for g in range(w.num_kv_heads):
            for _ in range(64):
                j = int(rng.integers(0, L - ql + 1))
                where = stored_row(s, j)
                if (where, g) not in used:
                    break
            used.add((where, g))
            u = rng.standard_normal(w.head_dim).astype(np.float32)
            c = logit / (w.scale * float(np.dot(u.astype(np.float64), u.astype(np.float64))))
            q[no[s]:no[s + 1], g * G:(g + 1) * G] = _store(u[None, None, :], w.dtype)
            arr = hk if where[0] == "h" else sk
            arr[where[1], g] = _store((c * u)[None, :], w.dtype)[0]
    hist = Batch(w.hist.query_lens, w.hist.seq_lens, w.hist.block_tables, hk, w.hist.v)
    step = Batch(w.step.query_lens, w.step.seq_lens, w.step.block_tables, sk, w.step.v)
    return Workload(w.name + "_needles", w.dtype, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
                    w.num_blocks, step, q, hist, [list(x) for x in w.hist_segments], w.seed, w.poison,
                    w.notes)


def permute_sequences(w: Workload, perm: Sequence[int]) -> Workload:
    """The same batch with its sequences in another order: new sequence i is
    old sequence perm[i] (its lengths, block-table row, new K/V/Q rows and
    history entries move with it).  Block placement and values are unchanged,
    so every sequence's attention is the same."""
    perm = [int(x) for x in perm]
    no = w.new_row_offsets()
    rows = np.concatenate([np.arange(no[s], no[s + 1], dtype=np.int64) for s in perm]) if perm else \
        np.zeros(0, dtype=np.int64)
    step = Batch(w.step.query_lens[perm], w.step.seq_lens[perm], w.step.block_tables[perm], w.step.k[rows],
                 w.step.v[rows])
    return Workload(w.name + "_permuted", w.dtype, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
                    w.num_blocks, step, w.q[rows], w.hist, [list(w.hist_segments[s]) for s in perm], w.seed,
                    w.poison, w.notes)

"""Pins for the CPU oracle: each check ties it to something other than itself.

  * the pages' worked examples (tests/golden/*.json, each with its citation);
  * a library routine: dense padded, masked attention (torch SDPA, float64);
  * brute force in plain Python loops;
  * closed forms and invariants the method implies.

The last test plants plausible mistakes in the oracle (on the CPU) and checks
that at least one pin catches each of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import paged_attention as PA
from workloads import Batch, Workload, accounting, config, random_batch, relabel_blocks, unshare
from workloads.generators import _pad_tables

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name + ".json")) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# pin checks (plain functions so the planted-mistake test can re-run them)
# ---------------------------------------------------------------------------
def pin_offsets():
    g = _golden("offsets_and_padding")
    a = g["query_start_loc_notes_page"]
    assert PA.prefix_offsets(a["lengths"]).tolist() == a["query_start_loc"]
    b = g["cu_seqlens_principle_page"]
    assert PA.prefix_offsets(b["lengths"]).tolist() == b["cu_seqlens"]
    c = g["static_padding_forward_shape_page"]
    assert int(PA.prefix_offsets(c["lengths"])[-1]) == c["real_tokens"]


def pin_forward_shape():
    g = _golden("forward_shape_example")
    bs = g["block_size"]
    tables = _pad_tables([g["block_tables"]["B"], [0], g["block_tables"]["A"]])
    md = PA.build_metadata(g["query_lens"], g["seq_lens"], sum(g["query_lens"]), tables, bs, 34)
    assert md.query_start_loc.tolist() == g["query_start_loc"]
    assert md.positions.tolist() == g["positions"]
    b7 = g["b7_physical"]
    assert int(md.slot_mapping[0]) == b7["block"] * bs + b7["slot_in_block"]
    assert [divmod(int(s), bs) for s in md.slot_mapping[2:7]] == [tuple(x) for x in g["a0_to_a4_physical"]]
    # B reads positions 0..3 from block 10 and 4..7 from block 21
    rd = g["B_read_path"]
    assert [PA.slot_of(tables[0], p, bs) // bs for p in range(8)] == [rd["positions_0_3"]] * 4 + [rd["positions_4_7"]] * 4
    assert md.stats.tolist() == [2, 1, 2, 5, 5, 8]
    # growth: position 8 of B needs logical block 2; after appending block 33 it lands there
    gr = g["B_growth"]
    grown = np.array(g["block_tables"]["B"] + [gr["appended_physical_block"]])
    assert gr["position"] // bs == gr["logical_block"]
    assert PA.slot_of(grown, gr["position"], bs) == gr["appended_physical_block"] * bs


def _dense_reference(w: Workload) -> np.ndarray:
    """Dense padded masked attention from the generator's logical rows (no
    paging at all), via torch's scaled_dot_product_attention in float64."""
    S, Hq, Hkv, D = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim
    ql, sl = w.step.query_lens.astype(int), w.step.seq_lens.astype(int)
    Lq, Lk = max(1, ql.max()), max(1, sl.max())
    Qp = torch.zeros(S, Hq, Lq, D, dtype=torch.float64)
    Kp = torch.zeros(S, Hq, Lk, D, dtype=torch.float64)
    Vp = torch.zeros(S, Hq, Lk, D, dtype=torch.float64)
    mask = torch.zeros(S, 1, Lq, Lk, dtype=torch.bool)
    offs = np.concatenate([[0], np.cumsum(ql)])
    G = Hq // Hkv
    for s in range(S):
        k, v = w.logical_kv(s)
        k64 = torch.from_numpy(PA.widen(k, w.dtype))   # [L, Hkv, D]
        v64 = torch.from_numpy(PA.widen(v, w.dtype))
        Kp[s, :, :sl[s]] = k64.permute(1, 0, 2).repeat_interleave(G, dim=0)
        Vp[s, :, :sl[s]] = v64.permute(1, 0, 2).repeat_interleave(G, dim=0)
        Qp[s, :, :ql[s]] = torch.from_numpy(PA.widen(w.q[offs[s]:offs[s + 1]], w.dtype)).permute(1, 0, 2)
        for i in range(Lq):
            if i < ql[s]:
                qpos = sl[s] - ql[s] + i
                mask[s, 0, i, :qpos + 1] = True
            else:
                mask[s, 0, i, 0] = True   # padding row: keep it finite, discarded below
    O = torch.nn.functional.scaled_dot_product_attention(Qp, Kp, Vp, attn_mask=mask, scale=w.scale)
    out = np.zeros((int(ql.sum()), Hq, D))
    for s in range(S):
        out[offs[s]:offs[s + 1]] = O[s, :, :ql[s]].permute(1, 0, 2).numpy()
    return out


DENSE_CASES = [
    dict(seed=11, S=3, Hq=2, Hkv=2, D=16, bs=4),
    dict(seed=12, S=4, Hq=4, Hkv=2, D=4, bs=1),
    dict(seed=13, S=4, Hq=8, Hkv=2, D=16, bs=2),
    dict(seed=14, S=2, Hq=3, Hkv=1, D=8, bs=4, max_ctx=3),
    dict(seed=15, S=5, Hq=4, Hkv=4, D=16, bs=3, max_q=7, decode_frac=0.2),
]


def pin_dense(case):
    w = random_batch(case["seed"], S=case["S"], Hq=case["Hq"], Hkv=case["Hkv"], D=case["D"],
                     bs=case["bs"], max_ctx=case.get("max_ctx", 12), max_q=case.get("max_q", 5),
                     decode_frac=case.get("decode_frac", 0.4))
    _, _, _, out = PA.run_step(w)
    ref = _dense_reference(w)
    assert np.isfinite(out).all()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def _brute_force(w: Workload) -> np.ndarray:
    """Scalar Python loops with math.exp, straight from the definition."""
    Hq, Hkv, D = w.num_q_heads, w.num_kv_heads, w.head_dim
    ql, sl = w.step.query_lens.tolist(), w.step.seq_lens.tolist()
    out = np.zeros((w.num_tokens, Hq, D))
    t = 0
    for s in range(w.num_seqs):
        k, v = w.logical_kv(s)
        k, v = PA.widen(k, w.dtype).tolist(), PA.widen(v, w.dtype).tolist()
        for i in range(ql[s]):
            qpos = sl[s] - ql[s] + i
            qrow = PA.widen(w.q[t], w.dtype).tolist()
            for h in range(Hq):
                g = h * Hkv // Hq
                xs = [w.scale * sum(qrow[h][d] * k[j][g][d] for d in range(D)) for j in range(qpos + 1)]
                m = max(xs)
                es = [math.exp(x - m) for x in xs]
                z = sum(es)
                for d in range(D):
                    out[t, h, d] = sum(es[j] * v[j][g][d] for j in range(qpos + 1)) / z
            t += 1
    return out


def pin_brute_force():
    w = random_batch(21, S=3, Hq=4, Hkv=2, D=4, bs=2, max_ctx=6, max_q=4)
    _, _, _, out = PA.run_step(w)
    np.testing.assert_allclose(out, _brute_force(w), rtol=0, atol=1e-12)


def pin_single_key():
    """The first row of a fresh prefill sees only itself: o = v exactly
    (forward-shape page §2.3, a0 sees A position 0 only)."""
    w = config(1)
    _, _, _, out = PA.run_step(w)
    # sequence A is third; its first new row is flat row 2
    a0 = 2
    G = w.num_q_heads // w.num_kv_heads
    for h in range(w.num_q_heads):
        np.testing.assert_array_equal(out[a0, h], PA.widen(w.step.v[a0], w.dtype)[h // G])


def pin_closed_form_equal_keys():
    """If every visible key is the same vector, all scores tie and the output
    is the plain mean of the visible value rows."""
    w = random_batch(31, S=3, Hq=4, Hkv=2, D=8, bs=4, max_ctx=9, max_q=4)
    w.hist.k[:] = w.hist.k[:1]
    w.step.k[:] = w.hist.k[:1] if w.hist.k.shape[0] else w.step.k[:1]
    _, _, _, out = PA.run_step(w)
    G = w.num_q_heads // w.num_kv_heads
    offs = w.new_row_offsets()
    for s in range(w.num_seqs):
        _, v = w.logical_kv(s)
        v64 = PA.widen(v, w.dtype)
        L, q = int(w.step.seq_lens[s]), int(w.step.query_lens[s])
        for i in range(q):
            p = L - q + i
            for h in range(w.num_q_heads):
                np.testing.assert_allclose(out[offs[s] + i, h], v64[:p + 1, h // G].mean(axis=0),
                                           rtol=0, atol=1e-13)


def _sdpa_rows(q, k, v, scale):
    """Attention of query rows q [n, Hq, D] over all of k/v [L, Hkv, D] (no
    mask) via torch SDPA in float64, GQA by repeating KV heads."""
    G = q.shape[1] // k.shape[1]
    Q = torch.from_numpy(q).permute(1, 0, 2)[None]
    K = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    V = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    return torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)[0].permute(1, 0, 2).numpy()


def pin_copy_on_write():
    """The parallel-sampling walk-through of the vLLM principles page (§2.1):
    A1 and A2 share physical blocks 7 and 1 holding a 7-token prompt; A1's
    first write into shared block 1 copies it to block 3 and repoints A1's
    table; A2 then writes into block 1 in place.  Each branch must then see
    the prompt plus its own new token and nothing of the other's."""
    g = _golden("copy_on_write")["parallel_sampling_cow"]
    bs, n = g["block_size_implied"], g["prompt_tokens"]
    assert -(-n // bs) == g["logical_blocks"] and n - (g["logical_blocks"] - 1) * bs == g["tokens_in_last_block"]
    rng = np.random.default_rng(61)
    Hq, Hkv, D, NB = 4, 2, 8, 8
    kc = PA.empty_pool((NB, bs, Hkv, D), "f32", np.nan)
    vc = PA.empty_pool((NB, bs, Hkv, D), "f32", np.nan)
    pk = rng.standard_normal((n, Hkv, D)).astype(np.float32)
    pv = rng.standard_normal((n, Hkv, D)).astype(np.float32)
    shared = np.array([g["shared_physical_blocks"]], np.int32)
    md = PA.build_metadata([n], [n], n, shared, bs, NB)
    PA.write_kv(pk, pv, md.slot_mapping, kc, vc)
    # A1 writes first: copy-on-write of the shared last block
    PA.copy_blocks(kc, vc, kc, vc, [[g["cow_source_block"], g["cow_new_block"]]])
    tables = np.array([g["a1_table_after"], g["a2_table_after"]], np.int32)
    nk = rng.standard_normal((2, Hkv, D)).astype(np.float32)   # "fathers" (A1), "mothers" (A2)
    nv = rng.standard_normal((2, Hkv, D)).astype(np.float32)
    q = rng.standard_normal((2, Hq, D)).astype(np.float32)
    md = PA.build_metadata([1, 1], [n + 1, n + 1], 2, tables, bs, NB)
    assert md.positions.tolist() == [g["new_token_position"]] * 2
    PA.write_kv(nk, nv, md.slot_mapping, kc, vc)
    out = PA.attention(q, kc, vc, tables, md.query_start_loc, np.array([n + 1, n + 1]), Hkv, 0.5, "f32")
    for b, (kk, vv) in enumerate(zip(nk, nv)):
        k_log = np.concatenate([pk, kk[None]]).astype(np.float64)
        v_log = np.concatenate([pv, vv[None]]).astype(np.float64)
        np.testing.assert_allclose(out[b], _sdpa_rows(q[b:b + 1].astype(np.float64), k_log, v_log, 0.5)[0],
                                   rtol=0, atol=1e-12)
    # the source block still holds the prompt tail plus A2's row only
    np.testing.assert_array_equal(kc[g["cow_source_block"], :n - bs], pk[bs:])
    np.testing.assert_array_equal(kc[g["cow_source_block"], n - bs], nk[1])
    np.testing.assert_array_equal(vc[g["cow_new_block"], n - bs], nv[0])


def _decode_16bit(bits: np.ndarray, exp_bits: int, man_bits: int) -> np.ndarray:
    """Value of each 16-bit pattern from the format's definition: sign bit,
    `exp_bits` biased exponent bits, `man_bits` stored mantissa bits;
    exponent field 0 is subnormal (no implicit 1, minimum exponent), the
    all-ones field is infinity (mantissa 0) or NaN.  Written with integer
    arithmetic and np.ldexp, so every value is exact in float64."""
    b = bits.astype(np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    e = (b >> man_bits) & ((1 << exp_bits) - 1)
    m = b & ((1 << man_bits) - 1)
    bias = (1 << (exp_bits - 1)) - 1
    normal = np.ldexp((m + (1 << man_bits)).astype(np.float64), (e - bias - man_bits).astype(np.int32))
    sub = np.ldexp(m.astype(np.float64), np.full(b.shape, 1 - bias - man_bits, dtype=np.int32))
    inf_nan = np.where(m == 0, np.inf, np.nan)
    top = (1 << exp_bits) - 1
    return sign * np.where(e == 0, sub, np.where(e == top, inf_nan, normal))


def pin_widen():
    """The exact widening of stored 16-bit values (the pages keep K/V in 16
    bits, "LLM 推理引擎 Continuous Batching 与 PagedAttention" §1.2): known bit
    patterns from the bfloat16 (8 exponent, 7 mantissa bits) and IEEE binary16
    (5, 10) definitions, then every one of the 65,536 patterns against the
    definition decoded from the bit fields and against torch's own
    conversion, compared as float64 bit patterns (so -0.0 and 0.0 differ)."""
    known_bf16 = {0x3F80: 1.0, 0xC040: -3.0, 0x7F7F: float.fromhex("0x1.fep127"), 0x0001: 2.0 ** -133,
                  0x8000: -0.0, 0x0080: 2.0 ** -126, 0x3E80: 0.25, 0x4049: 3.140625, 0x7F80: np.inf,
                  0xFF80: -np.inf}
    known_f16 = {0x3C00: 1.0, 0xC200: -3.0, 0x7BFF: 65504.0, 0x0001: 2.0 ** -24, 0x8000: -0.0,
                 0x0400: 2.0 ** -14, 0x3555: float.fromhex("0x1.554p-2"), 0x7C00: np.inf, 0xFC00: -np.inf}
    for dtype, known in (("bf16", known_bf16), ("f16", known_f16)):
        bits = np.array(sorted(known), dtype=np.uint16)
        got = PA.widen(bits, dtype)
        want = np.array([known[int(b)] for b in bits], dtype=np.float64)
        assert np.array_equal(got.view(np.uint64), want.view(np.uint64)), dtype
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    as_i16 = torch.from_numpy(allbits.view(np.int16).copy())
    for dtype, eb, mb, tdt in (("bf16", 8, 7, torch.bfloat16), ("f16", 5, 10, torch.float16)):
        with np.errstate(invalid="ignore"):   # signalling-NaN patterns warn when widened
            got = PA.widen(allbits, dtype)
        want = _decode_16bit(allbits, eb, mb)
        lib = as_i16.view(tdt).to(torch.float64).numpy()
        ok = ~np.isnan(want)
        assert np.array_equal(np.isnan(got), ~ok), dtype
        assert np.array_equal(got[ok].view(np.uint64), want[ok].view(np.uint64)), dtype
        assert np.array_equal(got[ok].view(np.uint64), lib[ok].view(np.uint64)), dtype


ALL_PINS = [pin_widen, pin_offsets, pin_forward_shape, pin_brute_force, pin_single_key,
            pin_closed_form_equal_keys, pin_copy_on_write] + [(lambda c=c: pin_dense(c)) for c in DENSE_CASES]


# ---------------------------------------------------------------------------
# tests
# ---------------------------------------------------------------------------
def test_widen_16bit_exact():
    pin_widen()


def test_offsets_pages():
    pin_offsets()


def test_forward_shape_example():
    pin_forward_shape()


@pytest.mark.parametrize("case", DENSE_CASES, ids=lambda c: f"seed{c['seed']}")
def test_oracle_equals_dense_padded_masked(case):
    pin_dense(case)


def test_oracle_equals_brute_force():
    pin_brute_force()


def test_copy_on_write_walkthrough():
    pin_copy_on_write()


def test_copy_blocks_semantics():
    """Whole blocks move bit for bit between pools (swap out to a host pool
    and back in at other ids), both K and V, and nothing else changes."""
    rng = np.random.default_rng(62)
    kc = rng.integers(0, 2**16, (6, 4, 2, 8), dtype=np.uint16)
    vc = rng.integers(0, 2**16, (6, 4, 2, 8), dtype=np.uint16)
    k0, v0 = kc.copy(), vc.copy()
    hk = np.zeros((3, 4, 2, 8), np.uint16)
    hv = np.zeros((3, 4, 2, 8), np.uint16)
    PA.copy_blocks(kc, vc, hk, hv, [[4, 0], [1, 2]])          # swap out
    assert (hk[0] == k0[4]).all() and (hv[2] == v0[1]).all() and (hk[1] == 0).all()
    PA.copy_blocks(hk, hv, kc, vc, [[0, 5], [2, 0]])          # swap in elsewhere
    assert (kc[5] == k0[4]).all() and (vc[5] == v0[4]).all() and (kc[0] == k0[1]).all() and (vc[0] == v0[1]).all()
    assert (kc[1:5] == k0[1:5]).all() and (vc[1:5] == v0[1:5]).all()
    for bad in ([[0, 1], [2, 1]], [[0, 1], [1, 2]], [[6, 0]], [[0, -1]]):
        with pytest.raises(oracle.OracleInputError):
            PA.copy_blocks(kc, vc, kc, vc, bad)


def test_single_key_identity():
    pin_single_key()


def test_closed_form_equal_keys():
    pin_closed_form_equal_keys()


def test_padding_accounting(golden):
    g = golden["offsets_and_padding"]
    c = g["static_padding_forward_shape_page"]
    lens = c["lengths"]
    assert len(lens) * max(lens) == c["padded_slots"]
    assert c["padded_slots"] - int(PA.prefix_offsets(lens)[-1]) == c["padding_waste"]
    a = g["query_start_loc_notes_page"]
    assert len(a["lengths"]) * max(a["lengths"]) == a["padded_slots"]
    assert int(PA.prefix_offsets(a["lengths"])[-1]) == a["real_tokens"]
    # the ragged-prefill workload flattens exactly those lengths
    w = config(2, scale_down=1)
    assert w.num_tokens == c["real_tokens"]


def test_byte_formulas(golden):
    g = golden["block_tables_and_bytes"]
    a = g["kv_bytes_per_token_llama2_7b"]
    assert accounting.kv_bytes_per_token(a["layers"], a["kv_heads"], a["head_dim"], a["itemsize"]) == a["bytes_per_token"]
    assert a["tokens"] * a["bytes_per_token"] == 2 * 2**30
    b = g["gpt3_kv_cache"]
    got = accounting.kv_cache_bytes_gpt(b["batch"], b["seq"], b["d_model"], b["layers"], b["itemsize"])
    assert got == b["bytes"] and round(got / 1e6) == 472
    c = g["block_bytes"]
    assert accounting.block_bytes(c["layers"], c["block_size"], c["kv_heads"], c["head_dim"], c["itemsize"]) == c["bytes"]
    # one layer's share per token for the decode workload's shape (32 heads x 128, bf16)
    assert accounting.kv_bytes_per_token(1, 32, 128, 2) == 16384


def test_padded_block_tables(golden):
    g = golden["block_tables_and_bytes"]["padded_block_tables"]
    bt = np.array(g["flat"], dtype=np.int32).reshape(g["rows"], -1)
    bs = 4
    used = g["used_blocks"]
    seq_lens = [len(u) * bs for u in used]
    md = PA.build_metadata([1] * 3, seq_lens, 3, bt, bs, 8)
    for s, u in enumerate(used):
        assert (bt[s, :len(u)] == u).all() and (bt[s, len(u):] == -1).all()
        # every position of the sequence maps into its own used blocks
        assert sorted({PA.slot_of(bt[s], p, bs) // bs for p in range(seq_lens[s])}) == u
    assert md.slot_mapping.tolist() == [PA.slot_of(bt[s], seq_lens[s] - 1, bs) for s in range(3)]
    # a -1 inside the used range is invalid
    with pytest.raises(oracle.OracleInputError):
        PA.build_metadata([1] * 3, [13, 16, 4], 3, bt, bs, 8)


def test_new_block_needed_iff_len_mod_bs_is_1():
    """Appending the L-th token needs a fresh block exactly when L % bs == 1
    (vLLM 原理 §3.4 can_append / may_append)."""
    for bs in (1, 2, 4, 16):
        for L in range(1, 70):
            held = -(-(L - 1) // bs)                       # blocks holding positions 0..L-2
            needed = PA.position_of(L, 1, 0) // bs + 1     # logical blocks once position L-1 exists
            assert (needed > held) == (L % bs == 1 if bs > 1 else True)


def test_stats_and_counters():
    md = PA.build_metadata([1, 0, 4, 1, 3], [5, 2, 4, 9, 7], 9)
    assert md.stats.tolist() == [2, 2, 2, 7, 4, 9]
    assert md.query_start_loc.tolist() == [0, 1, 1, 5, 6, 9]
    assert md.seq_start_loc.tolist() == [0, 5, 7, 11, 20, 27]
    assert md.token_to_seq.tolist() == [0, 2, 2, 2, 2, 3, 4, 4, 4]
    assert md.positions.tolist() == [4, 0, 1, 2, 3, 8, 4, 5, 6]


@pytest.mark.parametrize("bad", ["qlen_gt_seqlen", "sum", "negative", "block_oob", "block_neg"])
def test_invalid_batches_raise(bad):
    bt = np.array([[0, 1], [2, -1]], np.int32)
    args = dict(query_lens=[2, 1], seq_lens=[5, 3], num_tokens=3, block_tables=bt, block_size=4, num_blocks=3)
    if bad == "qlen_gt_seqlen":
        args["query_lens"], args["num_tokens"] = [6, 1], 7
    elif bad == "sum":
        args["num_tokens"] = 4
    elif bad == "negative":
        args["query_lens"], args["num_tokens"] = [-1, 1], 0
    elif bad == "block_oob":
        args["block_tables"] = np.array([[0, 3], [2, -1]], np.int32)
    elif bad == "block_neg":
        args["block_tables"] = np.array([[0, -1], [2, -1]], np.int32)
    with pytest.raises(oracle.OracleInputError):
        PA.build_metadata(**args)


def test_write_kv_semantics():
    kc = np.full((3, 2, 1, 2), np.nan, np.float32)
    vc = np.full((3, 2, 1, 2), np.nan, np.float32)
    k = np.arange(8, dtype=np.float32).reshape(4, 1, 2)
    v = -k
    PA.write_kv(k, v, np.array([5, -1, 0, 2]), kc, vc)
    assert (kc[2, 1] == k[0]).all() and (vc[2, 1] == v[0]).all()
    assert (kc[0, 0] == k[2]).all() and (kc[1, 0] == k[3]).all()
    untouched = [(0, 1), (1, 1), (2, 0)]
    for b, o in untouched:
        assert np.isnan(kc[b, o]).all() and np.isnan(vc[b, o]).all()
    with pytest.raises(oracle.OracleInputError):
        PA.write_kv(k, v, np.array([1, 1, -1, -1]), kc, vc)
    with pytest.raises(oracle.OracleInputError):
        PA.write_kv(k, v, np.array([6, -1, -1, -1]), kc, vc)


def test_gqa_requires_divisible_heads():
    w = random_batch(5, S=2, Hq=4, Hkv=2, D=4, bs=2)
    _, kc, vc, _ = PA.run_step(w)
    with pytest.raises(oracle.OracleInputError):
        PA.attention(w.q[:, :3], kc, vc, w.step.block_tables, PA.prefix_offsets(w.step.query_lens),
                     w.step.seq_lens, 2, w.scale, w.dtype)


def _explicit(dtype, Hq, Hkv, D, bs, NB, step_q, step_l, tables, q, k_new, v_new,
              h_q, h_l, h_tables, hk, hv, segs):
    st = Batch(np.array(step_q, np.int32), np.array(step_l, np.int32), _pad_tables(tables), k_new, v_new)
    hi = Batch(np.array(h_q, np.int32), np.array(h_l, np.int32),
               _pad_tables(h_tables, st.block_tables.shape[1]) if h_tables else np.zeros((0, st.block_tables.shape[1]), np.int32),
               hk, hv)
    return Workload("explicit", dtype, Hq, Hkv, D, bs, NB, st, q, hi, segs)


def test_decode_equals_last_row_of_prefill():
    """Decoding position L-1 against L-1 cached rows gives the last row of a
    one-shot L-token prefill (vLLM 原理 §1.1: decode needs only the last row)."""
    rng = np.random.default_rng(41)
    L, Hq, Hkv, D, bs = 11, 4, 2, 8, 4
    K = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    V = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    Q = rng.standard_normal((L, Hq, D)).astype(np.float32)
    tab = [[3, 0, 5]]
    one = _explicit("f32", Hq, Hkv, D, bs, 6, [L], [L], tab, Q, K, V, [], [], [], K[:0], V[:0], [[]])
    dec = _explicit("f32", Hq, Hkv, D, bs, 6, [1], [L], tab, Q[L - 1:], K[L - 1:], V[L - 1:],
                    [L - 1], [L - 1], tab, K[:L - 1], V[:L - 1], [[0]])
    _, _, _, o1 = PA.run_step(one)
    _, _, _, o2 = PA.run_step(dec)
    np.testing.assert_array_equal(o1[L - 1], o2[0])


def test_verify_equals_sequential_decodes():
    """Verifying q draft tokens in one pass (query_len q over a cached
    context; "LLM 推理引擎 Continuous Batching 与 PagedAttention" §7.2) gives,
    row for row, what q successive single-token decode steps give, each with
    the earlier drafts already in the cache."""
    rng = np.random.default_rng(43)
    ctx, q, Hq, Hkv, D, bs = 9, 4, 8, 2, 8, 4
    L = ctx + q
    K = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    V = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    Q = rng.standard_normal((q, Hq, D)).astype(np.float32)
    tab = [[6, 2, 0, 4]]
    ver = _explicit("f32", Hq, Hkv, D, bs, 7, [q], [L], tab, Q, K[ctx:], V[ctx:],
                    [ctx], [ctx], tab, K[:ctx], V[:ctx], [[0]])
    _, _, _, o_ver = PA.run_step(ver)
    for i in range(q):
        n = ctx + i
        dec = _explicit("f32", Hq, Hkv, D, bs, 7, [1], [n + 1], tab, Q[i:i + 1], K[n:n + 1], V[n:n + 1],
                        [n], [n], tab, K[:n], V[:n], [[0]])
        _, _, _, o_dec = PA.run_step(dec)
        np.testing.assert_array_equal(o_ver[i], o_dec[0])


def test_chunked_prefill_equals_one_shot():
    """Prefill in two chunks ([0:c], then [c:L] with c cached) equals one shot
    (vLLM 原理 §2.4 chunked prefill)."""
    rng = np.random.default_rng(42)
    L, c, Hq, Hkv, D, bs = 13, 5, 4, 1, 8, 4
    K = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    V = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    Q = rng.standard_normal((L, Hq, D)).astype(np.float32)
    tab = [[6, 2, 0, 4]]
    one = _explicit("f32", Hq, Hkv, D, bs, 7, [L], [L], tab, Q, K, V, [], [], [], K[:0], V[:0], [[]])
    first = _explicit("f32", Hq, Hkv, D, bs, 7, [c], [c], tab, Q[:c], K[:c], V[:c], [], [], [], K[:0], V[:0], [[]])
    second = _explicit("f32", Hq, Hkv, D, bs, 7, [L - c], [L], tab, Q[c:], K[c:], V[c:],
                       [c], [c], tab, K[:c], V[:c], [[0]])
    _, _, _, o = PA.run_step(one)
    _, _, _, a = PA.run_step(first)
    _, _, _, b = PA.run_step(second)
    np.testing.assert_array_equal(o, np.concatenate([a, b]))


def test_isolation_outside_blocks():
    """Changing blocks outside sequence s's table leaves s's rows bit-identical;
    changing one of its used blocks does not (forward-shape page §2.3补充:
    each request reads only its own table)."""
    w = random_batch(51, S=3, Hq=2, Hkv=2, D=8, bs=2, max_ctx=8, max_q=3, extra_blocks=3)
    md, kc, vc, out = PA.run_step(w)
    s = 1
    bt = w.step.block_tables
    used = set(int(b) for b in bt[s, :-(-int(w.step.seq_lens[s]) // w.block_size)])
    kc2, vc2 = kc.copy(), vc.copy()
    for b in range(w.num_blocks):
        if b not in used:
            kc2[b] = 7.0
            vc2[b] = -7.0
    out2 = PA.attention(w.q, kc2, vc2, bt, md.query_start_loc, w.step.seq_lens, w.num_kv_heads, w.scale, w.dtype)
    t0, t1 = md.query_start_loc[s], md.query_start_loc[s + 1]
    np.testing.assert_array_equal(out[t0:t1], out2[t0:t1])
    vc3 = vc.copy()
    vc3[int(bt[s, 0]), 0] += 1.0
    out3 = PA.attention(w.q, kc, vc3, bt, md.query_start_loc, w.step.seq_lens, w.num_kv_heads, w.scale, w.dtype)
    assert not np.array_equal(out[t0:t1], out3[t0:t1])


def test_placement_invariance():
    """Renaming physical blocks (moving their contents with them) changes no
    output bit (forward-shape page §2.3补充: physical blocks may sit anywhere)."""
    w = random_batch(61, S=4, Hq=4, Hkv=2, D=8, bs=3, max_ctx=10, max_q=4, extra_blocks=5)
    perm = np.random.default_rng(0).permutation(w.num_blocks)
    _, _, _, a = PA.run_step(w)
    _, _, _, b = PA.run_step(relabel_blocks(w, perm))
    np.testing.assert_array_equal(a, b)


def test_sharing_invariance():
    """Sequences sharing prefix blocks give the same output as with private
    copies of those blocks (vLLM 原理 §2.1 ref-count sharing)."""
    w = config(5, scale_down=64)
    w.num_blocks += int((w.step.block_tables >= 0).sum())   # room for private copies
    used = set(int(b) for b in w.step.block_tables.ravel() if b >= 0)
    spare = [b for b in range(w.num_blocks) if b not in used]
    u = unshare(w, spare)
    assert len(set(int(b) for b in u.step.block_tables.ravel() if b >= 0)) > len(used)
    rows = list(range(w.num_tokens))
    _, _, _, a = PA.run_step(w, rows)
    _, _, _, b = PA.run_step(u, rows)
    np.testing.assert_array_equal(a, b)


def test_configs_shapes():
    """Structure of the five workloads at full size (lengths only; values are
    not generated for the big ones here)."""
    w1 = config(1)
    assert w1.step.query_lens.tolist() == [1, 1, 5] and w1.step.seq_lens.tolist() == [8, 3, 5]
    assert w1.num_blocks == 16 and w1.dtype == "f32"


def test_scale_down_configs_run():
    for n in (2, 3, 4, 5):
        w = config(n, scale_down=64)
        md, _, _, out = PA.run_step(w, rows=[0, w.num_tokens - 1])
        assert np.isfinite(out).all()


# ---------------------------------------------------------------------------
# planted mistakes: each must trip at least one pin
# ---------------------------------------------------------------------------
def _bad_position(L, q, i):
    return L - q + i - 1 if i > 0 else L - q + i


def _bad_kv_head(h, Hq, Hkv):
    return h % Hkv


def _bad_slot(row, pos, bs):
    return int(row[pos % len(row)]) * bs + pos // bs


def _bad_offsets(lengths):
    out = np.zeros(len(lengths) + 1, dtype=np.int64)
    for s, n in enumerate(lengths):
        out[s + 1] = out[s] + int(n) - (1 if s == 0 and n > 0 else 0)
    return out


def _bad_softmax(scores, values):
    w = np.exp(scores)
    return (w @ values) / (w.sum(axis=-1, keepdims=True) + 1e-3)


def _bad_copy_blocks(src_k, src_v, dst_k, dst_v, pairs):
    for a, b in np.asarray(pairs).reshape(-1, 2):
        dst_k[int(b)] = src_k[int(a)]     # V left behind


def _bad_widen_bf16(a, dtype):
    out = _GOOD_WIDEN(a, dtype)
    return out * 1.01 if dtype == "bf16" else out


def _bad_widen_f16(a, dtype):
    if dtype != "f16":
        return _GOOD_WIDEN(a, dtype)
    # read as bfloat16 bits: a plausible mix-up of the two 16-bit formats
    return _GOOD_WIDEN(a, "bf16")


_GOOD_WIDEN = PA.widen

MUTANTS = {
    "widen_bf16_one_percent_off": ("widen", _bad_widen_bf16),
    "widen_f16_read_as_bf16": ("widen", _bad_widen_f16),
    "copy_blocks_drops_v": ("copy_blocks", _bad_copy_blocks),
    "position_off_by_one": ("position_of", _bad_position),
    "gqa_head_mapping_transposed": ("kv_head_of", _bad_kv_head),
    "slot_block_offset_swapped": ("slot_of", _bad_slot),
    "prefix_sum_dropped_term": ("prefix_offsets", _bad_offsets),
    "softmax_normaliser_wrong": ("softmax_weighted_sum", _bad_softmax),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name, monkeypatch):
    attr, bad = MUTANTS[name]
    monkeypatch.setattr(PA, attr, bad)
    caught = 0
    for pin in ALL_PINS:
        try:
            pin()
        except (AssertionError, oracle.OracleInputError, IndexError, ValueError):
            caught += 1
    assert caught >= 1, f"no pin caught planted mistake {name}"

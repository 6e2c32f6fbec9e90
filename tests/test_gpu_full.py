"""GPU parity at the workloads' full sizes, in the launch configuration
bench.py times, plus edge cases.

Full sizes: metadata compared in full (bit-exact), the pool compared in full
(bit-exact, NaN poison included) for the decode and shared-prefix batches,
attention compared to the dtype's tolerance on every row of the ragged
prefill, decode and shared-prefix batches and on the longest chunks and
decodes of the chunked mixed batch, with the fast kernels forced and checked
to have run; the same batches again with one dominant key planted per
(sequence, KV head), which a wrong-block read cannot hide under the
tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import ragged_paged_attention_amd as rpa
from tests.gpu_path import DeviceRun, max_abs_err, tol_for
from workloads import Batch, Workload, config, plant_needles, random_batch
from workloads.device import to_numpy_bits
from workloads.generators import _pad_tables

pytestmark = pytest.mark.gpu


_WORKLOADS = {}


def _full(n):
    """The full-size workload n, generated once per module (the decode batch's
    3.3 GB of history takes a while to draw)."""
    if n not in _WORKLOADS:
        _WORKLOADS[n] = config(n)
    return _WORKLOADS[n]


def _rows_for(w, n):
    """Rows compared against the oracle: every row of the ragged prefill, the
    decode and the shared-prefix batches; for the chunked mixed batch every
    row of its two longest chunks and of its 32 longest decodes, plus the
    first and last rows."""
    if n != 4:
        return None
    ql, sl = w.step.query_lens, w.step.seq_lens
    offs = w.new_row_offsets()
    chunks = [s for s in np.argsort(-sl, kind="stable") if ql[s] > 1][:2]
    decodes = [s for s in np.argsort(-sl, kind="stable") if ql[s] == 1][:32]
    rows = {0, w.num_tokens - 1}
    for s in list(chunks) + list(decodes):
        rows |= set(range(int(offs[s]), int(offs[s + 1])))
    return sorted(rows)


# kernels each full-size batch must run on the MFMA paths (and the generic
# kernel must not run)
_EXPECTED_KERNELS = {2: {"prefill_kernel"}, 3: {"decode_kernel", "merge_kernel"},
                     4: {"decode_kernel", "prefill_kernel", "merge_kernel"},
                     5: {"decode_kernel", "prefill_kernel", "merge_kernel"}}


def _bits(a):
    a = np.asarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


def _run_fast(w):
    """The step through the C ABI with the fast paths forced (a call they do
    not support fails instead of falling back), timing which kernels ran."""
    prev = rpa.pa_set_kernel_policy(rpa.PA_POLICY_FAST)
    try:
        g = DeviceRun(w).fill_history()
        torch.cuda.synchronize()
        rpa.pa_bench_timing_begin()
        g.step()
        torch.cuda.synchronize()
        kernels = set(rpa.pa_bench_timing_end())
    finally:
        rpa.pa_set_kernel_policy(prev)
    return g, kernels


def _compare(w, n, g, rows, label):
    md, kc, vc, ref = oracle.run_step(w, rows=rows)
    got = g.out if rows is None else g.out[torch.tensor(rows, device="cuda")]
    err = max_abs_err(got, ref)
    print(f"[full] config {n} {label}: {len(ref)} rows compared, max_abs_err={err:.3e}, "
          f"max|ref|={float(np.max(np.abs(ref))):.3f}", flush=True)
    assert err <= tol_for(w.dtype)
    assert torch.isfinite(g.out).all()
    return md, kc, vc


@pytest.mark.timeout(900)
@pytest.mark.parametrize("n", [2, 3, 4, 5])
def test_full_size_config(n):
    w = _full(n)
    print(f"[full] config {n} {w.summary()}", flush=True)
    rows = _rows_for(w, n)
    g, kernels = _run_fast(w)
    print(f"[full] config {n}: kernels {sorted(kernels)}", flush=True)
    assert _EXPECTED_KERNELS[n] <= kernels and "attn_generic_kernel" not in kernels
    assert g.err() == 0
    md, kc, vc = _compare(w, n, g, rows, "N(0,1) data")
    for name in ("query_start_loc", "seq_start_loc", "positions", "token_to_seq", "slot_mapping", "stats"):
        assert np.array_equal(g.meta[name].cpu().numpy(), getattr(md, name)), name
    if n in (3, 5):
        assert np.array_equal(_bits(to_numpy_bits(g.k_cache)), _bits(kc)), "k_cache differs"
        assert np.array_equal(_bits(to_numpy_bits(g.v_cache)), _bits(vc)), "v_cache differs"


@pytest.mark.timeout(900)
@pytest.mark.parametrize("n", [3, 4, 5])
def test_full_size_needles(n):
    """Each sequence reads only its own blocks, which sit anywhere in the pool
    ("vLLM Continuous Batching：从 Forward Shape 理解两个核心参数" §2.3补充).
    With one dominant key per (sequence, KV head) every output row is that
    key's V row, so a block read from the wrong place (a wrong id in the
    decode kernel's block-id window, a misrouted shared prefix) moves a row by
    O(1) instead of hiding under the tolerance."""
    w = plant_needles(_full(n), seed=100 + n)
    print(f"[needles] config {n} {w.summary()}", flush=True)
    rows = _rows_for(w, n)
    g, kernels = _run_fast(w)
    assert _EXPECTED_KERNELS[n] <= kernels and "attn_generic_kernel" not in kernels
    assert g.err() == 0
    _compare(w, n, g, rows, "needles")


def test_empty_batch_is_a_no_op():
    w = config(1)
    g = DeviceRun(w).run()
    out = torch.full_like(g.db.q, 7.0)
    qsl = torch.zeros(1, dtype=torch.int32, device="cuda")
    sl = torch.zeros(0, dtype=torch.int32, device="cuda")
    st = rpa.library().pa_attention(g.db.q.data_ptr(), g.k_cache.data_ptr(), g.v_cache.data_ptr(),
                                    g.db.block_tables.data_ptr(), qsl.data_ptr(), sl.data_ptr(), 0, 0,
                                    w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.num_blocks,
                                    w.max_blocks_per_seq, 1, 1, 0.25, 0, out.data_ptr(), None, 0, None, None)
    torch.cuda.synchronize()
    assert st == 0 and bool((out == 7.0).all())


def _explicit(dtype, Hq, Hkv, D, bs, NB, q_lens, s_lens, tables, seed, hist_tables=None):
    """A workload with given lengths: history for every sequence, random values."""
    from workloads.generators import build_workload
    return build_workload("explicit", dtype, Hq, Hkv, D, bs, NB, q_lens, s_lens, tables, seed)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_length_queries_mixed_in(dtype):
    """Sequences with query_len 0 own no rows and must not disturb others."""
    rng = np.random.default_rng(3)
    ql = [0, 3, 0, 1, 0, 40, 1, 0]
    sl = [5, 9, 0, 30, 17, 77, 1, 16]
    bs = 16
    counts = [-(-L // bs) for L in sl]
    ids = rng.permutation(64)
    tables, o = [], 0
    for c in counts:
        tables.append([int(x) for x in ids[o:o + c]])
        o += c
    w = _explicit(dtype, 8, 2, 128, bs, 64, ql, sl, tables, 5)
    g = DeviceRun(w).run()
    _, _, _, ref = oracle.run_step(w)
    assert g.err() == 0
    assert max_abs_err(g.out, ref) <= tol_for(dtype)


def test_small_hints_flagged_and_still_correct_when_covered():
    """A max_query_len below the true maximum flags PA_DERR_HINT.  Here it
    still sends the long prompts to the prefill kernel (40 rows > the 32 of
    two decode tiles), which covers any length, so the rows are right; a
    too-small max_seq_len only makes split parts longer."""
    w = config(2, scale_down=4)
    g = DeviceRun(w).fill_history().write_step_rows()
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = rpa.pa_attention(g.db.q, g.k_cache, g.v_cache, g.db.block_tables, g.meta["query_start_loc"],
                           g.db.seq_lens, 40, 3, w.scale, d_err=d_err)
    torch.cuda.synchronize()
    _, _, _, ref = oracle.run_step(w)
    assert int(d_err.item()) == rpa.PA_DERR_HINT
    assert max_abs_err(out, ref) <= tol_for(w.dtype)


@pytest.mark.parametrize("needles", [False, True])
def test_very_long_decode_context_beyond_part_cap(needles):
    """A 70,001-token context needs more than 64 parts of 768 tokens: parts
    get longer instead (69 blocks each, so the decode kernel's 64-entry
    block-id window is refetched inside a part), and the result stays exact;
    with a planted dominant key, a wrong id after the refetch would show."""
    L = 70001
    bs = 16
    nb = -(-L // bs)
    rng = np.random.default_rng(9)
    tables = [[int(x) for x in rng.permutation(nb + 8)[:nb]]]
    w = _explicit("bf16", 4, 1, 128, bs, nb + 8, [1], [L], tables, 11)
    if needles:
        w = plant_needles(w, seed=12)
    g = DeviceRun(w).run()
    _, _, _, ref = oracle.run_step(w)
    assert g.err() == 0
    err = max_abs_err(g.out, ref)
    print(f"[long] L={L} needles={needles} max_abs_err={err:.3e} max|ref|={float(np.abs(ref).max()):.3f}", flush=True)
    assert err <= tol_for("bf16")


@pytest.mark.parametrize("shape", [dict(Hq=64, Hkv=1, D=128, bs=16),   # G = 64 > 16: generic path
                                   dict(Hq=4, Hkv=2, D=256, bs=8),     # head_dim 256
                                   dict(Hq=8, Hkv=8, D=128, bs=64)],   # large blocks on the fast path
                         ids=["G64", "D256", "bs64"])
def test_other_shapes(shape):
    w = random_batch(77, S=5, Hq=shape["Hq"], Hkv=shape["Hkv"], D=shape["D"], bs=shape["bs"], dtype="bf16",
                     max_ctx=300, max_q=70)
    g = DeviceRun(w).run()
    _, _, _, ref = oracle.run_step(w)
    assert g.err() == 0
    assert max_abs_err(g.out, ref) <= tol_for("bf16")


def test_invalid_block_ids_on_the_mfma_paths():
    """Block-table entries out of range (-1 and >= num_blocks) in a bf16 batch
    that runs the decode and prefill kernels: PA_DERR_BLOCK_OOB is raised,
    every access stays inside the pool (the kernels clamp a bad id to block
    0 after flagging it), and the sequences whose tables are valid still
    match the oracle.  The rows of the two damaged sequences are
    unspecified and not compared."""
    w = config(4, scale_down=8)
    g = DeviceRun(w).fill_history().write_step_rows()
    ql, sl = w.step.query_lens, w.step.seq_lens
    G = w.num_q_heads // w.num_kv_heads
    dec = [s for s in range(w.num_seqs) if ql[s] == 1]
    pre = [s for s in range(w.num_seqs) if ql[s] * G > 32]
    sd = max(dec, key=lambda s: sl[s])                  # a decode row with a long context
    sp = max(pre, key=lambda s: sl[s])                  # a chunk on the prefill kernel
    assert sl[sd] > 2 * w.block_size and pre
    bt = g.db.block_tables.clone()
    bt[sd, (int(sl[sd]) - 1) // w.block_size // 2] = -1
    bt[sp, 0] = w.num_blocks + 7
    print(f"[invalid ids] decode seq {sd} (len {sl[sd]}), prefill seq {sp} (len {sl[sp]})", flush=True)
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = rpa.pa_attention(g.db.q, g.k_cache, g.v_cache, bt, g.meta["query_start_loc"], g.db.seq_lens,
                           max(1, w.max_query_len), max(1, w.max_seq_len), w.scale, d_err=d_err)
    torch.cuda.synchronize()
    assert int(d_err.item()) & rpa.PA_DERR_BLOCK_OOB
    _, _, _, ref = oracle.run_step(w)
    offs = w.new_row_offsets()
    keep = np.ones(w.num_tokens, dtype=bool)
    for s in (sd, sp):
        keep[int(offs[s]):int(offs[s + 1])] = False
    assert max_abs_err(out[torch.from_numpy(keep).to("cuda")], ref[keep]) <= tol_for(w.dtype)

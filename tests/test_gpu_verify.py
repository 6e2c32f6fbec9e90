"""GPU parity for multi-token decode rows: the verify step of speculative
decoding ("LLM 推理引擎 Continuous Batching 与 PagedAttention" §7.2: the
target model checks a few draft tokens in one pass), query_len 2..8 over long
cached contexts.

Such a sequence has query_len x G query rows per KV head (G = Hq / Hkv).  Up
to 16 rows take the one-tile decode kernel, 17..32 rows the two-tile one
(split-K over the context either way), more rows the prefill kernel; every
class is compared with the oracle, alone and mixed in one batch.
"""
import numpy as np
import pytest
import torch

import oracle
import ragged_paged_attention_amd as rpa
from tests.gpu_path import DeviceRun, capture_stderr, max_abs_err, tol_for
from workloads import verify_batch
from workloads.generators import build_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["auto", "generic"])
def policy(request):
    prev = rpa.pa_set_kernel_policy(rpa.PA_POLICY_AUTO if request.param == "auto" else rpa.PA_POLICY_GENERIC)
    yield request.param
    rpa.pa_set_kernel_policy(prev)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_verify_batch_scaled(seed, dtype, policy):
    w = verify_batch(seed=seed, dtype=dtype, scale_down=8)
    print(f"[verify] seed={seed} {dtype} {policy} {w.summary()}", flush=True)
    g = DeviceRun(w).run()
    _, _, _, ref = oracle.run_step(w)
    assert g.err() == 0
    assert max_abs_err(g.out, ref) <= tol_for(dtype)


def _explicit(Hq, Hkv, ql, ctx, seed, dtype="bf16", bs=16):
    rng = np.random.default_rng(seed)
    sl = [int(c) + int(q) for c, q in zip(ctx, ql)]
    counts = [-(-L // bs) for L in sl]
    NB = int(sum(counts)) + 16
    ids = rng.permutation(NB)
    tables, o = [], 0
    for c in counts:
        tables.append([int(x) for x in ids[o:o + c]])
        o += c
    return build_workload("explicit", dtype, Hq, Hkv, 128, bs, NB, list(ql), sl, tables, seed)


@pytest.mark.parametrize("Hq,Hkv,ql", [
    (32, 8, [1, 2, 3, 4, 5, 6, 7, 8, 9, 0, 40]),     # G 4: rows 4..36, every class, one call
    (32, 2, [1, 2, 3, 1, 2]),                        # G 16: 16 rows, 32 rows, 48 rows
    (16, 16, [17, 32, 16, 1, 33, 20]),               # G 1: two-tile items of 17..32 tokens
    (64, 8, [2, 4, 3, 5, 1]),                        # G 8: 16, 32, 24, 40, 8 rows
], ids=["G4_all_classes", "G16", "G1", "G8"])
def test_row_classes_mixed_in_one_call(Hq, Hkv, ql):
    """Contexts long enough to split into several parts (and one short one
    that does not), so the two-tile partials go through the merge."""
    rng = np.random.default_rng(len(ql) * Hq)
    ctx = [int(x) for x in rng.integers(700, 3000, len(ql))]
    ctx[0] = 40
    w = _explicit(Hq, Hkv, ql, ctx, seed=Hq + Hkv)
    print(f"[verify] classes Hq={Hq} Hkv={Hkv} ql={ql}", flush=True)
    g = DeviceRun(w).run()
    _, _, _, ref = oracle.run_step(w)
    assert g.err() == 0
    assert max_abs_err(g.out, ref) <= tol_for("bf16")


def test_verify_full_size_sampled_rows():
    """The verify workload at full size (64 sequences, query_len 2..8,
    contexts 2k..16k): every row of the 8 longest sequences and of 8 random
    others, against the oracle.  Its two-tile list would fill between one
    and two waves of that launch at the default part length, so the plan
    gives it parts twice as long (the trace says so)."""
    w = verify_batch()
    offs = w.new_row_offsets()
    rng = np.random.default_rng(0)
    pick = set(np.argsort(-w.step.seq_lens)[:8].tolist()) | set(rng.choice(w.num_seqs, 8, replace=False).tolist())
    rows = sorted(r for s in pick for r in range(int(offs[s]), int(offs[s + 1])))
    print(f"[verify] full {w.summary()} rows={len(rows)}", flush=True)
    prev = rpa.pa_set_trace(1)
    try:
        g, text = capture_stderr(lambda: DeviceRun(w).run())
    finally:
        rpa.pa_set_trace(prev)
    assert "(parts of at most 768, 1536 tokens)" in text
    _, _, _, ref = oracle.run_step(w, rows=rows)
    assert g.err() == 0
    err = max_abs_err(g.out[torch.tensor(rows, device="cuda")], ref)
    print(f"[verify] full max_abs_err={err:.3e}", flush=True)
    assert err <= tol_for("bf16")
    assert torch.isfinite(g.out).all()


def test_too_small_query_len_hint_is_flagged():
    """max_query_len = 1 while sequences carry 2..8 rows: PA_DERR_HINT is
    raised; sequences whose rows still fit one decode tile are computed,
    the others come back as zeros (never garbage)."""
    w = verify_batch(seed=3, scale_down=8)
    g = DeviceRun(w).fill_history().write_step_rows()
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.full_like(g.db.q, float("nan"))
    rpa.pa_attention(g.db.q, g.k_cache, g.v_cache, g.db.block_tables, g.meta["query_start_loc"], g.db.seq_lens,
                     1, w.max_seq_len, w.scale, out=out, d_err=d_err)
    torch.cuda.synchronize()
    assert int(d_err.item()) & rpa.PA_DERR_HINT
    _, _, _, ref = oracle.run_step(w)
    offs = w.new_row_offsets()
    G = w.num_q_heads // w.num_kv_heads
    for s in range(w.num_seqs):
        got = out[int(offs[s]):int(offs[s + 1])]
        if int(w.step.query_lens[s]) * G <= 16:
            assert max_abs_err(got, ref[int(offs[s]):int(offs[s + 1])]) <= tol_for(w.dtype)
        else:
            assert bool((got == 0).all())

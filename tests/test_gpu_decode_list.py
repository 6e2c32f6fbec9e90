"""GPU parity of the decode kernels driven by the plan's work lists.

When the planning kernel runs (prefill rows or possible shared prefixes), it
lists every (sequence, part) item of the one-tile and two-tile decode
instances, heaviest part first, and the decode grids take those lists instead
of walking every (sequence, KV head, part) slot.  Which workgroup computes an
item changes nothing in the result, so the plain oracle is the reference
("LLM 推理引擎 Continuous Batching 与 PagedAttention" §3.3: parts of a context
combined by the running-max rescaling).  The cases use sequence counts that
are not multiples of the 16-entry XCD runs, both item orders (fewer and more
than 16 KV heads), contexts from 1 to ~9000 tokens (many parts), two-tile
verify rows and a violated max_query_len hint.
"""
import numpy as np
import pytest
import torch

import oracle
import ragged_paged_attention_amd as rpa
from tests.gpu_path import DeviceRun, max_abs_err, tol_for
from workloads.generators import build_workload

pytestmark = pytest.mark.gpu


def _batch(Hq, Hkv, ql, sl, seed, bs=16):
    rng = np.random.default_rng(seed)
    counts = [-(-L // bs) for L in sl]
    NB = int(sum(counts)) + 16
    ids = rng.permutation(NB)
    tables, o = [], 0
    for c in counts:
        tables.append([int(x) for x in ids[o:o + c]])
        o += c
    return build_workload("decode_list", "bf16", Hq, Hkv, 128, bs, NB, list(ql), list(sl), tables, seed)


def _mixed(S, Hq, Hkv, seed):
    rng = np.random.default_rng(seed)
    ctx = [int(x) for x in np.rint(np.exp(rng.uniform(0, np.log(9000), S)))]
    ql = [1] * S
    ql[S // 3] = 300                      # a prefill chunk: the plan runs
    ql[S // 2] = 5                        # verify rows (two-tile at G >= 4)
    ql[S - 1] = 2
    sl = [max(c, 1) + q - 1 for c, q in zip(ctx, ql)]
    sl[0] = 1                             # a one-token context
    return _batch(Hq, Hkv, ql, sl, seed)


@pytest.mark.parametrize("S,Hq,Hkv", [(37, 32, 8), (21, 32, 32), (50, 16, 4)], ids=["grouped37", "flat21", "g4_50"])
def test_decode_lists_match_oracle(S, Hq, Hkv):
    w = _mixed(S, Hq, Hkv, seed=S)
    print(f"[decode_list] {w.summary()}", flush=True)
    rpa.pa_bench_timing_begin()
    g = DeviceRun(w).run()
    t = rpa.pa_bench_timing_end()
    assert "attn_plan_kernel" in t       # the lists exist in this call
    _, _, _, ref = oracle.run_step(w)
    assert g.err() == 0
    err = max_abs_err(g.out, ref)
    print(f"[decode_list] max_abs_err={err:.3e}", flush=True)
    assert err <= tol_for("bf16")


def test_decode_lists_zero_fill_when_hint_is_violated():
    """Shared-prefix detection makes the plan run without prefill rows; a
    sequence longer than the max_query_len hint then gets a zero-fill entry
    in the one-tile list and PA_DERR_HINT is raised, while the others are
    computed."""
    S = 12
    ql = [1] * S
    ql[4] = 9                             # 36 rows at G = 4: above the one-tile cap of the hint
    sl = [2100 + 37 * i for i in range(S)]
    w = _batch(32, 8, ql, sl, seed=9)
    g = DeviceRun(w).fill_history().write_step_rows()
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.full_like(g.db.q, float("nan"))
    rpa.pa_bench_timing_begin()
    rpa.pa_attention(g.db.q, g.k_cache, g.v_cache, g.db.block_tables, g.meta["query_start_loc"], g.db.seq_lens,
                     1, w.max_seq_len, w.scale, out=out, d_err=d_err)
    torch.cuda.synchronize()
    t = rpa.pa_bench_timing_end()
    assert "attn_plan_kernel" in t
    assert int(d_err.item()) & rpa.PA_DERR_HINT
    _, _, _, ref = oracle.run_step(w)
    offs = w.new_row_offsets()
    for s in range(S):
        got = out[int(offs[s]):int(offs[s + 1])]
        if s == 4:
            assert bool((got == 0).all())
        else:
            assert max_abs_err(got, ref[int(offs[s]):int(offs[s + 1])]) <= tol_for("bf16")

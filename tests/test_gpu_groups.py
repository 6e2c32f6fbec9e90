"""GPU parity at GQA group sizes that are not powers of two, and KV head counts
that are not multiples of 4.

"LLM 推理引擎 Continuous Batching 与 PagedAttention" §3.1 and "vLLM 原理" §3.2
put the query heads of one KV head in a group that shares its K/V; nothing
there ties the group size to a power of two.  The fast kernels pack a
sequence's rows as (query, head in group) pairs, so a group of 3, 5 or 6
heads makes 128-row prefill tiles, 16/32-row decode tiles and cascade rows
split in the middle of a query; a KV head count that 4 does not divide
changes how the prefill work list groups heads per XCD run.  The plain oracle
is the reference for all of them.
"""
import numpy as np
import pytest

import oracle
import ragged_paged_attention_amd as rpa
from tests.gpu_path import DeviceRun, max_abs_err, tol_for
from workloads.generators import build_workload

pytestmark = pytest.mark.gpu


def _batch(Hq, Hkv, ql, sl, seed, dtype="bf16", bs=16, shared=None, tables=None):
    rng = np.random.default_rng(seed)
    counts = [-(-L // bs) for L in sl]
    NB = int(sum(counts)) + 16
    if tables is None:
        ids = rng.permutation(NB)
        tables, o = [], 0
        for c in counts:
            tables.append([int(x) for x in ids[o:o + c]])
            o += c
    kw = dict(shared=shared) if shared else {}
    return build_workload(f"groups_{Hq}x{Hkv}", dtype, Hq, Hkv, 128, bs, NB, list(ql), list(sl), tables, seed,
                          rng, **kw)


# decode rows, verify rows (query_len 2..7, so G x q crosses the 16- and
# 32-row decode tiles), prefill chunks of lengths that end mid-tile, a one-token
# context and a context long enough for several split-K parts
QL = [1, 5, 1, 43, 3, 1, 7, 300, 1, 2]
SL = [2900, 905, 1, 43, 1203, 640, 2007, 1500, 17, 4100]


@pytest.mark.parametrize("Hq,Hkv", [(6, 2), (15, 3), (12, 2), (6, 3), (10, 5), (24, 8)],
                         ids=["g3", "g5", "g6", "kv3", "kv5", "g3kv8"])
def test_group_sizes_match_oracle(Hq, Hkv):
    w = _batch(Hq, Hkv, QL, SL, seed=Hq * 10 + Hkv)
    print(f"[groups] Hq={Hq} Hkv={Hkv}", flush=True)
    rpa.pa_bench_timing_begin()
    g = DeviceRun(w).run()
    t = rpa.pa_bench_timing_end()
    _, _, _, ref = oracle.run_step(w)
    assert g.err() == 0
    err = max_abs_err(g.out, ref)
    print(f"[groups] max_abs_err={err:.3e} kernels={sorted(t)}", flush=True)
    assert err <= tol_for("bf16")
    assert "decode_kernel" in t and "prefill_kernel" in t  # the fast kernels ran


def test_group_of_five_fp16():
    w = _batch(20, 4, [1, 6, 129, 1], [3000, 700, 129, 9], seed=5, dtype="f16")
    g = DeviceRun(w).run()
    _, _, _, ref = oracle.run_step(w)
    assert g.err() == 0
    assert max_abs_err(g.out, ref) <= tol_for("f16")


def test_shared_prefix_group_of_three():
    """Cascade rows are (member, query head) pairs: with 3 heads per group a
    prefix part's 128 rows hold 42 members and a partial one."""
    bs, prefix = 16, 2048
    rng = np.random.default_rng(11)
    n = 45                                    # more members than one 128-row part holds at G = 3
    sl = [prefix + int(x) for x in rng.integers(1, 400, n)]
    ql = [1] * n
    need = prefix // bs + sum(-(-L // bs) - prefix // bs for L in sl)
    NB = need + 16
    ids = iter(int(x) for x in rng.permutation(NB))
    pre = [next(ids) for _ in range(prefix // bs)]
    tables = [pre + [next(ids) for _ in range(-(-L // bs) - prefix // bs)] for L in sl]
    w = _batch(24, 8, ql, sl, seed=11, tables=tables, shared=[(list(range(n)), prefix)])
    rpa.pa_bench_timing_begin()
    g = DeviceRun(w).run()
    t = rpa.pa_bench_timing_end()
    _, _, _, ref = oracle.run_step(w)
    assert g.err() == 0
    assert max_abs_err(g.out, ref) <= tol_for("bf16")
    assert "prefill_kernel" in t  # decode rows only: the prefill kernel ran for the prefix parts

"""GPU parity of shared-prefix (cascade) decode, and a guard on workspace use.

Sequences whose block tables map the same physical blocks at the same logical
positions share those blocks' contents ("vLLM 原理" §2.1; the shared prefixes
and prefix caching of "LLM 推理引擎 Continuous Batching 与 PagedAttention"
§4.1, §4.2).  pa_attention groups single-token decode sequences whose tables
start with the same block and agree on at least 1024 tokens, wherever they
sit in the batch, reads each such prefix once for the whole group, and merges
it with every member's own suffix.  The results must be those of
plain per-sequence attention (the oracle), whatever the grouping.
"""
import re

import numpy as np
import pytest
import torch

import oracle
import ragged_paged_attention_amd as rpa
from tests.gpu_path import DeviceRun, capture_stderr, max_abs_err, one_stream_output, tol_for
from workloads import config, permute_sequences, unshare, verify_batch
from workloads.generators import build_workload

pytestmark = pytest.mark.gpu


def grouped_batch(seed, segments, Hq, Hkv, dtype="bf16", bs=16):
    """segments, in batch order: ("group", members, prefix_tokens, tail_lo,
    tail_hi) -- decode sequences sharing `prefix_tokens` (a multiple of bs)
    then a private tail of tail_lo..tail_hi tokens -- or ("single", query_len,
    seq_len) -- a sequence with private blocks only."""
    rng = np.random.default_rng(seed)
    ql, sl, shared, plan = [], [], [], []
    for seg in segments:
        if seg[0] == "group":
            _, n, prefix, lo, hi = seg
            assert prefix % bs == 0
            first = len(ql)
            for _ in range(n):
                ql.append(1)
                sl.append(prefix + int(rng.integers(lo, hi + 1)))
            shared.append((list(range(first, first + n)), prefix))
            plan.append(("group", first, n, prefix))
        else:
            _, q, L = seg
            ql.append(q)
            sl.append(L)
            plan.append(("single", len(ql) - 1))
    need = 0
    for p in plan:
        if p[0] == "group":
            _, first, n, prefix = p
            need += prefix // bs + sum(-(-sl[k] // bs) - prefix // bs for k in range(first, first + n))
        else:
            need += -(-sl[p[1]] // bs)
    NB = need + 32
    ids = iter(int(x) for x in rng.permutation(NB))
    tables = [None] * len(ql)
    for p in plan:
        if p[0] == "group":
            _, first, n, prefix = p
            pre = [next(ids) for _ in range(prefix // bs)]
            for k in range(first, first + n):
                tables[k] = pre + [next(ids) for _ in range(-(-sl[k] // bs) - prefix // bs)]
        else:
            tables[p[1]] = [next(ids) for _ in range(-(-sl[p[1]] // bs))]
    return build_workload("grouped", dtype, Hq, Hkv, 128, bs, NB, ql, sl, tables, seed, rng, shared=shared)


# the launch considers cascades only when max_seq_len >= 2048; one long
# sequence in a batch of shorter ones makes the hint say so
LONG = ("single", 1, 2100)

CASES = {
    # three groups of different sizes and prefix lengths (1040 and 1520 are
    # not whole 64-token tiles: the shared part is rounded down), singles in between
    "three_groups": dict(Hq=32, Hkv=4, segs=[("group", 5, 2048, 1, 200), ("single", 1, 900),
                                             ("group", 2, 1040, 1, 40), ("single", 37, 1500),
                                             ("group", 9, 1520, 30, 300)]),
    # a run of sharing decodes interrupted by a multi-token sequence
    "interrupted": dict(Hq=16, Hkv=2, segs=[("group", 3, 1536, 1, 64), ("single", 3, 1600),
                                            ("group", 4, 1536, 1, 64), LONG]),
    # G = 1: at most 128 members per group, so 150 sharing sequences make two groups
    "g1_many_members": dict(Hq=4, Hkv=4, segs=[("group", 150, 1024, 1, 50), LONG]),
    # more groups than prefix slots: the first 64 groups are cascaded, the rest not
    "seventy_pairs": dict(Hq=16, Hkv=2, segs=[("group", 2, 1024, 1, 20)] * 70 + [LONG]),
    # just under the 1024-token threshold (no cascade) next to exactly 1024
    "threshold": dict(Hq=16, Hkv=2, segs=[("group", 4, 1008, 1, 30), ("single", 1, 50),
                                          ("group", 4, 1024, 1, 30), LONG]),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_cascade_matches_oracle(name):
    c = CASES[name]
    w = grouped_batch(len(name), c["segs"], c["Hq"], c["Hkv"])
    print(f"[cascade] {name} {w.summary()}", flush=True)
    g = DeviceRun(w).run()
    _, _, _, ref = oracle.run_step(w)
    assert g.err() == 0
    err = max_abs_err(g.out, ref)
    print(f"[cascade] {name} max_abs_err={err:.3e}", flush=True)
    assert err <= tol_for(w.dtype)


def test_cascade_fp16_and_generic_agree():
    w = grouped_batch(11, [("group", 6, 2048, 1, 100), ("single", 1, 3000)], 32, 4, dtype="f16")
    g = DeviceRun(w).run()
    _, _, _, ref = oracle.run_step(w)
    assert max_abs_err(g.out, ref) <= tol_for("f16")
    prev = rpa.pa_set_kernel_policy(rpa.PA_POLICY_GENERIC)
    try:
        g2 = DeviceRun(w).run()
    finally:
        rpa.pa_set_kernel_policy(prev)
    assert max_abs_err(g.out, g2.out.to(torch.float64).cpu().numpy()) <= tol_for("f16")


@pytest.mark.parametrize("make", [lambda: config(2, scale_down=2), lambda: config(4, scale_down=8),
                                  lambda: config(5, scale_down=4), lambda: verify_batch(scale_down=4),
                                  lambda: grouped_batch(3, [("group", 5, 2048, 1, 200)], 32, 4)],
                         ids=["ragged_prefill", "chunked_mixed", "shared_prefix", "verify", "grouped"])
def test_workspace_writes_stay_inside_reported_size(make):
    """Every workspace byte pa_attention touches lies below
    pa_attention_workspace_size(): a guard region right after it keeps its
    pattern."""
    w = make()
    g = DeviceRun(w).fill_history().write_step_rows()
    need = rpa.pa_attention_workspace_size(w.num_seqs, w.num_tokens, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                           max(1, w.max_query_len), max(1, w.max_seq_len))
    guard = 1 << 16
    buf = torch.full((need + guard,), 0xA5, dtype=torch.uint8, device="cuda")
    print(f"[cascade] guard {w.name} need={need}", flush=True)
    out = rpa.pa_attention(g.db.q, g.k_cache, g.v_cache, g.db.block_tables, g.meta["query_start_loc"],
                           g.db.seq_lens, max(1, w.max_query_len), max(1, w.max_seq_len), w.scale,
                           workspace=buf[:max(need, 1)])
    torch.cuda.synchronize()
    assert bool((buf[need:] == 0xA5).all())
    _, _, _, ref = oracle.run_step(w, rows=[0, w.num_tokens - 1])
    assert max_abs_err(out[[0, w.num_tokens - 1]], ref) <= tol_for(w.dtype)


@pytest.mark.parametrize("scale_down", [1, 4])
def test_grouping_does_not_depend_on_batch_order(scale_down):
    """The shared-prefix batch, its sequences shuffled: every sequence's output
    is bit-identical to the unshuffled run's (the same groups, prefixes and
    parts are found however the sharers are spread over the batch), the
    grouping is really used (a copy with private blocks gives other bits),
    and both match the oracle."""
    w = config(5, scale_down=scale_down)
    perm = np.random.default_rng(17).permutation(w.num_seqs)
    wp = permute_sequences(w, perm)
    print(f"[cascade order] {w.summary()}", flush=True)
    a = DeviceRun(w).run().out
    b = DeviceRun(wp).run().out
    inv = np.argsort(perm)          # sequences are single-token: row i is sequence i
    b_back = b[torch.from_numpy(inv).to("cuda")]
    assert torch.equal(a.view(torch.int16), b_back.view(torch.int16))
    w.num_blocks += int((w.step.block_tables >= 0).sum())
    used = set(int(x) for x in w.step.block_tables.ravel() if x >= 0)
    u = unshare(w, [x for x in range(w.num_blocks) if x not in used])
    c = DeviceRun(u).run().out
    assert not torch.equal(a.view(torch.int16), c.view(torch.int16))
    rows = list(range(0, w.num_tokens, max(1, w.num_tokens // 16)))
    _, _, _, ref = oracle.run_step(wp, rows=rows)
    assert max_abs_err(b[torch.tensor(rows, device="cuda")], ref) <= tol_for(w.dtype)


def test_trace_lists_the_groups():
    """With the plan trace on, the call prints its plan: the three groups of
    the three_groups batch with their members and prefix tokens (2048; 1040
    and 1520 rounded down to whole 64-token tiles), and the output still
    matches the oracle."""
    c = CASES["three_groups"]
    w = grouped_batch(len("three_groups"), c["segs"], c["Hq"], c["Hkv"])
    prev = rpa.pa_set_trace(1)
    try:
        g, text = capture_stderr(lambda: DeviceRun(w).run())
    finally:
        rpa.pa_set_trace(prev)
    print(text, flush=True)
    assert "path=fast" in text and "shared_prefix=1" in text
    groups = {}
    for m in re.finditer(r"group \d+: prefix_tokens=(\d+) parts=(\d+) first_prefix_slot=\d+ members=(\d+) "
                         r"\[([0-9 ]*)\]", text):
        members = tuple(sorted(int(x) for x in m.group(4).split()))
        assert len(members) == int(m.group(3)) and int(m.group(2)) >= 1
        groups[members] = int(m.group(1))
    assert groups == {tuple(range(0, 5)): 2048, (6, 7): 1024, tuple(range(9, 18)): 1472}
    assert "d_err=0x0" in text
    _, _, _, ref = oracle.run_step(w)
    assert max_abs_err(g.out, ref) <= tol_for(w.dtype)


def test_groups_beside_prefill_chunks():
    """Shared prefixes in a large mixed batch: 66 decodes in three groups
    next to four prefill chunks run with the decode launches beside the
    prefill kernel (which also takes the groups' prefix parts).  The groups
    form as on their own, the output equals the one-stream path bit for bit
    and matches the oracle on every row."""
    segs = [("group", 22, 2048, 1, 200), ("single", 96, 1500), ("group", 22, 1024, 1, 300),
            ("single", 160, 2200), ("group", 22, 1536, 1, 300), ("single", 128, 900), ("single", 112, 2000)]
    w = grouped_batch(31, segs, 32, 8)
    print(f"[case] groups beside chunks: {w.summary()}", flush=True)
    need = rpa.pa_attention_workspace_size(w.num_seqs, w.num_tokens, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                           w.max_query_len, w.max_seq_len)
    prev = rpa.pa_set_trace(1)
    try:
        g, text = capture_stderr(lambda: DeviceRun(w).run())
    finally:
        rpa.pa_set_trace(prev)
    assert "decode_beside_prefill=1" in text and "shared_prefix=1" in text
    sizes = sorted(int(m.group(1)) for m in re.finditer(r"group \d+: prefix_tokens=(\d+)", text))
    assert sizes == [1024, 1536, 2048]
    assert g.err() == 0
    serial = one_stream_output(g, need)
    assert torch.equal(g.out.view(torch.int16), serial.view(torch.int16))
    _, _, _, ref = oracle.run_step(w)
    err = max_abs_err(g.out, ref)
    print(f"[groups beside chunks] max_abs_err={err:.3e}", flush=True)
    assert err <= tol_for(w.dtype)

"""CPU checks of the needle workloads used by the full-size GPU parity tests.

Each sequence reads only its own blocks, which may sit anywhere in the pool
("vLLM Continuous Batching：从 Forward Shape 理解两个核心参数" §2.3补充).  With
plain N(0, 1) data a long context averages thousands of value rows, so a
block read from the wrong place moves an output by far less than the bf16
tolerance.  A needle workload plants one dominant key per (sequence, KV
head); these tests show on the oracle that (a) every output row is then the
needle's V row, and (b) reading one block from the wrong place -- a mistake
planted in the oracle -- moves the affected rows by O(1), far beyond 2e-2.
"""
import numpy as np
import pytest

import oracle
from oracle import paged_attention as PA
from workloads import config, plant_needles

TOL_BF16 = 2e-2


def _needle_value_rows(w):
    """Per flat row and query head: the V row of the key with the largest
    score, found by brute force over the sequence's logical rows."""
    G = w.num_q_heads // w.num_kv_heads
    offs = w.new_row_offsets()
    best = np.zeros((w.num_tokens, w.num_q_heads, w.head_dim))
    for s in range(w.num_seqs):
        k, v = w.logical_kv(s)
        k64, v64 = PA.widen(k, w.dtype), PA.widen(v, w.dtype)
        L, ql = int(w.step.seq_lens[s]), int(w.step.query_lens[s])
        for i in range(ql):
            t = int(offs[s]) + i
            q64 = PA.widen(w.q[t], w.dtype)
            for h in range(w.num_q_heads):
                sc = k64[:L - ql + i + 1, h // G] @ q64[h]
                best[t, h] = v64[int(np.argmax(sc)), h // G]
    return best


@pytest.mark.parametrize("n", [3, 4, 5])
def test_needle_rows_equal_needle_values(n):
    w = plant_needles(config(n, scale_down=16), seed=n)
    _, _, _, out = oracle.run_step(w)
    np.testing.assert_allclose(out, _needle_value_rows(w), rtol=0, atol=1e-6)


@pytest.mark.parametrize("n", [3, 5])
def test_one_misrouted_block_is_caught(n, monkeypatch):
    """Plant a wrong-block read in the oracle: the block holding sequence 0's
    needle (KV head 0) is taken from another block of the pool.  The row of
    sequence 0 then differs from the correct one by more than ten times the
    bf16 tolerance."""
    w = plant_needles(config(n, scale_down=4), seed=1)
    _, _, _, good = oracle.run_step(w, rows=[0])
    k, _ = w.logical_kv(0)
    q64 = PA.widen(w.q[0], w.dtype)
    j = int(np.argmax(PA.widen(k, w.dtype)[:, 0] @ q64[0]))   # the needle of KV head 0
    lb = j // w.block_size
    mine = int(w.step.block_tables[0, lb])
    other = next(int(b) for b in w.step.block_tables[-1] if b >= 0 and b != mine)
    real_gather = PA.gather_sequence

    def misrouted(cache, row, seq_len, dtype):
        row = np.array(row, copy=True)
        if row[lb] == mine:
            row[lb] = other
        return real_gather(cache, row, seq_len, dtype)

    monkeypatch.setattr(PA, "gather_sequence", misrouted)
    _, _, _, bad = oracle.run_step(w, rows=[0])
    diff = float(np.max(np.abs(bad - good)))
    print(f"one misrouted block moves sequence 0's row by {diff:.3e}")
    assert diff > 10 * TOL_BF16, diff

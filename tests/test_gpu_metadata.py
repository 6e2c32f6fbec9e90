"""pa_build_metadata against the oracle's build_metadata, bit for bit, on
both launch shapes: one launch for a batch of up to 1024 sequences (a scan
workgroup beside one fill workgroup per sequence), a scan launch followed by
a fill grid for larger batches ("vLLM Continuous Batching：从 Forward Shape
理解两个核心参数" §2.1 running sums and positions, §2.3 slots).  Sequences with
no new token, history-only contexts and the flag for offsets past INT32_MAX
are covered on both sides of the boundary."""
import numpy as np
import pytest
import torch

import oracle
import ragged_paged_attention_amd as rpa

pytestmark = pytest.mark.gpu

BS = 16


def _batch(S, seed):
    """S sequences: 0..5 new tokens (0 = a sequence that only holds history
    this step), 0..60 history tokens, random distinct blocks of a pool."""
    rng = np.random.default_rng(seed)
    ql = rng.integers(0, 6, S).astype(np.int32)
    sl = (ql + rng.integers(0, 61, S)).astype(np.int32)
    used = -(-sl // BS)
    MB = max(1, int(used.max()))
    NB = int(used.sum()) + 7
    ids = rng.permutation(NB).astype(np.int32)
    bt = np.zeros((S, MB), dtype=np.int32)
    o = 0
    for s in range(S):
        bt[s, :used[s]] = ids[o:o + used[s]]
        o += used[s]
    return ql, sl, bt, NB


@pytest.mark.parametrize("S", [1, 2, 1023, 1024, 1025, 3000])
def test_metadata_bitexact_both_launch_shapes(S):
    ql, sl, bt, NB = _batch(S, seed=S)
    T = int(ql.sum())
    print(f"[case] metadata S={S} T={T} NB={NB}", flush=True)
    dev = lambda a: torch.from_numpy(a).to("cuda")
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    md = rpa.pa_build_metadata(dev(ql), dev(sl), T, dev(bt), BS, NB, d_err=d_err)
    torch.cuda.synchronize()
    ref = oracle.build_metadata(ql, sl, T, bt, BS, NB)
    assert int(d_err.item()) == 0
    assert md["query_start_loc"].cpu().numpy().tolist() == ref.query_start_loc.tolist()
    assert md["seq_start_loc"].cpu().numpy().tolist() == ref.seq_start_loc.tolist()
    assert md["positions"].cpu().numpy().tolist() == ref.positions.tolist()
    assert md["token_to_seq"].cpu().numpy().tolist() == ref.token_to_seq.tolist()
    assert md["slot_mapping"].cpu().numpy().tolist() == ref.slot_mapping.tolist()
    assert md["stats"].cpu().numpy().tolist() == ref.stats.tolist()


@pytest.mark.parametrize("S", [3, 1100])
def test_offsets_past_int32_are_flagged(S):
    """Contexts of 2^30 tokens: seq_start_loc passes INT32_MAX after two
    sequences, which sets PA_DERR_OVERFLOW (the clamped offsets are not
    specified); the one new token of each sequence still gets its position."""
    ql = np.ones(S, dtype=np.int32)
    sl = np.full(S, 1 << 30, dtype=np.int32)
    dev = lambda a: torch.from_numpy(a).to("cuda")
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    md = rpa.pa_build_metadata(dev(ql), dev(sl), S, None, 1, 1, d_err=d_err)
    torch.cuda.synchronize()
    assert int(d_err.item()) & rpa.PA_DERR_OVERFLOW
    assert md["query_start_loc"].cpu().numpy().tolist() == list(range(S + 1))
    assert md["positions"].cpu().numpy().tolist() == [(1 << 30) - 1] * S

"""Stream ordering of a call that uses the library's side stream: on a large
mixed batch the prefill kernel runs on the side stream beside the decode
launches, and the call joins it back into the caller's stream before the
merge.  Work the caller enqueues on its own (non-default) stream after the
call must see the finished output: a copy taken on that stream right after
the call, with no device-wide synchronisation in between, equals the output
read after everything is done.  (The parity tests synchronise the whole
device before they compare, which would hide a missing join.)"""
import pytest
import torch

import ragged_paged_attention_amd as rpa
from tests.gpu_path import DeviceRun, capture_stderr
from workloads import config

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fused", [False, True], ids=["attention", "write_kv_attention"])
def test_callers_stream_sees_the_side_streams_work(fused):
    w = config(4, scale_down=4)
    g = DeviceRun(w).fill_history()
    db = g.db
    md = rpa.pa_build_metadata(db.query_lens, db.seq_lens, w.num_tokens, db.block_tables, w.block_size,
                               w.num_blocks, d_err=g.d_err)
    rpa.pa_write_kv(db.k, db.v, md["slot_mapping"], g.k_cache, g.v_cache, d_err=g.d_err)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    snaps, outs = [], []
    prev = rpa.pa_set_trace(0)
    try:
        with torch.cuda.stream(s):
            for _ in range(3):
                out = torch.full_like(db.q, float("nan"))
                if fused:
                    rpa.pa_write_kv_attention(db.k, db.v, md["slot_mapping"], db.q, g.k_cache, g.v_cache,
                                              db.block_tables, md["query_start_loc"], db.seq_lens, w.max_query_len,
                                              w.max_seq_len, w.scale, out=out, d_err=g.d_err)
                else:
                    rpa.pa_attention(db.q, g.k_cache, g.v_cache, db.block_tables, md["query_start_loc"],
                                     db.seq_lens, w.max_query_len, w.max_seq_len, w.scale, out=out, d_err=g.d_err)
                snaps.append(out.clone())  # enqueued on s, right behind the call
                outs.append(out)
    finally:
        rpa.pa_set_trace(prev)
    torch.cuda.synchronize()
    assert g.err() == 0
    for snap, out in zip(snaps, outs):
        assert not torch.isnan(out).any()
        assert torch.equal(snap.view(torch.int16), out.view(torch.int16))
    # the batch does take the side stream
    _, text = capture_stderr(lambda: _traced_call(g, w, md))
    assert "decode_beside_prefill=1" in text


def _traced_call(g, w, md):
    prev = rpa.pa_set_trace(1)
    try:
        db = g.db
        return rpa.pa_attention(db.q, g.k_cache, g.v_cache, db.block_tables, md["query_start_loc"], db.seq_lens,
                                w.max_query_len, w.max_seq_len, w.scale, d_err=g.d_err)
    finally:
        rpa.pa_set_trace(prev)

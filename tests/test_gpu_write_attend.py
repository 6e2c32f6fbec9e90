"""pa_write_kv_attention (the KV write and the attention in one call, as the
attention layer's forward of "vLLM 原理" §3.7 stores then attends) against
pa_write_kv followed by pa_attention: the same caches and the same output,
bit for bit, on every path the call can take -- the write in the planning
launch's extra workgroups (large mixed batch with the CU split, planned
batches without it, shared-prefix groups), the write first on the caller's
stream (no plan; rows not 16-byte aligned; validation on; the generic
kernel) -- and the oracle on top."""
import numpy as np
import pytest
import torch

import oracle
import ragged_paged_attention_amd as rpa
from tests.gpu_path import DeviceRun, capture_stderr, max_abs_err, tol_for
from tests.test_gpu_cascade import grouped_batch
from workloads import config, verify_batch

pytestmark = pytest.mark.gpu

CASES = {
    "mixed_split": lambda: config(4, scale_down=4),         # 64 sequences: decode beside prefill
    "ragged_prefill": lambda: config(2, scale_down=4),      # a plan, no split
    "verify": lambda: verify_batch(scale_down=4),           # a plan (contexts long enough for shared prefixes)
    "decode_no_plan": lambda: config(3, scale_down=8),      # no plan: the write goes first
    "tiny_generic": lambda: config(1),                      # fp32: the generic kernel
    # the same mixed batch in fp16, and with blocks of 32 and of 8 tokens
    # (the instances for block sizes that divide 16)
    "mixed_split_f16": lambda: config(4, scale_down=4, dtype="f16"),
    "mixed_bs32": lambda: config(4, scale_down=4, block_size=32),
    "mixed_bs8": lambda: config(4, scale_down=4, block_size=8),
    # three shared-prefix groups next to prefill chunks: cascade matching
    # reads block tables while the write fills the groups' new rows
    "groups_split": lambda: grouped_batch(31, [("group", 22, 2048, 1, 200), ("single", 96, 1500),
                                               ("group", 22, 1024, 1, 300), ("single", 160, 2200),
                                               ("group", 22, 1536, 1, 300), ("single", 128, 900),
                                               ("single", 112, 2000)], 32, 8),
}
# where the trace says the write went ("in_plan": workgroups of the planning
# launch; "first": its own launch before everything else on the caller's
# stream); the generic kernel prints no split line
WRITE_AT = {"mixed_split": "in_plan", "ragged_prefill": "in_plan", "verify": "in_plan",
            "decode_no_plan": "first", "tiny_generic": None, "groups_split": "in_plan",
            "mixed_split_f16": "in_plan", "mixed_bs32": "in_plan", "mixed_bs8": "in_plan"}


def _separate(w, g):
    """pa_write_kv then pa_attention into fresh caches holding the same history."""
    h = DeviceRun(w).fill_history()
    md = rpa.pa_build_metadata(h.db.query_lens, h.db.seq_lens, w.num_tokens, h.db.block_tables, w.block_size,
                               w.num_blocks, d_err=h.d_err)
    rpa.pa_write_kv(h.db.k, h.db.v, md["slot_mapping"], h.k_cache, h.v_cache, d_err=h.d_err)
    out = rpa.pa_attention(h.db.q, h.k_cache, h.v_cache, h.db.block_tables, md["query_start_loc"], h.db.seq_lens,
                           max(1, w.max_query_len), max(1, w.max_seq_len), w.scale, d_err=h.d_err)
    torch.cuda.synchronize()
    return h, out


@pytest.mark.parametrize("name", list(CASES))
def test_fused_write_and_attention_equal_the_two_calls(name):
    w = CASES[name]()
    print(f"[case] {name} {w.summary()}", flush=True)
    prev = rpa.pa_set_trace(1)
    try:
        g, text = capture_stderr(lambda: DeviceRun(w).run())   # forward_step: metadata, then the fused call
    finally:
        rpa.pa_set_trace(prev)
    if name in ("mixed_split", "groups_split", "mixed_split_f16", "mixed_bs32"):
        assert "decode_beside_prefill=1" in text
    if WRITE_AT[name]:
        assert f"kv_write={WRITE_AT[name]}" in text
    else:
        assert "path=generic" in text
    h, out = _separate(w, g)
    assert g.err() == 0 and h.err() == 0
    assert torch.equal(g.k_cache.view(torch.int8), h.k_cache.view(torch.int8))
    assert torch.equal(g.v_cache.view(torch.int8), h.v_cache.view(torch.int8))
    assert torch.equal(g.out.view(torch.int8), out.view(torch.int8))
    _, _, _, ref = oracle.run_step(w)
    err = max_abs_err(g.out, ref)
    print(f"[fused] {name}: max_abs_err={err:.3e}", flush=True)
    assert err <= tol_for(w.dtype)


def _fused(g, w, k, v, slots, md):
    rpa.pa_write_kv_attention(k, v, slots, g.db.q, g.k_cache, g.v_cache, g.db.block_tables, md["query_start_loc"],
                              g.db.seq_lens, max(1, w.max_query_len), max(1, w.max_seq_len), w.scale, out=g.out,
                              d_err=g.d_err)


def test_fused_write_of_unaligned_rows_goes_first():
    """New k/v rows that start 2 bytes past a 16-byte boundary: the planning
    launch's workgroups copy 16-byte chunks only, so the write runs as its own
    launch first; the caches and output still equal the two separate calls."""
    w = config(2, scale_down=4)
    g = DeviceRun(w).fill_history()
    md = rpa.pa_build_metadata(g.db.query_lens, g.db.seq_lens, w.num_tokens, g.db.block_tables, w.block_size,
                               w.num_blocks, d_err=g.d_err)
    kbuf = torch.empty(g.db.k.numel() + 1, dtype=g.db.k.dtype, device=g.db.k.device)
    vbuf = torch.empty_like(kbuf)
    k = kbuf[1:].view(g.db.k.shape)
    v = vbuf[1:].view(g.db.v.shape)
    k.copy_(g.db.k)
    v.copy_(g.db.v)
    assert k.data_ptr() % 16 == 2
    g.out = torch.full_like(g.db.q, float("nan"))
    prev = rpa.pa_set_trace(1)
    try:
        _, text = capture_stderr(lambda: _fused(g, w, k, v, md["slot_mapping"], md))
    finally:
        rpa.pa_set_trace(prev)
    assert "kv_write=first" in text and "prefill_rows=1" in text
    h, out = _separate(w, g)
    assert g.err() == 0 and h.err() == 0
    assert torch.equal(g.k_cache.view(torch.int8), h.k_cache.view(torch.int8))
    assert torch.equal(g.v_cache.view(torch.int8), h.v_cache.view(torch.int8))
    assert torch.equal(g.out.view(torch.int8), out.view(torch.int8))


def test_fused_call_flags_duplicate_slots_with_validation():
    """With validation on, the write inside the fused call checks for
    repeated slots like pa_write_kv does."""
    w = config(4, scale_down=4)
    g = DeviceRun(w).fill_history()
    md = rpa.pa_build_metadata(g.db.query_lens, g.db.seq_lens, w.num_tokens, g.db.block_tables, w.block_size,
                               w.num_blocks, d_err=g.d_err)
    slots = md["slot_mapping"].clone()
    slots[5] = slots[3]
    g.out = torch.empty_like(g.db.q)
    prev = rpa.pa_set_validation(1)
    prev_t = rpa.pa_set_trace(1)
    try:
        _, text = capture_stderr(lambda: _fused(g, w, g.db.k, g.db.v, slots, md))
    finally:
        rpa.pa_set_validation(prev)
        rpa.pa_set_trace(prev_t)
    assert "kv_write=first" in text  # validation's check is a launch of its own, before the write
    assert g.err() & rpa.PA_DERR_DUP_SLOT


def test_fused_write_flags_slots_past_the_pool():
    """A slot past the pool, written by the planning launch's workgroups:
    PA_DERR_SLOT_OOB, and no cache row changes but the ones the other
    tokens name."""
    w = config(2, scale_down=4)
    g = DeviceRun(w).fill_history()
    md = rpa.pa_build_metadata(g.db.query_lens, g.db.seq_lens, w.num_tokens, g.db.block_tables, w.block_size,
                               w.num_blocks, d_err=g.d_err)
    torch.cuda.synchronize()
    assert g.err() == 0
    slots = md["slot_mapping"].clone()
    bad = w.num_tokens // 2
    slots[bad] = w.num_blocks * w.block_size
    h = DeviceRun(w).fill_history()
    slots_h = slots.clone()
    slots_h[bad] = -1  # the same write with that row skipped
    rpa.pa_write_kv(h.db.k, h.db.v, slots_h, h.k_cache, h.v_cache, d_err=h.d_err)
    g.out = torch.empty_like(g.db.q)
    prev = rpa.pa_set_trace(1)
    try:
        _, text = capture_stderr(lambda: _fused(g, w, g.db.k, g.db.v, slots, md))
    finally:
        rpa.pa_set_trace(prev)
    assert "kv_write=in_plan" in text
    assert g.err() & rpa.PA_DERR_SLOT_OOB
    assert torch.equal(g.k_cache.view(torch.int8), h.k_cache.view(torch.int8))
    assert torch.equal(g.v_cache.view(torch.int8), h.v_cache.view(torch.int8))

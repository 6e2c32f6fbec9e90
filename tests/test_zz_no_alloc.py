"""pa_attention_noalloc (the library's static scratch instead of a workspace)
against pa_attention (a caller's workspace) through the C ABI.

Three calls in a row, each smaller than the one before, so each later call
runs over what the earlier ones left in the shared scratch: a shared-prefix
batch (cascade partials, split-K), a mixed batch (work plan, prefill and
decode), and a verify batch (the two-tile decode launch).  Each output must
equal pa_attention's bit for bit and match the oracle to the bf16 tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import ragged_paged_attention_amd as rpa
from tests.gpu_path import DeviceRun, max_abs_err, tol_for
from workloads import config, verify_batch

pytestmark = pytest.mark.gpu


def test_noalloc_matches_pa_attention_on_consecutive_calls():
    cases = [("shared_prefix/4", config(5, scale_down=4)), ("chunked_mixed/8", config(4, scale_down=8)),
             ("spec_verify/8", verify_batch(scale_down=8))]
    prev_need = None
    for name, w in cases:
        need = rpa.pa_attention_workspace_size(w.num_seqs, w.num_tokens, w.num_q_heads, w.num_kv_heads,
                                               w.head_dim, w.max_query_len, w.max_seq_len)
        print(f"[noalloc] {name}: workspace need {need} bytes", flush=True)
        assert 0 < need <= rpa.PA_NOALLOC_SCRATCH_BYTES
        assert prev_need is None or need < prev_need
        prev_need = need
        g = DeviceRun(w).fill_history().write_step_rows()
        db, qsl = g.db, g.meta["query_start_loc"]
        args = (db.q, g.k_cache, g.v_cache, db.block_tables, qsl, db.seq_lens, w.max_query_len, w.max_seq_len,
                w.scale)
        ref_gpu = rpa.pa_attention(*args, workspace=torch.empty(need, dtype=torch.uint8, device="cuda"))
        d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
        out = torch.full_like(db.q, float("nan"))
        rpa.pa_attention_noalloc(*args, out=out, d_err=d_err)
        torch.cuda.synchronize()
        assert int(d_err.item()) == 0
        assert torch.equal(out.view(torch.int16), ref_gpu.view(torch.int16)), name
        _, _, _, ref = oracle.run_step(w)
        err = max_abs_err(out, ref)
        print(f"[noalloc] {name}: max_abs_err={err:.3e}", flush=True)
        assert err <= tol_for(w.dtype)

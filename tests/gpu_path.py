"""Run a Workload through the HIP library (C ABI) on the GPU.

History rows are placed by the library itself (pa_build_metadata on the
history batch, then pa_write_kv), then the step runs as metadata -> write ->
attention.  Nothing here computes any part of the method.
"""
from __future__ import annotations

import os
import tempfile

import numpy as np
import torch

import ragged_paged_attention_amd as rpa
from ragged_paged_attention_amd.step import forward_step
from workloads.device import DeviceBatch

DEVICE = "cuda"


class DeviceRun:
    def __init__(self, w, device=DEVICE):
        self.w = w
        self.db = DeviceBatch(w, device)
        self.d_err = torch.zeros(1, dtype=torch.int32, device=device)
        self.k_cache, self.v_cache = self.db.empty_pool()
        self.hist_meta = None
        self.out = None
        self.meta = None

    def fill_history(self):
        w, db = self.w, self.db
        if w.hist.num_seqs:
            self.hist_meta = rpa.pa_build_metadata(db.hist_query_lens, db.hist_seq_lens, w.hist.num_tokens,
                                                   db.hist_block_tables, w.block_size, w.num_blocks,
                                                   d_err=self.d_err)
            rpa.pa_write_kv(db.hist_k, db.hist_v, self.hist_meta["slot_mapping"], self.k_cache, self.v_cache,
                            d_err=self.d_err)
        return self

    def write_step_rows(self):
        """Metadata and KV write of the step's new rows, no attention (for
        timing attention alone)."""
        w, db = self.w, self.db
        self.meta = rpa.pa_build_metadata(db.query_lens, db.seq_lens, w.num_tokens, db.block_tables, w.block_size,
                                          w.num_blocks, d_err=self.d_err)
        rpa.pa_write_kv(db.k, db.v, self.meta["slot_mapping"], self.k_cache, self.v_cache, d_err=self.d_err)
        torch.cuda.synchronize()
        return self

    def step(self, workspace=None):
        w, db = self.w, self.db
        self.out, self.meta = forward_step(db.q, db.k, db.v, self.k_cache, self.v_cache, db.query_lens,
                                           db.seq_lens, db.block_tables, w.scale, max(1, w.max_query_len),
                                           max(1, w.max_seq_len), workspace=workspace, d_err=self.d_err)
        return self

    def run(self):
        self.fill_history().step()
        torch.cuda.synchronize()
        return self

    def err(self) -> int:
        return int(self.d_err.item())


def tol_for(dtype: str) -> float:
    return 1e-5 if dtype == "f32" else 2e-2


def max_abs_err(gpu_out, ref: np.ndarray) -> float:
    g = gpu_out.detach().to(torch.float64).cpu().numpy()
    return float(np.max(np.abs(g - ref))) if ref.size else 0.0


def capture_stderr(fn):
    """Runs fn() (then waits for the GPU) with file descriptor 2 sent to a
    temporary file; returns fn's result and what was written there (the
    library's trace goes to stderr)."""
    with tempfile.TemporaryFile(mode="w+b") as tmp:
        saved = os.dup(2)
        try:
            os.dup2(tmp.fileno(), 2)
            res = fn()
            torch.cuda.synchronize()
        finally:
            os.dup2(saved, 2)
            os.close(saved)
        tmp.seek(0)
        return res, tmp.read().decode()


def one_stream_output(g, workspace_bytes):
    """The same call as g's last step through pa_attention_noalloc, which
    keeps every launch on the caller's stream (no side stream); returns its
    output."""
    w, db = g.w, g.db
    assert 0 < workspace_bytes <= rpa.PA_NOALLOC_SCRATCH_BYTES
    out = torch.full_like(db.q, float("nan"))
    d_err = torch.zeros(1, dtype=torch.int32, device=db.q.device)
    rpa.pa_attention_noalloc(db.q, g.k_cache, g.v_cache, db.block_tables, g.meta["query_start_loc"], db.seq_lens,
                             max(1, w.max_query_len), max(1, w.max_seq_len), w.scale, out=out, d_err=d_err)
    torch.cuda.synchronize()
    assert int(d_err.item()) == 0
    return out

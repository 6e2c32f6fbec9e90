"""One attention step of continuous batching through the C ABI.

The order follows "vLLM Continuous Batching：从 Forward Shape 理解两个核心参数"
§2.3 (the attention layer first writes the new K/V, then attends) and the
Attention.forward of "vLLM 原理" §3.7: build the flat-batch metadata, then
scatter the new rows by slot_mapping and run ragged paged attention (one
call, pa_write_kv_attention, which lets the library plan the attention while
the write runs).  All of it is library kernels on the current stream;
nothing here synchronises.
"""
from __future__ import annotations

from . import _lib


def forward_step(q, k, v, k_cache, v_cache, query_lens, seq_lens, block_tables, scale: float,
                 max_query_len: int, max_seq_len: int, out=None, workspace=None, d_err=None,
                 meta_out=None):
    """q [T, Hq, D], k/v [T, Hkv, D] new rows; caches [NB, BS, Hkv, D] (updated
    in place); query_lens/seq_lens [S] int32; block_tables [S, MB] int32.
    Returns (out [T, Hq, D], metadata dict)."""
    NB, BS = int(k_cache.shape[0]), int(k_cache.shape[1])
    md = _lib.pa_build_metadata(query_lens, seq_lens, int(q.shape[0]), block_tables, BS, NB,
                                out=meta_out, d_err=d_err)
    out = _lib.pa_write_kv_attention(k, v, md["slot_mapping"], q, k_cache, v_cache, block_tables,
                                     md["query_start_loc"], seq_lens, max_query_len, max_seq_len, scale, out=out,
                                     workspace=workspace, d_err=d_err)
    return out, md

"""Ragged paged attention for continuous batching on MI355X (gfx950).

The computation lives in libpa.so (hand-written HIP kernels behind a C ABI,
declared in include/pa.h); this package is its thin Python binding.
"""
from ._lib import (  # noqa: F401
    LIB_PATH, PA_BF16, PA_DERR_BLOCK_OOB, PA_DERR_OVERFLOW, PA_DERR_QLEN_GT_SEQLEN, PA_DERR_SLOT_OOB,
    PA_DERR_TOKEN_SUM, PA_DERR_HINT, PA_DERR_DUP_SLOT, PA_F16, PA_F32, PA_POLICY_AUTO, PA_POLICY_FAST, PA_POLICY_GENERIC, PAError,
    PA_NOALLOC_SCRATCH_BYTES, declared_symbols, library, pa_attention, pa_attention_noalloc, pa_write_kv_attention, pa_bench_paged_read, pa_bench_stream_read, pa_bench_timing_begin, pa_bench_timing_end, pa_copy_blocks, pa_attention_workspace_size, pa_build_metadata,
    pa_set_kernel_policy, pa_set_trace, pa_set_validation, pa_version, pa_write_kv, status_string,
)

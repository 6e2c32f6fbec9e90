"""CPU oracle (float64 NumPy).  TEST INFRASTRUCTURE ONLY: imported by tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg, never by the product
path."""
from .paged_attention import (  # noqa: F401
    Metadata, OracleInputError, attention, build_metadata, copy_blocks, check_batch, empty_pool, fill_history,
    gather_sequence, kv_head_of, position_of, prefix_offsets, run_step, slot_of,
    softmax_weighted_sum, widen, write_kv,
)

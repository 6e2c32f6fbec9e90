"""Seeded synthetic workloads shared by the tests, the bench and the smoke check.

Nothing here computes any step of ragged paged attention; see generators.py.
"""
from .generators import (  # noqa: F401
    CONFIG_NAMES, DTYPES, Batch, Workload, build_workload, config, decode_variant, f32_to_bf16_bits, prefill_variant,
    permute_sequences, plant_needles, poison_value, random_batch, relabel_blocks, storage_dtype, unshare, verify_batch,
)
from . import accounting  # noqa: F401

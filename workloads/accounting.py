"""Byte and FLOP accounting used to express measured times as rates.

These are workload descriptions (how much data a pass must move, how many
multiply-adds it must do), not part of the attention computation itself.

- KV bytes per token, whole model: two tensors (K and V) per layer, per KV
  head, per head-dim element ("LLM 推理引擎 Continuous Batching 与
  PagedAttention", §1.2, Llama-2-7B example).
- KV cache of a batch: the garbled "22bsdl" of "vLLM 原理" §1.1 read as
  2 (K,V) x 2 (bytes, half precision) x b x s x d x l.
- Bytes of one physical block across all layers ("vLLM 原理" §3.6,
  allocate_kv_cache).
"""
from __future__ import annotations

import numpy as np


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, itemsize: int) -> int:
    return 2 * layers * kv_heads * head_dim * itemsize


def kv_cache_bytes_gpt(batch: int, seq: int, d_model: int, layers: int, itemsize: int = 2) -> int:
    return 2 * itemsize * batch * seq * d_model * layers


def block_bytes(layers: int, block_size: int, kv_heads: int, head_dim: int, itemsize: int) -> int:
    return 2 * layers * block_size * kv_heads * head_dim * itemsize


def itemsize(dtype: str) -> int:
    return 4 if dtype == "f32" else 2


def attention_flops(query_lens, seq_lens, num_q_heads: int, head_dim: int) -> int:
    """Multiply-add FLOPs of QK^T and PV over the (query, key) pairs each query
    is allowed to see: query i of a sequence with query_len q and seq_len L sees
    L - q + i + 1 keys.  2 FLOP per multiply-add, two products."""
    q = np.asarray(query_lens, dtype=np.int64)
    L = np.asarray(seq_lens, dtype=np.int64)
    # sum_{i<q} (L - q + i + 1) = q*(L - q) + q*(q+1)/2
    pairs = int((q * (L - q) + q * (q + 1) // 2).sum())
    return 4 * head_dim * num_q_heads * pairs


def pairs(query_lens, seq_lens) -> int:
    q = np.asarray(query_lens, dtype=np.int64)
    L = np.asarray(seq_lens, dtype=np.int64)
    return int((q * (L - q) + q * (q + 1) // 2).sum())


def kv_read_bytes(seq_lens, num_kv_heads: int, head_dim: int, dtype: str) -> int:
    """Each sequence's K and V rows, read once per KV head."""
    return int(np.asarray(seq_lens, dtype=np.int64).sum()) * 2 * num_kv_heads * head_dim * itemsize(dtype)


def unique_kv_bytes(block_tables, seq_lens, block_size: int, num_kv_heads: int, head_dim: int,
                    dtype: str) -> int:
    """Bytes of distinct (physical block, slot) rows the batch touches."""
    seen = set()
    bt = np.asarray(block_tables)
    for s, L in enumerate(np.asarray(seq_lens)):
        nb = -(-int(L) // block_size)
        for j in range(nb):
            used = min(block_size, int(L) - j * block_size)
            b = int(bt[s, j])
            for o in range(used):
                seen.add((b, o))
    return len(seen) * 2 * num_kv_heads * head_dim * itemsize(dtype)


def unique_kv_bytes_fast(block_tables, seq_lens, block_size: int, num_kv_heads: int, head_dim: int,
                         dtype: str) -> int:
    """Same as unique_kv_bytes, vectorised per block (a block's used prefix)."""
    bt = np.asarray(block_tables)
    used_of = {}
    for s, L in enumerate(np.asarray(seq_lens)):
        nb = -(-int(L) // block_size)
        for j in range(nb):
            used = min(block_size, int(L) - j * block_size)
            b = int(bt[s, j])
            if used > used_of.get(b, 0):
                used_of[b] = used
    return sum(used_of.values()) * 2 * num_kv_heads * head_dim * itemsize(dtype)

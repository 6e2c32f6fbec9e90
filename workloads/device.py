"""Copy a Workload's arrays into torch tensors (host or device).

Pure data movement: 16-bit payloads are reinterpreted (uint16 bits -> the
torch 16-bit float type), nothing is computed.
"""
from __future__ import annotations

import numpy as np


def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]


def tensor(a: np.ndarray, dtype: str, device):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype in ("bf16", "f16") and a.dtype == np.uint16:
        t = t.view(torch.int16).view(torch_dtype(dtype))
    return t.to(device)


def ints(a: np.ndarray, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def to_numpy_bits(t) -> np.ndarray:
    """Tensor -> numpy in the generator's storage format (uint16 bits for
    16-bit floats)."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


class DeviceBatch:
    """Device copies of one Workload: the step's inputs and the history batch."""

    def __init__(self, w, device="cuda"):
        self.w = w
        self.device = device
        self.q = tensor(w.q, w.dtype, device)
        self.k = tensor(w.step.k, w.dtype, device)
        self.v = tensor(w.step.v, w.dtype, device)
        self.query_lens = ints(w.step.query_lens, device)
        self.seq_lens = ints(w.step.seq_lens, device)
        self.block_tables = ints(w.step.block_tables, device)
        self.hist_query_lens = ints(w.hist.query_lens, device)
        self.hist_seq_lens = ints(w.hist.seq_lens, device)
        self.hist_block_tables = ints(w.hist.block_tables, device)
        self.hist_k = tensor(w.hist.k, w.dtype, device)
        self.hist_v = tensor(w.hist.v, w.dtype, device)

    def empty_pool(self):
        """Two caches [NB, BS, Hkv, D] filled with the workload's fill value
        (NaN poison in correctness runs, zero otherwise)."""
        import torch
        w = self.w
        fill = float("nan") if w.poison else 0.0
        kc = torch.full(w.pool_shape(), fill, dtype=torch_dtype(w.dtype), device=self.device)
        vc = torch.full(w.pool_shape(), fill, dtype=torch_dtype(w.dtype), device=self.device)
        return kc, vc

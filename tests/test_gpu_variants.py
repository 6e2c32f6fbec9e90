"""GPU parity of the head-dim and block-size variants of the fast decode path.

The method is the same at every head dim and block size: "LLM 推理引擎
Continuous Batching 与 PagedAttention" §3.4 weighs block sizes 1/8/16/32 as a
trade-off between waste and lookup cost, "vLLM 原理" §3.2 uses 256, and the
head dim only sets the length of the dot products.  So the plain oracle is
the reference for all of them.  The decode and prefill kernels take head_dim
64, 128 and 256 and a block size that is a multiple of 16 or divides 16 (each
lane, or each DMA row, then finds its own token's block).
"""
import numpy as np
import pytest
import torch

import oracle
import ragged_paged_attention_amd as rpa
from tests.gpu_path import DeviceRun, max_abs_err, tol_for
from workloads import plant_needles
from workloads.generators import build_workload

pytestmark = pytest.mark.gpu


def _batch(Hq, Hkv, D, bs, ql, sl, seed, dtype="bf16"):
    rng = np.random.default_rng(seed)
    counts = [-(-L // bs) for L in sl]
    NB = int(sum(counts)) + 16
    ids = rng.permutation(NB)
    tables, o = [], 0
    for c in counts:
        tables.append([int(x) for x in ids[o:o + c]])
        o += c
    return build_workload(f"variant_d{D}_bs{bs}", dtype, Hq, Hkv, D, bs, NB, list(ql), list(sl), tables, seed)


# decode rows over contexts long enough for several split-K parts, one short
# context, and (mixed) verify rows and a prefill chunk in the same call
SHAPES = {
    "decode": dict(ql=[1, 1, 1, 1, 1], sl=[3000, 17, 1700, 800, 2049]),
    "mixed": dict(ql=[1, 3, 1, 200, 7, 1, 517], sl=[2500, 900, 40, 1300, 2000, 1, 517]),
}


@pytest.mark.parametrize("shape", sorted(SHAPES))
@pytest.mark.parametrize("D,bs", [(64, 16), (256, 16), (128, 8), (64, 8), (256, 8), (128, 4), (64, 32),
                                  (128, 256)])
@pytest.mark.parametrize("Hq,Hkv", [(16, 4), (8, 8)])
def test_variant_matches_oracle(shape, D, bs, Hq, Hkv):
    c = SHAPES[shape]
    w = _batch(Hq, Hkv, D, bs, c["ql"], c["sl"], seed=D + bs + Hq)
    print(f"[variant] {shape} D={D} bs={bs} Hq={Hq} Hkv={Hkv}", flush=True)
    rpa.pa_bench_timing_begin()
    g = DeviceRun(w).run()
    t = rpa.pa_bench_timing_end()
    _, _, _, ref = oracle.run_step(w)
    assert g.err() == 0
    err = max_abs_err(g.out, ref)
    print(f"[variant] max_abs_err={err:.3e} kernels={sorted(t)}", flush=True)
    assert err <= tol_for(w.dtype)
    assert "decode_kernel" in t          # the fast decode path ran
    if shape == "mixed":
        assert "prefill_kernel" in t     # and the MFMA prefill kernel


@pytest.mark.parametrize("D,bs", [(64, 8), (256, 16)])
def test_variant_fp16(D, bs):
    w = _batch(32, 8, D, bs, [1, 1, 2, 1], [1500, 3100, 600, 33], seed=D, dtype="f16")
    g = DeviceRun(w).run()
    _, _, _, ref = oracle.run_step(w)
    assert g.err() == 0
    assert max_abs_err(g.out, ref) <= tol_for("f16")


def test_variant_shared_prefix_bs8():
    """Sequences sharing their leading blocks at block size 8, head_dim 128:
    the shared-prefix (cascade) path reads the prefix through the prefill
    kernel's per-row block lookup."""
    bs, prefix = 8, 2048
    rng = np.random.default_rng(3)
    n = 6
    sl = [prefix + int(x) for x in rng.integers(1, 300, n)] + [2100]
    ql = [1] * n + [1]
    need = prefix // bs + sum(-(-L // bs) - prefix // bs for L in sl[:n]) + -(-sl[n] // bs)
    NB = need + 16
    ids = iter(int(x) for x in rng.permutation(NB))
    pre = [next(ids) for _ in range(prefix // bs)]
    tables = [pre + [next(ids) for _ in range(-(-L // bs) - prefix // bs)] for L in sl[:n]]
    tables.append([next(ids) for _ in range(-(-sl[n] // bs))])
    w = build_workload("shared_bs8", "bf16", 32, 4, 128, bs, NB, ql, sl, tables, 3, rng,
                       shared=[(list(range(n)), prefix)])
    g = DeviceRun(w).run()
    _, _, _, ref = oracle.run_step(w)
    assert g.err() == 0
    assert max_abs_err(g.out, ref) <= tol_for("bf16")


@pytest.mark.parametrize("D,bs", [(128, 4), (128, 8), (64, 1), (128, 256)])
def test_variant_needles(D, bs):
    """One dominant key per (sequence, KV head) at block sizes below 16 (each
    lane or DMA row looks its block up itself, and the decode kernel's id
    window moves every 64 blocks) and at 256: a wrong block shows as an O(1)
    error."""
    c = SHAPES["mixed"]
    w = plant_needles(_batch(16, 4, D, bs, c["ql"], c["sl"], seed=D + bs), seed=bs)
    g = DeviceRun(w).run()
    _, _, _, ref = oracle.run_step(w)
    assert g.err() == 0
    err = max_abs_err(g.out, ref)
    print(f"[variant needles] D={D} bs={bs} max_abs_err={err:.3e}", flush=True)
    assert err <= tol_for(w.dtype)

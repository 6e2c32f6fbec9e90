"""GPU parity of pa_copy_blocks: whole-block copies for copy-on-write and swap.

Pools are compared bit for bit with the oracle's copy_blocks; the parallel
sampling walk-through of the vLLM principles page (§2.1: branches share the
prompt's blocks, the first write into a shared block copies it) runs end to
end through the library and is compared with the oracle; a swap out to a
pinned host pool and back in at other block ids leaves attention unchanged
bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import ragged_paged_attention_amd as rpa
from ragged_paged_attention_amd.step import forward_step
from tests.gpu_path import DeviceRun, max_abs_err, tol_for
from workloads import random_batch
from workloads.device import tensor, to_numpy_bits, torch_dtype
from workloads.generators import _pad_tables, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

BLOCK_OOB = 4


def _random_bits(rng, shape, dtype):
    if dtype == "f32":
        return rng.integers(0, 2**32, shape, dtype=np.uint32).view(np.float32)
    return rng.integers(0, 2**16, shape, dtype=np.uint16)


def _bits(a):
    a = np.asarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


def _values(rng, shape, dtype):
    x = rng.standard_normal(shape).astype(np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x.astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("dtype,bs,Hkv,D", [("bf16", 16, 8, 128), ("f32", 8, 2, 64), ("f16", 1, 1, 8),
                                            ("bf16", 64, 1, 256)])
def test_copy_blocks_bit_exact(dtype, bs, Hkv, D):
    rng = np.random.default_rng(bs * 7 + D)
    NB = 97
    k0, v0 = _random_bits(rng, (NB, bs, Hkv, D), dtype), _random_bits(rng, (NB, bs, Hkv, D), dtype)
    perm = rng.permutation(NB)
    srcs = rng.choice(perm[:20], 40)          # one source may feed several destinations (a fork)
    dsts = perm[20:60]
    pairs = np.stack([srcs, dsts], axis=1).astype(np.int32)
    print(f"[blocks] copy dtype={dtype} bs={bs} Hkv={Hkv} D={D} pairs={len(pairs)}", flush=True)
    kc, vc = tensor(k0, dtype, "cuda"), tensor(v0, dtype, "cuda")
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    rpa.pa_copy_blocks(kc, vc, kc, vc, torch.from_numpy(pairs).cuda(), d_err=d_err)
    torch.cuda.synchronize()
    ek, ev = k0.copy(), v0.copy()
    oracle.copy_blocks(ek, ev, ek, ev, pairs)
    assert int(d_err.item()) == 0
    assert np.array_equal(_bits(to_numpy_bits(kc)), _bits(ek))
    assert np.array_equal(_bits(to_numpy_bits(vc)), _bits(ev))


def test_copy_blocks_out_of_range_pairs_are_skipped_and_flagged():
    rng = np.random.default_rng(5)
    NB = 12
    k0, v0 = _random_bits(rng, (NB, 16, 2, 128), "bf16"), _random_bits(rng, (NB, 16, 2, 128), "bf16")
    kc, vc = tensor(k0, "bf16", "cuda"), tensor(v0, "bf16", "cuda")
    pairs = torch.tensor([[0, 5], [NB, 3], [2, -1], [4, 6], [-3, 7]], dtype=torch.int32, device="cuda")
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    rpa.pa_copy_blocks(kc, vc, kc, vc, pairs, d_err=d_err)
    torch.cuda.synchronize()
    ek, ev = k0.copy(), v0.copy()
    oracle.copy_blocks(ek, ev, ek, ev, [[0, 5], [4, 6]])
    assert int(d_err.item()) & BLOCK_OOB
    assert np.array_equal(to_numpy_bits(kc), ek) and np.array_equal(to_numpy_bits(vc), ev)


def test_copy_blocks_rejects_bad_arguments():
    lib = rpa.library()
    kc = torch.zeros(4, 16, 2, 128, dtype=torch.bfloat16, device="cuda")
    pairs = torch.zeros(1, 2, dtype=torch.int32, device="cuda")
    p = kc.data_ptr()
    assert lib.pa_copy_blocks(p, p, p, p, 4, 4, pairs.data_ptr(), 1, 8200, None, None) == 2   # not 16-aligned
    assert lib.pa_copy_blocks(p, p, p, p, 0, 4, pairs.data_ptr(), 1, 8192, None, None) == 2
    assert lib.pa_copy_blocks(p, None, p, p, 4, 4, pairs.data_ptr(), 1, 8192, None, None) == 1
    assert lib.pa_copy_blocks(p, p, p, p, 4, 4, None, 0, 8192, None, None) == 0           # nothing to do


@pytest.mark.parametrize("prompt_len", [100, 96], ids=["tail_shared", "block_aligned"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_parallel_sampling_copy_on_write(prompt_len, dtype):
    """Four branches share a prompt's blocks.  When the prompt ends inside a
    block, every branch but the last copies that block before writing its
    first token there; the last writes in place.  When it ends on a block
    boundary each branch just gets a fresh block and nothing is copied."""
    rng = np.random.default_rng(prompt_len)
    Hq, Hkv, D, bs, NB, n_br = 32, 8, 128, 16, 64, 4
    n_blk = -(-prompt_len // bs)
    ids = [int(x) for x in rng.permutation(NB)]
    shared, spare = ids[:n_blk], ids[n_blk:]
    pk, pv = _values(rng, (prompt_len, Hkv, D), dtype), _values(rng, (prompt_len, Hkv, D), dtype)
    print(f"[blocks] cow dtype={dtype} prompt={prompt_len}", flush=True)

    # prompt written once, through the shared table
    shared_bt = _pad_tables([shared])
    fill = np.float32(np.nan) if dtype == "f32" else np.uint16(0x7FC0)
    ek = oracle.empty_pool((NB, bs, Hkv, D), dtype, fill)
    ev = oracle.empty_pool((NB, bs, Hkv, D), dtype, fill)
    md = oracle.build_metadata([prompt_len], [prompt_len], prompt_len, shared_bt, bs, NB)
    oracle.write_kv(pk, pv, md.slot_mapping, ek, ev)
    kc = torch.full((NB, bs, Hkv, D), float("nan"), dtype=torch_dtype(dtype), device="cuda")
    vc = torch.full_like(kc, float("nan"))
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    gmd = rpa.pa_build_metadata(torch.tensor([prompt_len], dtype=torch.int32, device="cuda"),
                                torch.tensor([prompt_len], dtype=torch.int32, device="cuda"), prompt_len,
                                torch.from_numpy(shared_bt).cuda(), bs, NB, d_err=d_err)
    rpa.pa_write_kv(tensor(pk, dtype, "cuda"), tensor(pv, dtype, "cuda"), gmd["slot_mapping"], kc, vc, d_err=d_err)

    # branch tables after the first decode step's allocation / copy-on-write
    tables, pairs = [], []
    if prompt_len % bs:
        for b in range(n_br):
            if b < n_br - 1:
                nb = spare.pop()
                pairs.append([shared[-1], nb])
                tables.append(shared[:-1] + [nb])
            else:
                tables.append(list(shared))
    else:
        tables = [shared + [spare.pop()] for _ in range(n_br)]
    pairs = np.array(pairs, dtype=np.int32).reshape(-1, 2)
    oracle.copy_blocks(ek, ev, ek, ev, pairs)
    rpa.pa_copy_blocks(kc, vc, kc, vc, torch.from_numpy(pairs).cuda(), d_err=d_err)

    # one decode row per branch
    bt = _pad_tables(tables)
    ql, sl = [1] * n_br, [prompt_len + 1] * n_br
    q = _values(rng, (n_br, Hq, D), dtype)
    nk, nv = _values(rng, (n_br, Hkv, D), dtype), _values(rng, (n_br, Hkv, D), dtype)
    md = oracle.build_metadata(ql, sl, n_br, bt, bs, NB)
    oracle.write_kv(nk, nv, md.slot_mapping, ek, ev)
    ref = oracle.attention(q, ek, ev, bt, md.query_start_loc, np.array(sl), Hkv, D ** -0.5, dtype)
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device="cuda")
    out, _ = forward_step(tensor(q, dtype, "cuda"), tensor(nk, dtype, "cuda"), tensor(nv, dtype, "cuda"), kc, vc,
                          i32(ql), i32(sl), torch.from_numpy(bt).cuda(), D ** -0.5, 1, prompt_len + 1, d_err=d_err)
    torch.cuda.synchronize()
    assert int(d_err.item()) == 0
    assert np.array_equal(_bits(to_numpy_bits(kc)), _bits(ek)) and np.array_equal(_bits(to_numpy_bits(vc)), _bits(ev))
    assert max_abs_err(out, ref) <= tol_for(dtype)
    assert np.abs(ref[0] - ref[-1]).max() > 1e-3          # the branches really see different tokens


def test_swap_out_and_in_through_pinned_host_memory():
    """Swap a few sequences' blocks out to a pinned host pool, poison their
    device blocks, swap them back in at other ids and repoint the tables:
    attention is bit-identical to the run before the swap."""
    w = random_batch(404, S=6, Hq=8, Hkv=2, D=128, bs=16, dtype="bf16", max_ctx=300, max_q=40, extra_blocks=60)
    g = DeviceRun(w).run()
    out0 = g.out.clone()
    bt = w.step.block_tables.copy()
    used = set(int(x) for x in bt[bt >= 0])
    spare = [b for b in range(w.num_blocks) if b not in used]
    moved = [1, 4]
    blocks = sorted({int(x) for s in moved for x in bt[s][bt[s] >= 0]} -
                    {int(x) for s in range(w.num_seqs) if s not in moved for x in bt[s][bt[s] >= 0]})
    assert len(blocks) <= len(spare) and len(blocks) > 0
    print(f"[blocks] swap {len(blocks)} blocks", flush=True)
    host_k = torch.empty((len(blocks),) + tuple(g.k_cache.shape[1:]), dtype=g.k_cache.dtype, pin_memory=True)
    host_v = torch.empty_like(host_k, pin_memory=True)
    out_pairs = torch.tensor([[b, i] for i, b in enumerate(blocks)], dtype=torch.int32, device="cuda")
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    rpa.pa_copy_blocks(g.k_cache, g.v_cache, host_k, host_v, out_pairs, d_err=d_err)
    torch.cuda.synchronize()
    assert torch.equal(host_k.view(torch.int16), g.k_cache[blocks].cpu().view(torch.int16))
    assert torch.equal(host_v.view(torch.int16), g.v_cache[blocks].cpu().view(torch.int16))
    g.k_cache[blocks] = float("nan")
    g.v_cache[blocks] = float("nan")
    new_ids = spare[:len(blocks)]
    in_pairs = torch.tensor([[i, n] for i, n in enumerate(new_ids)], dtype=torch.int32, device="cuda")
    rpa.pa_copy_blocks(host_k, host_v, g.k_cache, g.v_cache, in_pairs, d_err=d_err)
    remap = dict(zip(blocks, new_ids))
    bt2 = bt.copy()
    for s in moved:
        bt2[s] = [remap.get(int(x), int(x)) if x >= 0 else -1 for x in bt[s]]
    out1 = rpa.pa_attention(g.db.q, g.k_cache, g.v_cache, torch.from_numpy(bt2).cuda(), g.meta["query_start_loc"],
                            g.db.seq_lens, max(1, w.max_query_len), max(1, w.max_seq_len), w.scale, d_err=d_err)
    torch.cuda.synchronize()
    assert int(d_err.item()) == 0
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))

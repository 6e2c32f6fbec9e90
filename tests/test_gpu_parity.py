"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Metadata and the KV scatter must match bit for bit; attention must match to
max-abs-error 1e-5 for fp32 inputs and 2e-2 for bf16/f16 inputs (fp32
accumulation), on the same seeded inputs.  Unwritten pool slots hold NaN, so
any read outside a sequence's visible rows shows up as NaN.
"""

import numpy as np
import pytest
import torch

import oracle
import ragged_paged_attention_amd as rpa
from workloads import config, decode_variant, random_batch, relabel_blocks, unshare
from workloads.device import to_numpy_bits

from tests.gpu_path import DeviceRun, capture_stderr, max_abs_err, one_stream_output, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _policy_reset():
    prev = rpa.pa_set_kernel_policy(rpa.PA_POLICY_AUTO)
    yield
    rpa.pa_set_kernel_policy(prev)


def _meta_equal(gpu_md, ref: oracle.Metadata, T):
    assert gpu_md["query_start_loc"].cpu().numpy().tolist() == ref.query_start_loc.tolist()
    assert gpu_md["seq_start_loc"].cpu().numpy().tolist() == ref.seq_start_loc.tolist()
    assert gpu_md["positions"].cpu().numpy().tolist() == ref.positions.tolist()
    assert gpu_md["token_to_seq"].cpu().numpy().tolist() == ref.token_to_seq.tolist()
    assert gpu_md["slot_mapping"].cpu().numpy().tolist() == ref.slot_mapping.tolist()
    assert gpu_md["stats"].cpu().numpy().tolist() == ref.stats.tolist()


def _bits(a):
    a = np.asarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


SMALL = [("tiny_mixed", lambda: config(1))] + \
    [(f"random{s}", (lambda s=s: random_batch(s, S=5, Hq=4, Hkv=2, D=16, bs=4, max_ctx=40, max_q=9)))
     for s in range(3)] + \
    [(f"cfg{n}_small", (lambda n=n: config(n, scale_down=32))) for n in (2, 3, 4, 5)]


@pytest.mark.parametrize("name,make", SMALL, ids=[n for n, _ in SMALL])
def test_metadata_and_scatter_bitexact(name, make):
    w = make()
    print(f"[case] {name} {w.summary()}", flush=True)
    g = DeviceRun(w).run()
    md, kc, vc, _ = oracle.run_step(w, rows=[0])
    _meta_equal(g.meta, md, w.num_tokens)
    assert np.array_equal(_bits(to_numpy_bits(g.k_cache)), _bits(kc)), "k_cache differs"
    assert np.array_equal(_bits(to_numpy_bits(g.v_cache)), _bits(vc)), "v_cache differs"
    assert g.err() == 0


def test_tiny_mixed_fp32_attention():
    """The forward-shape walkthrough batch (B, C decode; A prefills 5)."""
    w = config(1)
    g = DeviceRun(w).run()
    _, _, _, ref = oracle.run_step(w)
    err = max_abs_err(g.out, ref)
    print(f"[tiny_mixed] max_abs_err={err:.3e}", flush=True)
    assert err <= 1e-5
    # a0 sees only itself: the output is its own V row, exactly
    G = w.num_q_heads // w.num_kv_heads
    v64 = oracle.widen(w.step.v[2], w.dtype)
    out = g.out.double().cpu().numpy()
    for h in range(w.num_q_heads):
        assert np.array_equal(out[2, h], v64[h // G])
    assert g.err() == 0


SWEEP = []
for seed in range(6):
    for dtype in ("f32", "bf16", "f16"):
        for (Hq, Hkv, D, bs) in ((4, 2, 16, 4), (8, 1, 64, 16), (4, 4, 128, 16), (8, 2, 128, 32), (2, 1, 32, 1)):
            SWEEP.append(dict(seed=seed * 7 + 100, dtype=dtype, Hq=Hq, Hkv=Hkv, D=D, bs=bs))


@pytest.mark.parametrize("policy", ["auto", "generic"])
@pytest.mark.parametrize("case", SWEEP, ids=lambda c: f"s{c['seed']}-{c['dtype']}-{c['Hq']}x{c['Hkv']}-D{c['D']}-bs{c['bs']}")
def test_random_sweep(case, policy):
    rpa.pa_set_kernel_policy(rpa.PA_POLICY_GENERIC if policy == "generic" else rpa.PA_POLICY_AUTO)
    w = random_batch(case["seed"], S=6, Hq=case["Hq"], Hkv=case["Hkv"], D=case["D"], bs=case["bs"],
                     dtype=case["dtype"], max_ctx=70, max_q=40, decode_frac=0.5)
    g = DeviceRun(w).run()
    _, _, _, ref = oracle.run_step(w)
    err = max_abs_err(g.out, ref)
    assert err <= tol_for(w.dtype), f"max_abs_err {err}"
    assert g.err() == 0


@pytest.mark.parametrize("policy", ["auto", "generic"])
@pytest.mark.parametrize("n", [2, 3, 4, 5])
def test_scaled_configs(n, policy):
    """Same structure and head shapes as the full workloads, lengths / 16:
    several tiles per sequence, ragged tails, every row checked."""
    rpa.pa_set_kernel_policy(rpa.PA_POLICY_GENERIC if policy == "generic" else rpa.PA_POLICY_AUTO)
    w = config(n, scale_down=16)
    print(f"[case] scaled config {n} {w.summary()}", flush=True)
    g = DeviceRun(w).run()
    _, _, _, ref = oracle.run_step(w)
    err = max_abs_err(g.out, ref)
    print(f"[scaled cfg{n} {policy}] max_abs_err={err:.3e}", flush=True)
    assert err <= tol_for(w.dtype)
    assert g.err() == 0


def test_placement_invariance_bitexact():
    """Relabelled physical blocks give bit-identical outputs."""
    w = config(4, scale_down=16)
    perm = np.random.default_rng(5).permutation(w.num_blocks)
    a = DeviceRun(w).run().out
    b = DeviceRun(relabel_blocks(w, perm)).run().out
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_sharing_invariance_bitexact():
    """Shared prefix blocks and private copies give bit-identical outputs."""
    w = config(5, scale_down=16)
    w.num_blocks += int((w.step.block_tables >= 0).sum())
    used = set(int(b) for b in w.step.block_tables.ravel() if b >= 0)
    u = unshare(w, [b for b in range(w.num_blocks) if b not in used])
    a = DeviceRun(w).run().out
    b = DeviceRun(u).run().out
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("n", [4, 5])
def test_isolation_from_other_sequences_blocks_bitexact(n):
    """Overwriting every cache block that the even-numbered sequences' tables
    do not map (the odd sequences' blocks and the unused pool) leaves the
    even sequences' outputs bit-identical ("vLLM Continuous Batching：从
    Forward Shape 理解两个核心参数" §2.3补充: a sequence reads only through its
    own block table), while the odd sequences' outputs change."""
    w = config(n, scale_down=8)
    print(f"[case] isolation cfg{n} {w.summary()}", flush=True)
    g = DeviceRun(w).run()
    before = g.out.clone()
    bt = w.step.block_tables
    keep = sorted(set(int(b) for s in range(0, w.num_seqs, 2) for b in bt[s] if b >= 0))
    mask = torch.ones(w.num_blocks, dtype=torch.bool)
    mask[keep] = False
    other = mask.nonzero().flatten().to("cuda")
    gen = torch.Generator(device="cuda").manual_seed(n)
    for cache in (g.k_cache, g.v_cache):
        noise = torch.randn((len(other),) + tuple(cache.shape[1:]), generator=gen, device="cuda") * 3
        cache[other] = noise.to(cache.dtype)
    g.step()  # metadata, this step's K/V write, attention
    torch.cuda.synchronize()
    assert g.err() == 0
    qsl = w.new_row_offsets()
    even = torch.cat([torch.arange(int(qsl[s]), int(qsl[s + 1])) for s in range(0, w.num_seqs, 2)]).to("cuda")
    odd = torch.cat([torch.arange(int(qsl[s]), int(qsl[s + 1])) for s in range(1, w.num_seqs, 2)]).to("cuda")
    assert torch.equal(before[even].view(torch.int16), g.out[even].view(torch.int16))
    assert not torch.equal(before[odd].view(torch.int16), g.out[odd].view(torch.int16))


def test_mixed_batch_decode_beside_prefill():
    """A large mixed batch (128 sequences, 4096 tokens) runs its decode
    launches beside the prefill kernel on the library's side stream; every
    decode row and the last rows of every chunk match the oracle, and two
    calls give the same bits."""
    w = config(4, scale_down=2)
    print(f"[case] beside {w.summary()}", flush=True)
    prev = rpa.pa_set_trace(1)
    try:
        g, text = capture_stderr(lambda: DeviceRun(w).run())
    finally:
        rpa.pa_set_trace(prev)
    assert "decode_beside_prefill=1" in text
    assert g.err() == 0
    ql = w.step.query_lens
    offs = w.new_row_offsets()
    rows = [int(offs[s]) for s in range(w.num_seqs) if ql[s] == 1]
    rows += [int(offs[s + 1]) - 1 for s in range(w.num_seqs) if ql[s] > 1]
    _, _, _, ref = oracle.run_step(w, rows=rows)
    err = max_abs_err(g.out[torch.tensor(rows, device="cuda")], ref)
    print(f"[beside] rows {len(rows)} max_abs_err={err:.3e}", flush=True)
    assert err <= tol_for(w.dtype)
    first = g.out.clone()
    g.step()
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), g.out.view(torch.int16))


@pytest.mark.parametrize("dtype,bs", [("bf16", 16), ("f16", 16), ("bf16", 32)])
def test_mixed_batch_beside_equals_one_stream(dtype, bs):
    """The CU split changes where the kernels run, not what they compute: a
    mixed batch of 64 sequences (60 decodes beside 4 chunks) through
    pa_attention (decode launches on the side stream, prefill at one
    workgroup per CU) gives the same bits as through pa_attention_noalloc
    (every launch on the caller's stream, prefill at two workgroups per CU),
    on every row; all rows match the oracle."""
    w = config(4, scale_down=4, dtype=dtype, block_size=bs)
    print(f"[case] beside vs one stream {dtype} bs {bs}: {w.summary()}", flush=True)
    need = rpa.pa_attention_workspace_size(w.num_seqs, w.num_tokens, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                           w.max_query_len, w.max_seq_len)
    prev = rpa.pa_set_trace(1)
    try:
        g, text = capture_stderr(lambda: DeviceRun(w).run())
    finally:
        rpa.pa_set_trace(prev)
    assert "decode_beside_prefill=1" in text
    assert g.err() == 0
    serial = one_stream_output(g, need)
    assert torch.equal(g.out.view(torch.int16), serial.view(torch.int16))
    _, _, _, ref = oracle.run_step(w)
    err = max_abs_err(g.out, ref)
    print(f"[beside] {dtype} bs {bs}: max_abs_err={err:.3e}", flush=True)
    assert err <= tol_for(w.dtype)


def test_deterministic():
    w = config(4, scale_down=8)
    g = DeviceRun(w).run()
    first = g.out.clone()
    g.step()
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), g.out.view(torch.int16))


def test_error_flags_from_host_forced_data():
    """Invalid metadata is flagged on the device and no access leaves the
    buffers (the pool is NaN-poisoned; outputs of flagged rows are zero)."""
    w = config(1)
    g = DeviceRun(w).run()          # history and this step's rows are in the pool
    dev = g.db
    # query_len > seq_len for sequence 0
    bad_sl = dev.seq_lens.clone()
    bad_sl[0] = 0
    qsl = torch.tensor([0, 1, 2, 7], dtype=torch.int32, device="cuda")
    d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    rpa.pa_attention(dev.q, g.k_cache, g.v_cache, dev.block_tables, qsl, bad_sl, 5, 8, w.scale, d_err=d_err)
    torch.cuda.synchronize()
    assert int(d_err.item()) & rpa.PA_DERR_QLEN_GT_SEQLEN
    # a -1 block inside the used range
    bad_bt = dev.block_tables.clone()
    bad_bt[0, 0] = -1
    d_err.zero_()
    md = rpa.pa_build_metadata(dev.query_lens, dev.seq_lens, w.num_tokens, bad_bt, w.block_size, w.num_blocks,
                               d_err=d_err)
    out = rpa.pa_attention(dev.q, g.k_cache, g.v_cache, bad_bt, md["query_start_loc"], dev.seq_lens, 5, 8,
                           w.scale, d_err=d_err)
    torch.cuda.synchronize()
    assert int(d_err.item()) & rpa.PA_DERR_BLOCK_OOB
    assert torch.isfinite(out[1:]).all()
    # sum(query_lens) != num_tokens
    d_err.zero_()
    rpa.pa_build_metadata(dev.query_lens, dev.seq_lens, w.num_tokens + 1, dev.block_tables, w.block_size,
                          w.num_blocks, d_err=d_err)
    torch.cuda.synchronize()
    assert int(d_err.item()) & rpa.PA_DERR_TOKEN_SUM
    # slot beyond the pool
    d_err.zero_()
    slots = torch.full((w.num_tokens,), -1, dtype=torch.int32, device="cuda")
    slots[0] = w.num_blocks * w.block_size
    before = g.k_cache.clone()
    rpa.pa_write_kv(dev.k, dev.v, slots, g.k_cache, g.v_cache, d_err=d_err)
    torch.cuda.synchronize()
    assert int(d_err.item()) & rpa.PA_DERR_SLOT_OOB
    assert torch.equal(before.view(torch.int32), g.k_cache.view(torch.int32))


def test_workspace_too_small_is_rejected():
    """A mixed batch needs workspace (the work plan and split-K partials); one
    byte less is refused with PA_ERR_WORKSPACE and nothing runs."""
    w = config(4, scale_down=8)
    g = DeviceRun(w).fill_history()
    need = rpa.pa_attention_workspace_size(w.num_seqs, w.num_tokens, w.num_q_heads, w.num_kv_heads,
                                           w.head_dim, w.max_query_len, w.max_seq_len)
    assert need > 0
    md = rpa.pa_build_metadata(g.db.query_lens, g.db.seq_lens, w.num_tokens, g.db.block_tables, w.block_size,
                               w.num_blocks)
    small = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    out = torch.full_like(g.db.q, 3.0)
    with pytest.raises(rpa.PAError) as e:
        rpa.pa_attention(g.db.q, g.k_cache, g.v_cache, g.db.block_tables, md["query_start_loc"], g.db.seq_lens,
                         w.max_query_len, w.max_seq_len, w.scale, out=out, workspace=small)
    assert e.value.status == 5
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())


class _Scaled:
    """A workload seen with another softmax scale (same data)."""

    def __init__(self, w, scale):
        self._w, self.scale = w, scale

    def __getattr__(self, name):
        return getattr(self._w, name)


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.7])
@pytest.mark.parametrize("n", [4, 5])
def test_any_finite_scale(n, scale):
    """Attention is defined for any finite softmax scale.  A mixed batch (decode
    rows and prefill chunks) and a shared-prefix batch, compared with the
    oracle at scale 0 (every visible key weighs the same), a negative scale
    and a large positive one; scale <= 0 runs on the generic kernel."""
    w = _Scaled(config(n, scale_down=16), scale)
    g = DeviceRun(w).run()
    _, _, _, ref = oracle.run_step(w)
    err = max_abs_err(g.out, ref)
    print(f"[scale {scale}] config {n} max_abs_err={err:.3e}", flush=True)
    assert g.err() == 0
    assert err <= tol_for(w.dtype)


def test_duplicate_slots_flagged_with_validation():
    """Two rows of one write with the same slot are invalid input (the
    copy-on-write rule of "vLLM 原理" §2.1 keeps writers apart).  With
    validation on, pa_write_kv flags PA_DERR_DUP_SLOT; a write with distinct
    slots (a whole mixed step) is not flagged; with validation off nothing is
    checked."""
    w = config(4, scale_down=8)
    g = DeviceRun(w)
    prev = rpa.pa_set_validation(1)
    try:
        g.fill_history()
        g.step()
        torch.cuda.synchronize()
        assert g.err() == 0                       # history and step writes: every slot distinct
        slots = g.meta["slot_mapping"].clone()
        for a, b in ((5, 700), (w.num_tokens - 1, 0), (300, 301)):
            bad = slots.clone()
            bad[b] = bad[a]
            d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
            rpa.pa_write_kv(g.db.k, g.db.v, bad, g.k_cache, g.v_cache, d_err=d_err)
            torch.cuda.synchronize()
            assert int(d_err.item()) == rpa.PA_DERR_DUP_SLOT, (a, b)
        bad = slots.clone()
        bad[7] = -1
        bad[9] = -1                               # skipped rows are not duplicates
        d_err = torch.zeros(1, dtype=torch.int32, device="cuda")
        rpa.pa_write_kv(g.db.k, g.db.v, bad, g.k_cache, g.v_cache, d_err=d_err)
        torch.cuda.synchronize()
        assert int(d_err.item()) == 0
        rpa.pa_set_validation(0)
        bad = slots.clone()
        bad[1] = bad[0]
        d_err.zero_()
        rpa.pa_write_kv(g.db.k, g.db.v, bad, g.k_cache, g.v_cache, d_err=d_err)
        torch.cuda.synchronize()
        assert int(d_err.item()) == 0
    finally:
        rpa.pa_set_validation(prev)


def test_plan_doubles_the_parts_of_a_list_between_one_and_two_waves():
    """40 decode sequences of 2101 tokens at 32 KV heads: with a plan (the
    contexts are long enough for shared-prefix detection) the one-tile list
    would hold 120 entries of 768-token parts against 96 that one wave of
    the launch holds (3 waves per SIMD x 1024 SIMDs / 32 heads), so the plan
    cuts 1536-token parts instead (80 entries, the trace says so); every row
    matches the oracle."""
    w = decode_variant(128, 16, S=40, hist_len=2100)
    print(f"[case] doubled parts {w.summary()}", flush=True)
    prev = rpa.pa_set_trace(1)
    try:
        g, text = capture_stderr(lambda: DeviceRun(w).run())
    finally:
        rpa.pa_set_trace(prev)
    assert "decode items 80 one-tile, 0 two-tile (parts of at most 1536, 768 tokens)" in text
    assert g.err() == 0
    _, _, _, ref = oracle.run_step(w)
    err = max_abs_err(g.out, ref)
    print(f"[doubled parts] max_abs_err={err:.3e}", flush=True)
    assert err <= tol_for(w.dtype)

"""Throughput of one continuous-batching attention step on one MI355X.

A step is the whole hot path over one batch, in the order the pages give
("vLLM Continuous Batching：从 Forward Shape 理解两个核心参数" §2.3): build the
flat-batch metadata, scatter the new K/V by slot_mapping, then ragged paged
attention.  All three run as libpa kernels (C ABI) on the current stream.

Default workload: the chunked-prefill mixed batch (240 decode sequences with
log-uniform contexts 128..8192 plus 16 prefill chunks of 497 tokens with
0..4096 earlier context; T = 8192, GQA 32/8, head_dim 128, block_size 16,
bf16).  The decode-only batch (100 x 2001-token contexts, 32/32 heads) is
timed too, for the decode KV-read bandwidth and the roofline line.

Prints ONE JSON line.  Inputs are seeded synthetic data, resident in HBM
before the timed region starts.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "decode KV-read GB/s (% HBM peak) + mixed-batch attn tokens/s, 1 MI355X"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4, help="workload for the step (1-5)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["step", "decode", "prefill", "shared"], default=None,
                    help="run one leg only (for profiling)")
    ap.add_argument("--cpu-sample-rows", type=int, default=2048)
    return ap.parse_args()


class Timer:
    """HIP events on torch's current stream, which is the stream every libpa
    call below is enqueued on."""

    def __init__(self, torch):
        self.torch = torch

    def time(self, fn, iters, warmup):
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(iters):
            fn()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / iters  # ms


def setup(w, torch):
    from tests.gpu_path import GpuRun
    g = GpuRun(w).fill_history()
    torch.cuda.synchronize()
    return g


def step_fn(g, w, rpa, workspace, meta_out):
    db = g.db
    from ragged_paged_attention_amd.step import forward_step

    def fn():
        forward_step(db.q, db.k, db.v, g.k_cache, g.v_cache, db.query_lens, db.seq_lens, db.block_tables,
                     w.scale, max(1, w.max_query_len), max(1, w.max_seq_len), out=g.out_buf,
                     workspace=workspace, meta_out=meta_out)
    return fn


def cpu_baseline(w, rows_wanted, seed=0):
    """The oracle, as it stands, on a random sample of the step's rows: its
    metadata, its KV write of the step's rows, and attention for the sampled
    rows.  Pool filled with history first (untimed, like the GPU leg)."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_limits

    shape = w.pool_shape()
    kc = oracle.empty_pool(shape, w.dtype, w.pool_fill())
    vc = oracle.empty_pool(shape, w.dtype, w.pool_fill())
    oracle.fill_history(w.hist, kc, vc, w.block_size)
    rng = np.random.default_rng(seed)
    rows = sorted(rng.choice(w.num_tokens, size=min(rows_wanted, w.num_tokens), replace=False).tolist())
    st = w.step
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        md = oracle.build_metadata(st.query_lens, st.seq_lens, st.num_tokens, st.block_tables, w.block_size,
                                   w.num_blocks)
        oracle.write_kv(st.k, st.v, md.slot_mapping, kc, vc)
        oracle.attention(w.q, kc, vc, st.block_tables, md.query_start_loc, st.seq_lens, w.num_kv_heads,
                         w.scale, w.dtype, rows=rows)
        dt = time.perf_counter() - t0
    return {"value": len(rows) / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(rows)} random rows of the {w.num_tokens}-token step (seed {seed}), metadata + "
                      f"KV write of all new rows + fp64 attention of the sampled rows, {dt:.2f} s, BLAS pinned to 1 thread"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): this build has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import ragged_paged_attention_amd as rpa
    from workloads import accounting, config

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    timer = Timer(torch)
    result = {"metric": METRIC, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "data": "synthetic"}

    # ---------------- step on the mixed batch ----------------
    if args.only in (None, "step"):
        t0 = time.time()
        w = config(args.config, poison=False)
        print(f"[bench] generated config {args.config} {w.summary()} in {time.time() - t0:.1f}s", file=sys.stderr,
              flush=True)
        g = setup(w, torch)
        g.out_buf = torch.empty_like(g.db.q)
        need = rpa.pa_attention_workspace_size(w.num_seqs, w.num_tokens, w.num_q_heads, w.num_kv_heads,
                                               w.head_dim, w.max_seq_len)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        meta_out = {}
        fn = step_fn(g, w, rpa, ws, None)
        ms = timer.time(fn, args.steps, args.warmup)
        # per-call split of the step
        db = g.db
        md = rpa.pa_build_metadata(db.query_lens, db.seq_lens, w.num_tokens, db.block_tables, w.block_size,
                                   w.num_blocks)
        ms_meta = timer.time(lambda: rpa.pa_build_metadata(db.query_lens, db.seq_lens, w.num_tokens,
                                                           db.block_tables, w.block_size, w.num_blocks, out=md),
                             args.steps, 2)
        ms_write = timer.time(lambda: rpa.pa_write_kv(db.k, db.v, md["slot_mapping"], g.k_cache, g.v_cache),
                              args.steps, 2)
        attn = lambda: rpa.pa_attention(db.q, g.k_cache, g.v_cache, db.block_tables, md["query_start_loc"],
                                        db.seq_lens, w.max_query_len, w.max_seq_len, w.scale, out=g.out_buf,
                                        workspace=ws)
        ms_attn = timer.time(attn, args.steps, 2)
        kv_bytes = accounting.kv_read_bytes(w.step.seq_lens, w.num_kv_heads, w.head_dim, w.dtype)
        flops = accounting.attention_flops(w.step.query_lens, w.step.seq_lens, w.num_q_heads, w.head_dim)
        ql = w.step.query_lens
        result.update({
            "value": w.num_tokens / (ms / 1e3), "ms_per_step": ms, "dtype": w.dtype,
            "config": {"workload": w.name, "global_batch": w.num_seqs, "tokens": w.num_tokens,
                       "n_decode": int((ql == 1).sum()), "n_prefill": int((ql > 1).sum()),
                       "seq_len_max": w.max_seq_len, "heads": f"{w.num_q_heads}/{w.num_kv_heads}",
                       "head_dim": w.head_dim, "block_size": w.block_size, "seed": w.seed},
            "step_split_ms": {"pa_build_metadata": ms_meta, "pa_write_kv": ms_write, "pa_attention": ms_attn},
            "step_kv_bytes": kv_bytes, "step_flops": flops,
        })
        if not args.no_cpu_baseline:
            w_cpu = config(args.config, poison=False)
            result["cpu_baseline"] = cpu_baseline(w_cpu, args.cpu_sample_rows)
        del g, ws
        torch.cuda.empty_cache()

    # ---------------- decode-only batch: KV-read bandwidth ----------------
    if args.only in (None, "decode"):
        w3 = config(3, poison=False)
        g3 = setup(w3, torch)
        g3.out_buf = torch.empty_like(g3.db.q)
        db = g3.db
        md3 = rpa.pa_build_metadata(db.query_lens, db.seq_lens, w3.num_tokens, db.block_tables, w3.block_size,
                                    w3.num_blocks)
        rpa.pa_write_kv(db.k, db.v, md3["slot_mapping"], g3.k_cache, g3.v_cache)
        need = rpa.pa_attention_workspace_size(w3.num_seqs, w3.num_tokens, w3.num_q_heads, w3.num_kv_heads,
                                               w3.head_dim, w3.max_seq_len)
        ws3 = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        attn3 = lambda: rpa.pa_attention(db.q, g3.k_cache, g3.v_cache, db.block_tables, md3["query_start_loc"],
                                         db.seq_lens, w3.max_query_len, w3.max_seq_len, w3.scale, out=g3.out_buf,
                                         workspace=ws3)
        ms3 = timer.time(attn3, max(args.steps, 20), args.warmup)
        kv3 = accounting.kv_read_bytes(w3.step.seq_lens, w3.num_kv_heads, w3.head_dim, w3.dtype)
        gbs = kv3 / (ms3 / 1e3) / 1e9
        # ceilings on this machine: a contiguous streaming read of the K cache,
        # and the same paged gather as the decode kernel with no arithmetic
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        ms_stream = timer.time(lambda: rpa.pa_bench_stream_read(g3.k_cache, sink), 10, 3)
        stream_gbs = g3.k_cache.numel() * 2 / (ms_stream / 1e3) / 1e9
        ms_paged = timer.time(lambda: rpa.pa_bench_paged_read(g3.k_cache, g3.v_cache, db.block_tables, db.seq_lens,
                                                              w3.max_seq_len, sink), 20, 3)
        rounded = int(((w3.step.seq_lens.astype("int64") + 15) // 16 * 16).sum()) * 2 * w3.num_kv_heads * 256
        paged_gbs = rounded / (ms_paged / 1e3) / 1e9
        result["decode_kv_read"] = {"workload": w3.name, "GBps": gbs, "frac_hbm_peak": gbs / HBM_PEAK_GBS,
                                    "kv_bytes": kv3, "ms": ms3, "tokens": w3.num_tokens,
                                    "seqs": w3.num_seqs, "seq_len": w3.max_seq_len,
                                    "stream_read_GBps": stream_gbs, "paged_read_no_math_GBps": paged_gbs}
        result["roofline"] = {"bound": "hbm", "kernel": "pa_attention (decode batch)", "achieved": gbs,
                              "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "traffic": None}
    # ---------------- shared-prefix long-context decode ----------------
    if args.only in (None, "shared"):
        w5 = config(5, poison=False)
        g5 = setup(w5, torch)
        g5.out_buf = torch.empty_like(g5.db.q)
        db = g5.db
        md5 = rpa.pa_build_metadata(db.query_lens, db.seq_lens, w5.num_tokens, db.block_tables, w5.block_size,
                                    w5.num_blocks)
        rpa.pa_write_kv(db.k, db.v, md5["slot_mapping"], g5.k_cache, g5.v_cache)
        need = rpa.pa_attention_workspace_size(w5.num_seqs, w5.num_tokens, w5.num_q_heads, w5.num_kv_heads,
                                               w5.head_dim, w5.max_seq_len)
        ws5 = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        attn5 = lambda: rpa.pa_attention(db.q, g5.k_cache, g5.v_cache, db.block_tables, md5["query_start_loc"],
                                         db.seq_lens, w5.max_query_len, w5.max_seq_len, w5.scale, out=g5.out_buf,
                                         workspace=ws5)
        ms5 = timer.time(attn5, max(args.steps, 20), args.warmup)
        kv5 = accounting.kv_read_bytes(w5.step.seq_lens, w5.num_kv_heads, w5.head_dim, w5.dtype)
        uq5 = accounting.unique_kv_bytes_fast(w5.step.block_tables, w5.step.seq_lens, w5.block_size,
                                              w5.num_kv_heads, w5.head_dim, w5.dtype)
        result["shared_prefix_decode"] = {"workload": w5.name, "logical_GBps": kv5 / (ms5 / 1e3) / 1e9,
                                          "unique_GBps": uq5 / (ms5 / 1e3) / 1e9, "logical_bytes": kv5,
                                          "unique_bytes": uq5, "ms": ms5}
        del g5, ws5
        torch.cuda.empty_cache()

    # ---------------- ragged prefill batch: MFMA throughput ----------------
    if args.only in (None, "prefill"):
        w2 = config(2, poison=False)
        g2 = setup(w2, torch)
        g2.out_buf = torch.empty_like(g2.db.q)
        db = g2.db
        md2 = rpa.pa_build_metadata(db.query_lens, db.seq_lens, w2.num_tokens, db.block_tables, w2.block_size,
                                    w2.num_blocks)
        rpa.pa_write_kv(db.k, db.v, md2["slot_mapping"], g2.k_cache, g2.v_cache)
        attn2 = lambda: rpa.pa_attention(db.q, g2.k_cache, g2.v_cache, db.block_tables, md2["query_start_loc"],
                                         db.seq_lens, w2.max_query_len, w2.max_seq_len, w2.scale, out=g2.out_buf)
        ms2 = timer.time(attn2, max(args.steps, 20), args.warmup)
        fl2 = accounting.attention_flops(w2.step.query_lens, w2.step.seq_lens, w2.num_q_heads, w2.head_dim)
        tf = fl2 / (ms2 / 1e3) / 1e12
        result["prefill_mfma"] = {"workload": w2.name, "TFLOPs": tf, "frac_bf16_peak": tf / BF16_PEAK_TFLOPS,
                                  "flops": fl2, "ms": ms2, "tokens": w2.num_tokens}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

"""Throughput of one continuous-batching attention step on one MI355X.

A step is the whole hot path over one batch, in the order the pages give
("vLLM Continuous Batching：从 Forward Shape 理解两个核心参数" §2.3): build the
flat-batch metadata, scatter the new K/V by slot_mapping, then ragged paged
attention (decode rows, split-K merge, prefill chunks, one mixed batch).  All
of it runs as libpa kernels (C ABI) on torch's current stream.

Step workload (the JSON `value`): the chunked-prefill mixed batch -- 240
decode sequences with log-uniform contexts 128..8192 plus 16 prefill chunks of
497 tokens with 0..4096 earlier tokens; T = 8192 new tokens, S = 256, GQA
32/8 heads, head_dim 128, block_size 16, bf16, seeded synthetic data,
inputs resident in HBM before timing.  value = T / step time (tokens/s).

Also reported (same run): the decode batch's KV-read bandwidth (100 x
2001-token contexts, 32/32 heads) against HBM peak and against measured read
ceilings, the ragged prefill batch's TFLOP/s (16/128/1024/2048-token prompts),
the shared-prefix long-context decode batch, the speculative-decoding verify
batch (64 sequences, query_len 2..8 over 2k..16k-token contexts, 32/8 heads)
as KV-read bandwidth, block copies for copy-on-write
(device to device) and swap (device to pinned host and back), and the
oracle's CPU throughput on a sample of the step's rows.  Prints ONE JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, TFLOP/s (256 CU x 2.4 GHz x 4096 FLOP/clk)
METRIC = "decode KV-read GB/s (% HBM peak) + mixed-batch attn tokens/s, 1 MI355X"
PROFILES = os.path.join(ROOT, "profiles")
# name fragment that identifies each kernel in rocprofv3 output (bf16 instances)
KERNEL_MATCH = {
    "decode_kernel": "decode_kernel<pa::BF16, 1, 128, true",  # also the instance run beside the prefill kernel
    "decode_kernel_2t": "decode_kernel<pa::BF16, 2, 128, true",
    "merge_kernel": "merge_kernel<pa::BF16, 128>",
    "prefill_kernel": "prefill_kernel<pa::BF16, true, 128>",
    "write_kv_kernel": "write_kv_kernel",
    "copy_blocks_kernel": "copy_blocks_kernel",
}
KERNEL_SOURCES = {
    "decode_kernel": "ragged_paged_attention_amd/csrc/attn_fast.hip",
    "decode_kernel_2t": "ragged_paged_attention_amd/csrc/attn_fast.hip",
    "merge_kernel": "ragged_paged_attention_amd/csrc/attn_fast.hip",
    "prefill_kernel": "ragged_paged_attention_amd/csrc/attn_prefill.hip",
    "write_kv_kernel": "ragged_paged_attention_amd/csrc/write_kv.hip",
    "copy_blocks_kernel": "ragged_paged_attention_amd/csrc/copy_blocks.hip",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["step", "decode", "prefill", "shared", "verify", "blocks", "variants"],
                    default=None,
                    help="run one leg only (for profiling)")
    ap.add_argument("--cpu-sample-rows", type=int, default=2048)
    ap.add_argument("--no-sub-batch", action="store_true",
                    help="in the step leg, skip the prefill chunks' run on their own (profiles of the mixed step "
                         "then hold only its dispatches)")
    ap.add_argument("--cold-launches", type=int, default=50,
                    help="single launches timed after a cache flush each (median reported)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("ROCPROF_DIR", "OUT_MD"),
                    help="write a kernel-time summary (profiles/*.md) from a rocprofv3 --kernel-trace --stats "
                         "--output-format csv directory; no GPU needed")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "KERNEL", "WORKLOAD"),
                    help="write profiles/KERNEL.WORKLOAD.pmc.md from two rocprofv3 --pmc runs (FETCH_SIZE, "
                         "WRITE_SIZE) of a bench leg, calibrated on the leg's copy of known size; no GPU needed")
    ap.add_argument("--summarize-mfma", nargs=3, metavar=("PMC_DIR", "KERNEL", "WORKLOAD"),
                    help="write profiles/KERNEL.WORKLOAD.mfma.pmc.md from one rocprofv3 --pmc --kernel-trace run "
                         "with the MFMA counters; no GPU needed")
    ap.add_argument("--summarize-mempath", nargs=1, metavar="PMC_DIR",
                    help="write profiles/prefill_kernel.chunked_mixed.memory_path.pmc.md from one rocprofv3 --pmc run "
                         "of the step leg with the TA / TD / TCP / TCC counters; no GPU needed")
    ap.add_argument("--summarize-waves", nargs=2, metavar=("STEP_PMC_DIR", "PREFILL_PMC_DIR"),
                    help="write profiles/prefill_kernel.wave_states.pmc.md from rocprofv3 --pmc runs of the step and "
                         "prefill legs with the SQ wave-state counters; no GPU needed")
    ap.add_argument("--command", default="", help="the command that produced the rocprofv3 output (recorded; "
                                                  "for --summarize-waves, STEP_OR_PREFILL stands for the leg)")
    ap.add_argument("--note", default="", help="a paragraph added to a counter summary (how to read it)")
    return ap.parse_args()


def source_hash(rel: str) -> str:
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


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

    def time_cold(self, fn, iters=50, flush_bytes=1 << 30):
        """Median (and 10th / 90th percentile) over `iters` single calls, each
        preceded by a read of `flush_bytes` of a separate buffer (four times
        the 256 MB Infinity Cache, so the call starts with cold caches), each
        call bracketed by its own pair of events on the current stream.  The
        flush reads rather than writes: after a write, the caches hold dirty
        lines of the flush buffer whose write-back would land in the timed
        call."""
        torch = self.torch
        if getattr(self, "_flush", None) is None or self._flush.numel() != flush_bytes // 4:
            self._flush = torch.ones(flush_bytes // 4, dtype=torch.int32, device="cuda")
            self._flush_sum = torch.empty((), dtype=torch.int64, device="cuda")
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
        fn()
        torch.cuda.synchronize()
        for i in range(iters):
            torch.sum(self._flush, dim=0, dtype=torch.int64, out=self._flush_sum)
            ev[i][0].record()
            fn()
            ev[i][1].record()
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in ev)
        pick = lambda q: ts[min(len(ts) - 1, int(q * (len(ts) - 1) + 0.5))]
        return {"median_ms": pick(0.5), "p10_ms": pick(0.1), "p90_ms": pick(0.9), "launches": iters,
                "flush_bytes": flush_bytes}

    def kernels(self, rpa, fn, iters):
        """Per-kernel launch durations (library-side HIP events on the launch
        stream) over `iters` calls of fn: {name: (launches, avg ms)}."""
        self.torch.cuda.synchronize()
        rpa.pa_bench_timing_begin()
        for _ in range(iters):
            fn()
        res = rpa.pa_bench_timing_end()
        return {k: (n, ms / n) for k, (n, ms) in res.items()}


def setup(w, torch):
    from tests.gpu_path import DeviceRun
    g = DeviceRun(w).fill_history()
    torch.cuda.synchronize()
    return g


def metadata_and_write(w, g, rpa, timer, args):
    """pa_build_metadata and pa_write_kv of a leg's step, each on its own (the
    step itself runs the write inside pa_write_kv_attention's planning
    launch): back to back and cold-cache times.  The write's algorithmic bytes
    are 2 (K, V) x 2 (read, write) x T x Hkv x D x element size; rewriting the
    same rows leaves the cache as it was."""
    db = g.db
    md = rpa.pa_build_metadata(db.query_lens, db.seq_lens, w.num_tokens, db.block_tables, w.block_size,
                               w.num_blocks)
    meta = lambda: rpa.pa_build_metadata(db.query_lens, db.seq_lens, w.num_tokens, db.block_tables, w.block_size,
                                         w.num_blocks, out=md)
    write = lambda: rpa.pa_write_kv(db.k, db.v, md["slot_mapping"], g.k_cache, g.v_cache)
    n = max(args.steps, 20)
    ms_m, cold_m = timer.time(meta, n, args.warmup), timer.time_cold(meta, args.cold_launches)
    ms_w, cold_w = timer.time(write, n, args.warmup), timer.time_cold(write, args.cold_launches)
    wb = 4 * w.num_tokens * w.num_kv_heads * w.head_dim * (4 if w.dtype == "f32" else 2)
    gbs = wb / (ms_w / 1e3) / 1e9
    return {
        "pa_build_metadata": {"seqs": w.num_seqs, "tokens": w.num_tokens, "ms_per_call": ms_m,
                              "cold_median_ms": cold_m["median_ms"]},
        "pa_write_kv": {"rows": w.num_tokens, "bytes": wb, "ms_per_call": ms_w, "GBps": gbs,
                        "frac_hbm_peak": gbs / HBM_PEAK_GBS, "cold_median_ms": cold_w["median_ms"],
                        "cold_GBps": wb / (cold_w["median_ms"] / 1e3) / 1e9}}


def workspace_for(w, rpa, torch):
    need = rpa.pa_attention_workspace_size(w.num_seqs, w.num_tokens, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                           w.max_query_len, w.max_seq_len)
    return torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")


def traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, calibrated on a copy of known size), or None if
    there is none or the kernel's source changed since it was taken."""
    path = os.path.join(PROFILES, f"{kernel}.{workload}.pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_sha256_16:\s*([0-9a-f]{16})", text)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.e+]+)", text)
    if not m or not b or m.group(1) != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return float(b.group(1))


def cpu_baseline(w, rows_wanted, seed=0):
    """The oracle, as it stands, on a random sample of the step's rows: its
    metadata, its KV write of all the step's new rows, and fp64 attention for
    the sampled rows.  The pool is filled with history first (untimed, like
    the GPU leg)."""
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
            "sample": f"{len(rows)} random rows of the {w.num_tokens}-token mixed step (seed {seed}): metadata + "
                      f"KV write of all new rows + fp64 attention of the sampled rows in {dt:.2f} s; "
                      f"NumPy with BLAS pinned to 1 thread"}


def work_split(w, one_decode_launch=False):
    """Algorithmic work of each attention kernel of a call: KV/Q/O bytes of
    the sequences each decode kernel takes (query_len * G rows per KV head:
    up to 16 on one tile, 17..32 on two when the max_query_len hint allows
    them) and causal FLOPs of the prefill-class rest.  one_decode_launch:
    the call ran only the one-tile decode kernel (with the planning kernel's
    work list it takes every decode item, those of more than 16 rows in two
    passes), so it gets all the decode bytes."""
    import numpy as np
    from workloads import accounting
    G = w.num_q_heads // w.num_kv_heads
    ql, sl = w.step.query_lens.astype(np.int64), w.step.seq_lens.astype(np.int64)
    cap = 32 if max(1, w.max_query_len) * G > 16 else 16
    rows = ql * G
    es = accounting.itemsize(w.dtype)

    def dec_bytes(sel):
        return (accounting.kv_read_bytes(sl[sel], w.num_kv_heads, w.head_dim, w.dtype)
                + 2 * int(ql[sel].sum()) * w.num_q_heads * w.head_dim * es)

    if one_decode_launch:
        return {"decode_kernel": dec_bytes(rows <= cap), "decode_kernel_2t": 0,
                "prefill_kernel": accounting.attention_flops(ql[rows > cap], sl[rows > cap], w.num_q_heads,
                                                             w.head_dim)}
    return {"decode_kernel": dec_bytes(rows <= 16),
            "decode_kernel_2t": dec_bytes((rows > 16) & (rows <= cap)),
            "prefill_kernel": accounting.attention_flops(ql[rows > cap], sl[rows > cap], w.num_q_heads,
                                                         w.head_dim)}


def roofline_for(kernel, avg_ms, w, workload_tag, one_decode_launch=False):
    work = work_split(w, one_decode_launch)
    if kernel == "prefill_kernel":
        pre_flops = work[kernel]
        a = pre_flops / (avg_ms / 1e3) / 1e12
        return {"bound": "mfma", "kernel": kernel, "achieved": a, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": a / BF16_PEAK_TFLOPS, "traffic": traffic_from_profiles(kernel, workload_tag),
                "work_per_launch": pre_flops, "avg_launch_ms": avg_ms,
                "mfma_busy": mfma_from_profiles(kernel, workload_tag)}
    dec_bytes = work[kernel]
    a = dec_bytes / (avg_ms / 1e3) / 1e9
    return {"bound": "hbm", "kernel": kernel, "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": a / HBM_PEAK_GBS, "traffic": traffic_from_profiles(kernel, workload_tag),
            "work_per_launch": dec_bytes, "avg_launch_ms": avg_ms}


CAL_BYTES = 256 << 20  # calibration copy: 256 MiB read + 256 MiB written


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(dirpath, suffix):
    for root, _, files in os.walk(dirpath):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError(f"no *{suffix} under {dirpath}")


def summarize_trace(src_dir, out_md, command):
    rows = _csv_rows(_find(src_dir, "kernel_stats.csv"))
    lines = [f"# Kernel time summary: {os.path.basename(out_md)[:-3]}", "",
             f"Command (run from the repository root on one MI355X): `{command}`", "",
             "| kernel | calls | avg us | min us | max us | share of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = re.sub(r"\(anonymous namespace\)::", "", r["Name"])
        name = re.sub(r"\(.*", "", name).replace("void ", "")
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {out_md}")


def _counter_per_dispatch(rows, counter, kernel_substr):
    per = {}
    for r in rows:
        if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"]:
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return per


def summarize_pmc(fetch_dir, write_dir, kernel, workload, command):
    """FETCH_SIZE / WRITE_SIZE are in KiB per dispatch.  The bench leg runs a
    copy of CAL_BYTES (read CAL_BYTES, write CAL_BYTES); the ratio of what the
    counters report for it to CAL_BYTES is the calibration factor applied to
    the kernel's counts."""
    fr = _csv_rows(_find(fetch_dir, "counter_collection.csv"))
    wr = _csv_rows(_find(write_dir, "counter_collection.csv"))
    kf = _counter_per_dispatch(fr, "FETCH_SIZE", KERNEL_MATCH.get(kernel, kernel))
    kw = _counter_per_dispatch(wr, "WRITE_SIZE", KERNEL_MATCH.get(kernel, kernel))
    # torch's fill_ (writes) and copy_ (reads and writes) of the calibration buffers
    cf, cw = [], []
    for cal in ("copyBuffer", "elementwise_kernel"):
        cf += list(_counter_per_dispatch(fr, "FETCH_SIZE", cal).values())
        cw += list(_counter_per_dispatch(wr, "WRITE_SIZE", cal).values())
    cal_kib = CAL_BYTES / 1024
    f_fac = max(cf, key=lambda v: -abs(v - cal_kib)) / cal_kib if cf else 1.0
    w_fac = max(cw, key=lambda v: -abs(v - cal_kib)) / cal_kib if cw else 1.0
    fetch = sum(kf.values()) / max(1, len(kf)) * 1024 / f_fac
    write = sum(kw.values()) / max(1, len(kw)) * 1024 / w_fac
    out_md = os.path.join(PROFILES, f"{kernel}.{workload}.pmc.md")
    text = f"""# HBM traffic: {kernel} on the {workload} workload

Commands (run from the repository root on one MI355X):
- `{command.replace("COUNTER", "FETCH_SIZE")}`
- `{command.replace("COUNTER", "WRITE_SIZE")}`

Counters are KiB per dispatch.  Calibration: the same bench leg copies {CAL_BYTES >> 20} MiB with torch
(`copy_`); FETCH_SIZE read {f_fac:.4f}x and WRITE_SIZE {w_fac:.4f}x of the known bytes for it, and the
kernel's counts are divided by those factors.

| quantity | value |
|---|---|
| dispatches measured | {len(kf)} (FETCH) / {len(kw)} (WRITE) |
| FETCH_SIZE per dispatch, calibrated | {fetch / 1e6:.2f} MB |
| WRITE_SIZE per dispatch, calibrated | {write / 1e6:.2f} MB |
| calibration factors (fetch, write) | {f_fac:.4f}, {w_fac:.4f} |

hbm_bytes_per_launch: {fetch + write:.6e}
source_sha256_16: {source_hash(KERNEL_SOURCES[kernel])}
"""
    with open(out_md, "w") as f:
        f.write(text)
    print(f"wrote {out_md}")


SIMDS = 256 * 4  # MI355X: 256 CUs x 4 SIMDs


def _workload_flops(kernel, workload):
    """Algorithmic FLOPs one launch of `kernel` performs on the named workload."""
    from workloads import CONFIG_NAMES, config
    n = {v: k for k, v in CONFIG_NAMES.items()}[workload]
    w = config(n, poison=False)
    return work_split(w)[kernel]


def summarize_mfma(pmc_dir, kernel, workload, command, note=""):
    """MFMA counters of one kernel, per dispatch, and what they say:
      - MFMA busy fraction = SQ_VALU_MFMA_BUSY_CYCLES / (active cycles per XCD
        x 1024 SIMDs): GRBM_GUI_ACTIVE adds up the 8 XCDs, so the active cycles
        of one XCD (the kernel's duration in shader-clock cycles) are
        GRBM_GUI_ACTIVE / 8;
      - counted MFMA FLOPs = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (the counter
        is in units of 512 FLOPs) against the algorithmic FLOPs (causal pairs
        only; the kernel also multiplies the masked half of diagonal tiles);
      - the shader clock under the kernel = active cycles per XCD / duration."""
    rows = _csv_rows(_find(pmc_dir, "counter_collection.csv"))
    match = KERNEL_MATCH.get(kernel, kernel)
    names = sorted({r["Counter_Name"] for r in rows})
    per = {c: _counter_per_dispatch(rows, c, match) for c in names}
    avg = {c: sum(v.values()) / max(1, len(v)) for c, v in per.items() if v}
    n_disp = max((len(v) for v in per.values()), default=0)
    durs = []
    try:
        for r in _csv_rows(_find(pmc_dir, "kernel_trace.csv")):
            if match in r["Kernel_Name"]:
                durs.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    except FileNotFoundError:
        pass
    dur_us = sum(durs) / len(durs) if durs else None
    active = avg.get("GRBM_GUI_ACTIVE", 0.0) / 8
    busy = avg.get("SQ_VALU_MFMA_BUSY_CYCLES")
    frac = busy / (active * SIMDS) if busy and active else None
    counted = avg["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in avg else None
    alg = _workload_flops(kernel, workload)
    clock = active / (dur_us * 1e3) if dur_us and active else None
    lines = [f"# MFMA counters: {kernel} on the {workload} workload", "",
             "Command (run from the repository root on one MI355X):", f"- `{command}`", "",
             f"Per dispatch, averaged over {n_disp} dispatches of `{match}`.  GRBM_GUI_ACTIVE adds up the",
             "8 XCDs; one XCD's active cycles (GRBM_GUI_ACTIVE / 8) are the kernel's span in shader-clock",
             "cycles.  MFMA busy fraction = SQ_VALU_MFMA_BUSY_CYCLES / (those cycles x 1024 SIMDs).",
             "SQ_INSTS_VALU_MFMA_MOPS_BF16 counts bf16 MFMA work in units of 512 FLOPs.", ""]
    if note:
        lines += [note, ""]
    lines += ["| counter | per dispatch |", "|---|---|"]
    lines += [f"| {c} | {v:.4e} |" for c, v in sorted(avg.items())]
    lines += ["", "| derived | value |", "|---|---|"]
    if dur_us:
        lines.append(f"| kernel duration under counters (kernel trace) | {dur_us:.2f} us |")
    if clock:
        lines.append(f"| shader clock over the kernel | {clock:.3f} GHz |")
    if frac is not None:
        lines.append(f"| MFMA busy fraction | {frac:.4f} |")
    if counted:
        lines.append(f"| counted MFMA FLOPs | {counted:.4e} |")
    lines.append(f"| algorithmic FLOPs (causal) | {alg:.4e} |")
    if counted:
        lines.append(f"| counted / algorithmic | {counted / alg:.4f} |")
    if counted and busy:
        lines.append(f"| busy cycles per 1024 counted FLOPs | {busy * 1024 / counted:.4f} |")
    lines += ["", f"mfma_busy_frac: {frac if frac is not None else 'null'}",
              f"shader_clock_ghz: {clock if clock else 'null'}",
              f"source_sha256_16: {source_hash(KERNEL_SOURCES[kernel])}", ""]
    out_md = os.path.join(PROFILES, f"{kernel}.{workload}.mfma.pmc.md")
    with open(out_md, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {out_md}")


def _per_dispatch_avg(rows, kernel_substr):
    """{counter: value per dispatch, averaged} over the dispatches of one kernel."""
    per = {}
    for r in rows:
        if kernel_substr not in r["Kernel_Name"]:
            continue
        d = per.setdefault(r["Dispatch_Id"], {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    if not per:
        return {}, 0
    names = set().union(*per.values())
    return {c: sum(d.get(c, 0.0) for d in per.values()) / len(per) for c in names}, len(per)


SPLIT_NOTE = ("Counter collection runs the dispatches one at a time: on the mixed batch the prefill launch holds one "
              "workgroup per CU (the decode launch runs beside it in the timed step), so here it runs alone at half "
              "occupancy.")


def summarize_mempath(pmc_dir, command):
    """TA / TD busy per CU, the TCP data stall and L1-to-L2 reads, and the L2
    hit rate of the mixed step's prefill kernel, per dispatch."""
    avg, n = _per_dispatch_avg(_csv_rows(_find(pmc_dir, "counter_collection.csv")), KERNEL_MATCH["prefill_kernel"])
    act = avg["GRBM_GUI_ACTIVE"] / 8
    h, m = avg["TCC_HIT_sum"], avg["TCC_MISS_sum"]
    text = f"""# Memory-path counters: prefill_kernel on the chunked_mixed workload

Command (run from the repository root on one MI355X):
- `{command}`

Per dispatch, averaged over {n} dispatches.  `_sum` counters add up all instances (one TA,
TD and TCP per CU, 256 CUs); GRBM_GUI_ACTIVE adds up the 8 XCDs.  Busy fractions are per CU
against GRBM_GUI_ACTIVE / 8.  {SPLIT_NOTE}

| quantity | value |
|---|---|
| GRBM_GUI_ACTIVE | {avg['GRBM_GUI_ACTIVE']:.3e} |
| TA_TA_BUSY_sum | {avg['TA_TA_BUSY_sum']:.3e} ({avg['TA_TA_BUSY_sum'] / 256 / act:.0%} of the active cycles per CU) |
| TD_TD_BUSY_sum | {avg['TD_TD_BUSY_sum']:.3e} ({avg['TD_TD_BUSY_sum'] / 256 / act:.0%} per CU) |
| TCP_TCP_TA_DATA_STALL_CYCLES_sum | {avg['TCP_TCP_TA_DATA_STALL_CYCLES_sum']:.3e} |
| TCP_TCC_READ_REQ_sum | {avg['TCP_TCC_READ_REQ_sum']:.3e} |
| TCC_HIT_sum / TCC_MISS_sum | {h:.3e} / {m:.3e} (L2 hit rate {h / (h + m):.0%}) |

source_sha256_16: {source_hash(KERNEL_SOURCES['prefill_kernel'])}
"""
    out_md = os.path.join(PROFILES, "prefill_kernel.chunked_mixed.memory_path.pmc.md")
    with open(out_md, "w") as f:
        f.write(text)
    print(f"wrote {out_md}")


def summarize_waves(step_dir, prefill_dir, command):
    """Wave-state fractions of the prefill kernel's resident wave cycles on the
    mixed step and the ragged prefill legs."""
    cols = ["SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
            "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM"]
    lines = ["# Wave-state counters: prefill_kernel (chunked_mixed and ragged_prefill workloads)", "",
             "Commands (run from the repository root on one MI355X):",
             f"- `{command.replace('STEP_OR_PREFILL', 'step')}`", f"- `{command.replace('STEP_OR_PREFILL', 'prefill')}`",
             "", f"Per dispatch of `{KERNEL_MATCH['prefill_kernel']}`, averaged; fractions are of SQ_WAVE_CYCLES",
             "(every wave's resident cycles).  SQ_WAIT_ANY: waiting on a counter, a barrier or a dependency;",
             "SQ_WAIT_INST_ANY: an instruction ready but not issued; SQ_ACTIVE_INST_*: issuing.", SPLIT_NOTE, "",
             "| workload | dispatches | SQ_WAVE_CYCLES | wait_any | wait_inst_any | wait_inst_lds | active_any | "
             "active_valu | active_lds | active_vmem |", "|---|---|---|---|---|---|---|---|---|---|"]
    for d, wl in ((step_dir, "chunked_mixed"), (prefill_dir, "ragged_prefill")):
        avg, n = _per_dispatch_avg(_csv_rows(_find(d, "counter_collection.csv")), KERNEL_MATCH["prefill_kernel"])
        wc = avg["SQ_WAVE_CYCLES"]
        lines.append(f"| {wl} | {n} | {wc:.3e} | " + " | ".join(f"{avg[c] / wc:.2f}" for c in cols) + " |")
    lines += ["", f"source_sha256_16: {source_hash(KERNEL_SOURCES['prefill_kernel'])}", ""]
    out_md = os.path.join(PROFILES, "prefill_kernel.wave_states.pmc.md")
    with open(out_md, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {out_md}")


def mfma_from_profiles(kernel: str, workload: str):
    """MFMA busy fraction and shader clock from the committed counter summary,
    or None if there is none or the kernel's source changed since."""
    path = os.path.join(PROFILES, f"{kernel}.{workload}.mfma.pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_sha256_16:\s*([0-9a-f]{16})", text)
    b = re.search(r"mfma_busy_frac:\s*([0-9.e+-]+)", text)
    c = re.search(r"shader_clock_ghz:\s*([0-9.e+-]+)", text)
    if not m or not b or m.group(1) != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return {"mfma_busy_frac": float(b.group(1)), "shader_clock_ghz": float(c.group(1)) if c else None,
            "source": os.path.relpath(path, ROOT)}


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace[0], args.summarize_trace[1], args.command)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, args.command)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma, args.command, args.note)
        return
    if args.summarize_mempath:
        summarize_mempath(args.summarize_mempath[0], args.command)
        return
    if args.summarize_waves:
        summarize_waves(*args.summarize_waves, args.command)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} was asked for): the library has no multi-GPU "
              "path; run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    import ragged_paged_attention_amd as rpa
    from ragged_paged_attention_amd.step import forward_step
    from workloads import accounting, config, decode_variant, permute_sequences, prefill_variant, verify_batch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    timer = Timer(torch)
    # a copy of known size, for calibrating HBM byte counters in profiling runs
    cal_src = torch.empty(CAL_BYTES // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst
    result = {"metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) bf16, random block placement)"}

    # ---------------- the step: mixed batch ----------------
    if args.only in (None, "step"):
        t0 = time.time()
        w = config(4, poison=False)
        print(f"[bench] mixed batch {w.summary()} generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
        g = setup(w, torch)
        out = torch.empty_like(g.db.q)
        ws = workspace_for(w, rpa, torch)
        db = g.db

        def step():
            forward_step(db.q, db.k, db.v, g.k_cache, g.v_cache, db.query_lens, db.seq_lens, db.block_tables,
                         w.scale, w.max_query_len, w.max_seq_len, out=out, workspace=ws)

        ms = timer.time(step, args.steps, args.warmup)
        cold = timer.time_cold(step, args.cold_launches)
        kern = timer.kernels(rpa, step, args.steps)
        ql = w.step.query_lens
        one = "decode_kernel_2t" not in kern
        split = work_split(w, one)
        dec_bytes = split["decode_kernel"] + split["decode_kernel_2t"]
        result.update({
            "value": w.num_tokens / (ms / 1e3), "ms_per_step": ms, "dtype": w.dtype,
            "config": {"workload": "chunked-prefill mixed batch", "seqs": w.num_seqs, "tokens": w.num_tokens,
                       "n_decode": int((ql == 1).sum()), "n_prefill_chunks": int((ql > 1).sum()),
                       "chunk_len": int(ql.max()), "seq_len_max": w.max_seq_len,
                       "heads_q_kv": [w.num_q_heads, w.num_kv_heads], "head_dim": w.head_dim,
                       "block_size": w.block_size, "pool_blocks": w.num_blocks, "seed": w.seed},
            "kernels_ms_per_step": {k: round(n * avg / args.steps, 5) for k, (n, avg) in kern.items()},
            "cold_cache": {**cold, "tokens_per_s": w.num_tokens / (cold["median_ms"] / 1e3)},
            "step_work": {"decode_bytes": dec_bytes, "prefill_flops": split["prefill_kernel"]},
        })
        # the whole step against the two rooflines: the time the decode bytes
        # need at peak HBM bandwidth and the prefill flops at peak MFMA rate,
        # if the two overlapped perfectly (the larger) or ran one after the
        # other (the sum)
        t_hbm = dec_bytes / (HBM_PEAK_GBS * 1e9) * 1e3
        t_mfma = split["prefill_kernel"] / (BF16_PEAK_TFLOPS * 1e12) * 1e3
        result["step_roofline"] = {
            "decode_at_hbm_peak_ms": round(t_hbm, 5), "prefill_at_mfma_peak_ms": round(t_mfma, 5),
            "overlap_bound_ms": round(max(t_hbm, t_mfma), 5), "serial_bound_ms": round(t_hbm + t_mfma, 5),
            "frac_overlap": max(t_hbm, t_mfma) / ms, "frac_serial": (t_hbm + t_mfma) / ms}
        weight = lambda k: kern.get(k, (0, 0.0))[0] * kern.get(k, (0, 0.0))[1]
        # On this batch the library runs the decode launches beside the
        # prefill kernel (the two share every CU): their launch durations then
        # overlap and add up to more than the step.  The dominant kernel is
        # then the one whose roofline bounds the shared phase (HBM: the decode
        # bytes at peak bandwidth take longer than the prefill flops at peak
        # MFMA rate), and each launch's duration spans the shared phase.
        both = "decode_kernel" in kern and "prefill_kernel" in kern
        concurrent = both and kern["decode_kernel"][1] + kern["prefill_kernel"][1] > ms
        if concurrent:
            dominant = "decode_kernel" if t_hbm >= t_mfma else "prefill_kernel"
        else:
            dominant = max(("decode_kernel", "prefill_kernel"), key=weight)
        result["roofline"] = roofline_for(dominant, kern[dominant][1], w, w.name, one)
        other = "prefill_kernel" if dominant == "decode_kernel" else "decode_kernel"
        if other in kern:
            result["roofline_other_kernel"] = roofline_for(other, kern[other][1], w, w.name, one)
        if concurrent:
            result["roofline"]["concurrent_with"] = other
            result["roofline_other_kernel"]["concurrent_with"] = dominant
            for r in (result["roofline"], result["roofline_other_kernel"]):
                if r.get("mfma_busy"):
                    # counter collection runs dispatches one at a time
                    r["mfma_busy"]["measured_alone"] = True
        result["step_metadata_and_write"] = metadata_and_write(w, g, rpa, timer, args)
        del g, ws, out
        torch.cuda.empty_cache()
        # The prefill sub-batch alone (the chunks without the decode
        # sequences): the prefill kernel at two workgroups per CU, as in a
        # batch with few decodes, so its own roofline on this shape stands
        # next to the shared-phase figure above.
        chunks = [s for s in range(w.num_seqs) if int(ql[s]) > 1]
        if chunks and not args.no_sub_batch:
            wc = permute_sequences(w, chunks)
            gc = setup(wc, torch)
            outc = torch.empty_like(gc.db.q)
            wsc = workspace_for(wc, rpa, torch)
            dbc = gc.db

            def step_chunks():
                forward_step(dbc.q, dbc.k, dbc.v, gc.k_cache, gc.v_cache, dbc.query_lens, dbc.seq_lens,
                             dbc.block_tables, wc.scale, wc.max_query_len, wc.max_seq_len, out=outc, workspace=wsc)

            msc = timer.time(step_chunks, args.steps, args.warmup)
            kc = timer.kernels(rpa, step_chunks, args.steps)
            pk_ms = kc["prefill_kernel"][1]
            a_tf = split["prefill_kernel"] / (pk_ms / 1e3) / 1e12
            result["prefill_sub_batch_alone"] = {
                "workload": f"the step's {len(chunks)} prefill chunks alone", "ms_per_call": msc,
                "prefill_kernel_ms": pk_ms, "TFLOPs": a_tf, "frac_bf16_peak": a_tf / BF16_PEAK_TFLOPS,
                "kernels_ms": {k: round(n * avg / args.steps, 5) for k, (n, avg) in kc.items()}}
            del gc, wsc, outc
            torch.cuda.empty_cache()
        if not args.no_cpu_baseline:
            result["cpu_baseline"] = cpu_baseline(config(4, poison=False), args.cpu_sample_rows)

    # ---------------- decode-only batch: KV-read bandwidth ----------------
    if args.only in (None, "decode"):
        w3 = config(3, poison=False)
        g3 = setup(w3, torch).write_step_rows()
        db = g3.db
        ws3 = workspace_for(w3, rpa, torch)
        out3 = torch.empty_like(db.q)
        qsl3 = g3.meta["query_start_loc"]
        attn3 = lambda: rpa.pa_attention(db.q, g3.k_cache, g3.v_cache, db.block_tables, qsl3, db.seq_lens,
                                         w3.max_query_len, w3.max_seq_len, w3.scale, out=out3, workspace=ws3)
        ms3 = timer.time(attn3, max(args.steps, 20), args.warmup)
        cold3 = timer.time_cold(attn3, args.cold_launches)
        kern3 = timer.kernels(rpa, attn3, 10)
        kv3 = accounting.kv_read_bytes(w3.step.seq_lens, w3.num_kv_heads, w3.head_dim, w3.dtype)
        gbs = kv3 / (ms3 / 1e3) / 1e9
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        ms_stream = timer.time(lambda: rpa.pa_bench_stream_read(g3.k_cache, sink), 10, 3)
        stream_gbs = g3.k_cache.numel() * 2 / (ms_stream / 1e3) / 1e9
        ms_paged = timer.time(lambda: rpa.pa_bench_paged_read(g3.k_cache, g3.v_cache, db.block_tables,
                                                              db.seq_lens, w3.max_seq_len, sink), 20, 3)
        rounded = int(((w3.step.seq_lens.astype("int64") + 15) // 16 * 16).sum()) * 2 * w3.num_kv_heads * 256
        result["decode_kv_read"] = {
            "workload": "decode batch: 100 seqs x 2001 tokens, 32/32 heads, D 128, bs 16, bf16",
            "GBps": gbs, "frac_hbm_peak": gbs / HBM_PEAK_GBS, "kv_bytes": kv3, "ms_per_call": ms3,
            "cold_cache": {**cold3, "GBps": kv3 / (cold3["median_ms"] / 1e3) / 1e9},
            "kernels_ms": {k: round(avg, 5) for k, (n, avg) in kern3.items()},
            "decode_kernel_GBps": kv3 / (kern3["decode_kernel"][1] / 1e3) / 1e9,
            "ceiling_stream_read_GBps": stream_gbs,
            "ceiling_paged_read_no_math_GBps": rounded / (ms_paged / 1e3) / 1e9}
        result["decode_kv_read"]["metadata_and_write"] = metadata_and_write(w3, g3, rpa, timer, args)
        if args.only == "decode":
            result["roofline"] = roofline_for("decode_kernel", kern3["decode_kernel"][1], w3, w3.name)
        del g3, ws3, out3
        torch.cuda.empty_cache()

    # ---------------- head-dim and block-size variants of the decode batch ----------------
    if args.only in (None, "variants"):
        res = {}
        for D, bs in ((64, 16), (256, 16), (128, 8)):
            wv = decode_variant(D, bs, poison=False)
            gv = setup(wv, torch).write_step_rows()
            db = gv.db
            wsv = workspace_for(wv, rpa, torch)
            outv = torch.empty_like(db.q)
            qslv = gv.meta["query_start_loc"]
            attnv = lambda: rpa.pa_attention(db.q, gv.k_cache, gv.v_cache, db.block_tables, qslv, db.seq_lens,
                                             wv.max_query_len, wv.max_seq_len, wv.scale, out=outv, workspace=wsv)
            msv = timer.time(attnv, max(args.steps, 20), args.warmup)
            kernv = timer.kernels(rpa, attnv, 10)
            kvv = accounting.kv_read_bytes(wv.step.seq_lens, wv.num_kv_heads, wv.head_dim, wv.dtype)
            res[f"D{D}_bs{bs}"] = {
                "GBps": kvv / (msv / 1e3) / 1e9, "frac_hbm_peak": kvv / (msv / 1e3) / 1e9 / HBM_PEAK_GBS,
                "kv_bytes": kvv, "ms_per_call": msv,
                "decode_kernel_GBps": kvv / (kernv["decode_kernel"][1] / 1e3) / 1e9,
                "kernels_ms": {k: round(avg, 5) for k, (n, avg) in kernv.items()}}
            del gv, wsv, outv
            torch.cuda.empty_cache()
        result["decode_variants"] = {
            "workload": "decode batch: 100 seqs x 2001 tokens, 32/32 heads, bf16, at head_dim/block_size "
                        "64/16, 256/16 and 128/8", **res}
        res = {}
        for D, bs in ((64, 16), (256, 16), (128, 8)):
            wp = prefill_variant(D, bs, poison=False)
            gp = setup(wp, torch).write_step_rows()
            db = gp.db
            wsp = workspace_for(wp, rpa, torch)
            outp = torch.empty_like(db.q)
            qslp = gp.meta["query_start_loc"]
            attnp = lambda: rpa.pa_attention(db.q, gp.k_cache, gp.v_cache, db.block_tables, qslp, db.seq_lens,
                                             wp.max_query_len, wp.max_seq_len, wp.scale, out=outp, workspace=wsp)
            msp = timer.time(attnp, max(args.steps, 20), args.warmup)
            kernp = timer.kernels(rpa, attnp, 10)
            flp = accounting.attention_flops(wp.step.query_lens, wp.step.seq_lens, wp.num_q_heads, wp.head_dim)
            res[f"D{D}_bs{bs}"] = {
                "TFLOPs": flp / (msp / 1e3) / 1e12, "flops": flp, "ms_per_call": msp,
                "prefill_kernel_TFLOPs": flp / (kernp["prefill_kernel"][1] / 1e3) / 1e12,
                "kernels_ms": {k: round(avg, 5) for k, (n, avg) in kernp.items()}}
            del gp, wsp, outp
            torch.cuda.empty_cache()
        result["prefill_variants"] = {
            "workload": "ragged prefill: prompts 16/128/1024/2048, 32/32 heads, bf16, at head_dim/block_size "
                        "64/16, 256/16 and 128/8", **res}

    # ---------------- shared-prefix long-context decode ----------------
    if args.only in (None, "shared"):
        w5 = config(5, poison=False)
        g5 = setup(w5, torch).write_step_rows()
        db = g5.db
        ws5 = workspace_for(w5, rpa, torch)
        out5 = torch.empty_like(db.q)
        qsl5 = g5.meta["query_start_loc"]
        attn5 = lambda: rpa.pa_attention(db.q, g5.k_cache, g5.v_cache, db.block_tables, qsl5, db.seq_lens,
                                         w5.max_query_len, w5.max_seq_len, w5.scale, out=out5, workspace=ws5)
        ms5 = timer.time(attn5, max(args.steps, 20), args.warmup)
        cold5 = timer.time_cold(attn5, args.cold_launches)
        kern5 = timer.kernels(rpa, attn5, 10)
        kv5 = accounting.kv_read_bytes(w5.step.seq_lens, w5.num_kv_heads, w5.head_dim, w5.dtype)
        uq5 = accounting.unique_kv_bytes_fast(w5.step.block_tables, w5.step.seq_lens, w5.block_size,
                                              w5.num_kv_heads, w5.head_dim, w5.dtype)
        result["shared_prefix_decode"] = {
            "workload": "64 seqs in 4 groups sharing 16384-token prefixes + 512 private, 64/8 heads, bf16",
            "ms_per_call": ms5, "logical_GBps": kv5 / (ms5 / 1e3) / 1e9, "unique_GBps": uq5 / (ms5 / 1e3) / 1e9,
            "logical_bytes": kv5, "unique_bytes": uq5,
            "kernels_ms": {k: round(avg, 5) for k, (n, avg) in kern5.items()},
            "cold_cache": {**cold5, "logical_GBps": kv5 / (cold5["median_ms"] / 1e3) / 1e9,
                           "unique_GBps": uq5 / (cold5["median_ms"] / 1e3) / 1e9},
            "metadata_and_write": metadata_and_write(w5, g5, rpa, timer, args)}
        del g5, ws5, out5
        torch.cuda.empty_cache()

    # ---------------- speculative-decoding verify batch ----------------
    if args.only in (None, "verify"):
        t0 = time.time()
        w6 = verify_batch(poison=False)
        print(f"[bench] verify batch {w6.summary()} generated in {time.time() - t0:.1f}s", file=sys.stderr,
              flush=True)
        g6 = setup(w6, torch).write_step_rows()
        db = g6.db
        ws6 = workspace_for(w6, rpa, torch)
        out6 = torch.empty_like(db.q)
        qsl6 = g6.meta["query_start_loc"]
        attn6 = lambda: rpa.pa_attention(db.q, g6.k_cache, g6.v_cache, db.block_tables, qsl6, db.seq_lens,
                                         w6.max_query_len, w6.max_seq_len, w6.scale, out=out6, workspace=ws6)
        ms6 = timer.time(attn6, max(args.steps, 20), args.warmup)
        cold6 = timer.time_cold(attn6, args.cold_launches)
        kern6 = timer.kernels(rpa, attn6, 10)
        kv6 = accounting.kv_read_bytes(w6.step.seq_lens, w6.num_kv_heads, w6.head_dim, w6.dtype)
        result["verify_kv_read"] = {
            "workload": "verify batch: 64 seqs, query_len 2..8 over log-uniform 2k..16k contexts, 32/8 heads, "
                        "D 128, bs 16, bf16",
            "tokens": w6.num_tokens, "ms_per_call": ms6, "GBps": kv6 / (ms6 / 1e3) / 1e9,
            "frac_hbm_peak": kv6 / (ms6 / 1e3) / 1e9 / HBM_PEAK_GBS, "kv_bytes": kv6,
            "tokens_per_s": w6.num_tokens / (ms6 / 1e3),
            "cold_cache": {**cold6, "GBps": kv6 / (cold6["median_ms"] / 1e3) / 1e9},
            "kernels_ms": {k: round(avg, 5) for k, (n, avg) in kern6.items()}}
        one6 = "decode_kernel_2t" not in kern6
        split6 = work_split(w6, one6)
        for kname in ("decode_kernel", "decode_kernel_2t"):
            if kname in kern6:
                result["verify_kv_read"][kname + "_GBps"] = split6[kname] / (kern6[kname][1] / 1e3) / 1e9
        if args.only == "verify":
            k6 = "decode_kernel" if one6 else "decode_kernel_2t"
            result["roofline"] = roofline_for(k6, kern6[k6][1], w6, w6.name, one6)
        result["verify_kv_read"]["metadata_and_write"] = metadata_and_write(w6, g6, rpa, timer, args)
        del g6, ws6, out6
        torch.cuda.empty_cache()

    # ---------------- ragged prefill batch: MFMA throughput ----------------
    if args.only in (None, "prefill"):
        w2 = config(2, poison=False)
        g2 = setup(w2, torch).write_step_rows()
        db = g2.db
        out2 = torch.empty_like(db.q)
        ws2 = workspace_for(w2, rpa, torch)
        qsl2 = g2.meta["query_start_loc"]
        attn2 = lambda: rpa.pa_attention(db.q, g2.k_cache, g2.v_cache, db.block_tables, qsl2, db.seq_lens,
                                         w2.max_query_len, w2.max_seq_len, w2.scale, out=out2, workspace=ws2)
        ms2 = timer.time(attn2, max(args.steps, 20), args.warmup)
        cold2 = timer.time_cold(attn2, args.cold_launches)
        kern2 = timer.kernels(rpa, attn2, 10)
        fl2 = accounting.attention_flops(w2.step.query_lens, w2.step.seq_lens, w2.num_q_heads, w2.head_dim)
        tf = fl2 / (ms2 / 1e3) / 1e12
        result["prefill_mfma"] = {
            "workload": "ragged prefill: prompts 16/128/1024/2048 (T=3216), 32/32 heads, D 128, bs 16, bf16",
            "TFLOPs": tf, "frac_bf16_peak": tf / BF16_PEAK_TFLOPS, "flops": fl2, "ms_per_call": ms2,
            "cold_cache": {**cold2, "TFLOPs": fl2 / (cold2["median_ms"] / 1e3) / 1e12},
            "kernels_ms": {k: round(avg, 5) for k, (n, avg) in kern2.items()},
            "prefill_kernel_TFLOPs": fl2 / (kern2["prefill_kernel"][1] / 1e3) / 1e12,
            "mfma_busy": mfma_from_profiles("prefill_kernel", w2.name),
            "metadata_and_write": metadata_and_write(w2, g2, rpa, timer, args)}
        if args.only == "prefill":
            result["roofline"] = roofline_for("prefill_kernel", kern2["prefill_kernel"][1], w2, w2.name)

    # ---------------- block copies: copy-on-write and swap ----------------
    if args.only in (None, "blocks"):
        result["block_copies"] = bench_block_copies(torch, rpa, timer, args)
    print(json.dumps(result), flush=True)


def bench_block_copies(torch, rpa, timer, args):
    """pa_copy_blocks on the mixed batch's pool geometry (block_size 16, 8 KV
    heads, head_dim 128, bf16: 32 KiB per block of K or V): 4096 copy-on-write
    pairs inside one device pool, then 1024 blocks swapped out to a pinned
    host pool and back in.  Bytes = read + write of K and V per pair."""
    import numpy as np
    bs, hkv, d = 16, 8, 128
    nb, n_cow, n_swap = 9216, 4096, 1024
    kc = torch.zeros((nb, bs, hkv, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    block_bytes = bs * hkv * d * 2
    rng = np.random.default_rng(7)
    perm = rng.permutation(nb).astype(np.int32)
    cow = torch.from_numpy(np.stack([perm[:n_cow], perm[n_cow:2 * n_cow]], 1).copy()).cuda()
    ms = timer.time(lambda: rpa.pa_copy_blocks(kc, vc, kc, vc, cow), max(args.steps, 20), args.warmup)
    kern = timer.kernels(rpa, lambda: rpa.pa_copy_blocks(kc, vc, kc, vc, cow), 10)
    cow_bytes = n_cow * 2 * 2 * block_bytes
    hk = torch.empty((n_swap, bs, hkv, d), dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty_like(hk, pin_memory=True)
    out_pairs = torch.from_numpy(np.stack([perm[:n_swap], np.arange(n_swap, dtype=np.int32)], 1).copy()).cuda()
    in_pairs = torch.from_numpy(np.stack([np.arange(n_swap, dtype=np.int32), perm[n_cow:n_cow + n_swap]], 1)
                                .copy()).cuda()
    ms_out = timer.time(lambda: rpa.pa_copy_blocks(kc, vc, hk, hv, out_pairs), 5, 2)
    ms_in = timer.time(lambda: rpa.pa_copy_blocks(hk, hv, kc, vc, in_pairs), 5, 2)
    swap_bytes = n_swap * 2 * block_bytes
    res = {"workload": f"{n_cow} copy-on-write pairs in a {nb}-block pool + {n_swap}-block swap out/in, "
                       "bs 16, 8 KV heads, D 128, bf16",
           "cow_ms": ms, "cow_GBps": cow_bytes / (ms / 1e3) / 1e9,
           "cow_kernel_GBps": cow_bytes / (kern["copy_blocks_kernel"][1] / 1e3) / 1e9,
           "cow_frac_hbm_peak": cow_bytes / (kern["copy_blocks_kernel"][1] / 1e3) / 1e9 / HBM_PEAK_GBS,
           "swap_out_GBps": swap_bytes / (ms_out / 1e3) / 1e9, "swap_in_GBps": swap_bytes / (ms_in / 1e3) / 1e9}
    del kc, vc, hk, hv
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Throughput of the C128 compress-store path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--sweep PATH] [--no-cpu-baseline]

A step is one call of the plain entry point over the whole batch (one kernel
launch; at this size the staged schedule): 16384 boundary tokens (one per
request, position 128k-1, k ~ U{1..64}), each gathering 16 distinct blocks of a
262144-block fp32 state pool (8.59 GB, every block read once per call), then
RMSNorm, UE8M0/E4M3 quantisation, RoPE and the paged insert into a
KV-block-size-64 k_cache.  Inputs are resident in HBM before timing starts.

Prints one JSON line (metric, value = algorithmic GB/s, roofline, cpu_baseline, sweep).
After the timed region, one call through the debug entry point gives the fp32 pooled vectors
for the parity leg (its k_cache bytes must equal the timed calls').  ``sweep`` holds the
metric's token range, cold (a 1 GiB read before each call): decode batches of 1, 128 and 1024
tokens on the decode sweep's pool and the varlen prefill workload, each on the plain entry
point and on the fastest one for that batch (the fan-out up to 128 tokens, the compacted
schedule for prefill; at 1024 tokens the plain entry point is the fastest).
``--sweep PATH`` also writes per-workload JSONL with warm and cold timings and the
oracle's time beside each workload: the C128 decode sweep 1..4096 tokens, the
single-token, decode-batch and varlen-prefill workloads on every entry point
(plain: single pass or staged; fan-out; compacted), and the C4 and indexer compressors
(the indexer with its FP8 and its MXFP4 cache)
(``--sweep-filter REGEX`` keeps matching workloads; ``--mode sweep`` skips the
large-batch line).  ``--mode copy`` times a plain device-to-device copy (the
counter-calibration kernel for rocprofv3); ``--mode read`` times streaming and
window-gather reads, with plain and non-temporal loads (the attainable-bandwidth
reference lines); ``--mode read-small``, ``--mode read-idx`` and ``--mode read-c4`` time pure
reads of the small decode batches' windows and of the indexer's and the C4 compressor's access
patterns beside the kernels; ``--mode read-gather`` times the large batch's window gather over
id orders and launch shapes.
"""

from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("µs/call + achieved HBM GB/s (% peak) for C128 compress-store at 1..16384 tokens")
PEAK_GBS = 8000.0  # MI355X HBM3E peak
# algorithmic bytes per active token: state 128 rows x 4 KiB, 16 block ids, token_to_req +
# kv slot, one RoPE row of 64 fp32, the 584-byte k_cache record
ACTIVE_TOKEN_BYTES = 128 * 1024 * 4 + 64 + 8 + 256 + 584
ANY_TOKEN_BYTES = 8          # positions + slot_mapping, read for every token
CALL_BYTES = 512 * 4         # rms weight
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "c128_staged_16384tok_traffic.txt")
CSRC = os.path.join(ROOT, "paged_kv_cache_fp32_amd", "csrc")
STAGED_MIN_TOKENS = 2048  # the plain entry point's switch to the staged schedule
KERNEL_SOURCES = ("c128_kernel.hip", "c128_schedules.hip", "c128_device.h", "c128_params.h",
                  "c128_launch.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# C4 (ratio 4, 8-row overlapping window): per active token 4 KiB for each window row that
# exists (8, or 4 at position 3: kv half 2 KiB + score half 2 KiB), 4 B per distinct block id
# of the window, token_to_req + kv slot, one RoPE row, the k_cache record
C4_ROW_BYTES = 2 * 512 * 4
C4_TOKEN_BYTES = 8 + 256 + 584


# indexer (head 128, same window): 1 KiB per existing row (kv half 512 B + score half 512 B),
# the 128-byte record and its 4-byte scale
IDX_ROW_BYTES = 2 * 128 * 4
IDX_TOKEN_BYTES = 8 + 256 + 132
# its MXFP4 cache: a 64-byte record and 4 scale bytes instead
IDX_FP4_TOKEN_BYTES = 8 + 256 + 68


def algorithmic_bytes(wl) -> int:
    act = wl.active_mask()
    if getattr(wl, "indexer", False):
        pos = wl.positions[act].astype(np.int64)
        bs = wl.state.shape[1]
        first = np.maximum(pos - 7, 0)
        tok = IDX_FP4_TOKEN_BYTES if getattr(wl, "indexer_fp4", False) else IDX_TOKEN_BYTES
        per = (pos - first + 1) * IDX_ROW_BYTES + (pos // bs - first // bs + 1) * 4 + tok
        return int(per.sum()) + wl.num_tokens * ANY_TOKEN_BYTES + 128 * 4
    if getattr(wl, "compress_ratio", 128) == 4:
        pos = wl.positions[act].astype(np.int64)
        bs = wl.state.shape[1]
        first = np.maximum(pos - 7, 0)
        rows = pos - first + 1
        cols = pos // bs - first // bs + 1
        per = rows * C4_ROW_BYTES + cols * 4 + C4_TOKEN_BYTES
        return int(per.sum()) + wl.num_tokens * ANY_TOKEN_BYTES + CALL_BYTES
    return int(act.sum()) * ACTIVE_TOKEN_BYTES + wl.num_tokens * ANY_TOKEN_BYTES + CALL_BYTES


def code_text(path: str) -> str:
    """A C++ source with its comments and whitespace removed (the sources have no string
    literals that contain comment markers)."""
    import re
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """Hash of the code of the sources the large-batch kernel is built from (the staged
    schedule, its helpers and constants, and the dispatch in the single-pass file); edits to
    comments do not change it."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        h.update(code_text(os.path.join(CSRC, name)).encode())
    return h.hexdigest()[:16]


def measured_traffic(launch_bytes_unused=None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel source (else None)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        line = line.strip()
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Timer:
    """HIP events on the launch stream: one pair around the whole timed region and one pair
    around every launch."""

    def __init__(self, torch, stream, n):
        self.torch = torch
        self.stream = stream
        E = torch.cuda.Event
        self.begin, self.end = E(enable_timing=True), E(enable_timing=True)
        self.starts = [E(enable_timing=True) for _ in range(n)]
        self.stops = [E(enable_timing=True) for _ in range(n)]

    def region_ms(self):
        return self.begin.elapsed_time(self.end)

    def launch_ms(self):
        return [a.elapsed_time(b) for a, b in zip(self.starts, self.stops)]


def time_calls(torch, stream, calls, steps, warmup, flush=None):
    """Run ``calls[i % len(calls)]`` warmup + steps times; returns (region ms, per-launch ms)."""
    for i in range(warmup):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    tm = Timer(torch, stream, steps)
    tm.begin.record(stream)
    for i in range(steps):
        if flush is not None:
            flush()
        tm.starts[i].record(stream)
        calls[i % len(calls)]()
        tm.stops[i].record(stream)
    tm.end.record(stream)
    torch.cuda.synchronize()
    return tm.region_ms(), tm.launch_ms()


def main_line(args):
    import torch

    import paged_kv_cache_fp32_amd as c128
    import synth
    from synth.device import DeviceWorkload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    t0 = time.time()
    wl = synth.config4()
    log(f"[bench] generated {wl.name} in {time.time() - t0:.1f}s")
    d = DeviceWorkload(wl, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs resident on {props.name} ({props.multi_processor_count} CUs)")
    stream = torch.cuda.current_stream(dev)
    sid = stream.cuda_stream

    def call():
        c128.compress_store(*d.args(), stream=sid)

    region_ms, per_launch = time_calls(torch, stream, [call], args.steps, args.warmup)
    nbytes = algorithmic_bytes(wl)
    ms_per_step = region_ms / args.steps
    kernel_ms = float(np.mean(per_launch))
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (kernel_ms * 1e-3) / 1e9
    log(f"[bench] {args.steps} steps: {ms_per_step * 1e3:.1f} us/step, kernel avg "
        f"{kernel_ms * 1e3:.1f} us (min {min(per_launch) * 1e3:.1f}, max "
        f"{max(per_launch) * 1e3:.1f}), {value:.0f} GB/s")
    traffic = measured_traffic()

    body, guards_ok = d.k_cache_bytes()
    # Outside the timed region: one call through the debug entry point, whose fp32 pooled
    # vectors the parity leg checks; its k_cache bytes must equal the timed calls'.
    comp = torch.full((wl.num_tokens, 512), float("nan"), dtype=torch.float32, device=dev)
    c128.compress_store_debug(*d.args(), comp, stream=sid)
    torch.cuda.synchronize()
    body_debug, _ = d.k_cache_bytes()
    comp = comp.cpu().numpy()
    debug_bytes_equal = bool(np.array_equal(body, body_debug))
    del body_debug
    T = wl.num_tokens
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "C128 compress-store, 16384 boundary tokens (one per request, pos 128k-1, "
                        "k~U{1..64}), 16 distinct state blocks each from a 262144x[8,1024] fp32 "
                        "pool (8.59 GB, every block read once per call), KV block size 64",
            "tokens": T,
            "active_tokens": int(wl.active_mask().sum()),
            "algorithmic_bytes_per_call": nbytes,
            "us_per_call": round(ms_per_step * 1e3, 2),
            "compressed_tokens_per_s": round(int(wl.active_mask().sum()) / (ms_per_step * 1e-3)),
            "pct_peak_hbm": round(100.0 * value / PEAK_GBS, 2),
            "device": props.name,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_GBS, 4),
            "traffic": traffic,
            "kernel_avg_us": round(kernel_ms * 1e3, 2),
        },
        "cpu_baseline": None,
    }
    if not guards_ok:
        line["error"] = "k_cache guard bands were written"
    if not debug_bytes_equal:
        line["error"] = "the debug entry point wrote other k_cache bytes than the timed calls"
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, body, nbytes, comp)
    del d, comp
    torch.cuda.empty_cache()
    if not args.no_range:
        line["sweep"] = range_sweep(args)
    if args.sweep:
        sweep(args, args.sweep)
    print(json.dumps(line), flush=True)


def host_cpus() -> int:
    """CPUs this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(wl, gpu_body, nbytes, gpu_compressed=None):
    """The oracle on the host cores, on the same resident host inputs; also checks the GPU
    bytes (and, when given, the GPU's fp32 pooled vectors) of this run against it, outside the
    timer.  Threads: one per visible CPU, at most 16 (a one-GPU share of the host)."""
    import oracle
    import synth
    from oracle.compare import compare

    threads = synth.default_threads()
    t0 = time.perf_counter()
    orc = oracle.run(wl, threads)
    dt = time.perf_counter() - t0
    act = int(wl.active_mask().sum())
    rep = compare(wl, gpu_body, orc, gpu_compressed=gpu_compressed)
    log(f"[bench] oracle: {dt:.2f}s on {threads} threads; parity vs GPU: "
        f"{'ok' if rep.ok() else 'FAIL'} ({rep.summary()})")
    return {
        "value": round(nbytes / dt / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "host_cpus_visible": host_cpus(),
        "kind": "oracle",
        "sample": f"the full workload: all {wl.num_tokens} tokens ({act} active), fp64, "
                  f"{threads} threads",
        "seconds": round(dt, 3),
        "compressed_tokens_per_s": round(act / dt, 1),
        "parity_vs_gpu": "ok" if rep.ok() else "FAIL",
        "parity_detail": {k: rep.get(k) for k in (
            "scale_mismatch", "excused_blocks", "code_diff1_frac", "rope_max_ulp", "rope_band",
            "rope_band_max_use", "compressed_max_ratio")},
    }


def range_sweep(args):
    """The metric's token range in the bench line: cold calls (a 1 GiB read before each one
    evicts the L2s and the MALL) of decode batches of 1, 128 and 1024 tokens on the decode
    sweep's 65536-block pool, of a 1024-request decode step in which one token in 128 closes a
    window, and of the varlen prefill workload, each on the plain entry point and on the fastest
    entry point for that batch; median over the calls, per-call event time on the launch
    stream."""
    import torch

    import paged_kv_cache_fp32_amd as c128
    import synth
    from synth.device import DeviceWorkload

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sid = stream.cuda_stream
    scratch = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    sink = torch.empty((), dtype=torch.float32, device=dev)

    def flush():
        torch.sum(scratch, dim=0, out=sink)

    def entry(dws, kind):
        if kind.startswith("fan-out"):  # "fan-out": automatic split count, "fan-out N": N
            sp = int(kind.split()[1]) if " " in kind else 0
            wss = [c128.fanout_workspace(d.wl.num_tokens, sp, dev) for d in dws]
            return [(lambda d=d, w=w: c128.compress_store_ex(*d.args(), workspace=w, splits=sp,
                                                             stream=sid))
                    for d, w in zip(dws, wss)]
        if kind == "compacted":
            wss = [torch.empty(c128.varlen_workspace_bytes(d.wl.num_tokens), dtype=torch.uint8,
                               device=dev) for d in dws]
            return [(lambda d=d, w=w: c128.compress_store_varlen(*d.args(), workspace=w,
                                                                 stream=sid))
                    for d, w in zip(dws, wss)]
        return [(lambda d=d: c128.compress_store(*d.args(), stream=sid)) for d in dws]

    out = []

    def measure(name, dws, kinds):
        wl = dws[0].wl
        nbytes = algorithmic_bytes(wl)
        for kind in kinds:
            _, per = time_calls(torch, stream, entry(dws, kind), args.range_steps, 3,
                                flush=flush)
            us = float(np.median(per)) * 1e3
            gbs = nbytes / (us * 1e-6) / 1e9
            out.append({"workload": name, "tokens": wl.num_tokens,
                        "active": int(wl.active_mask().sum()), "entry": kind,
                        "us_cold": round(us, 2), "gbs": round(gbs, 1),
                        "frac": round(gbs / PEAK_GBS, 4)})
            log(f"[range] {json.dumps(out[-1])}")

    t0 = time.time()
    _, pool = synth.config3_pool()
    pool_dev = None
    for T, best in ((1, "fan-out"), (128, "fan-out"), (1024, None)):
        dws = []
        for s in range(4):
            d = DeviceWorkload(synth.config3(T, state=pool, window_set=s), device=dev,
                               state=pool_dev)
            pool_dev = (d.state_buf, d.state)
            dws.append(d)
        measure(f"decode T={T}", dws, ["plain"] + ([best] if best else []))
        del dws
    dws = []
    for s in range(4):
        d = DeviceWorkload(synth.decode_step(1024, state=pool, window_set=s), device=dev,
                           state=pool_dev)
        pool_dev = (d.state_buf, d.state)
        dws.append(d)
    measure("decode step T=1024, 1 in 128 active", dws, ["plain", "fan-out 4"])
    del dws
    del pool, pool_dev
    torch.cuda.empty_cache()
    d2 = DeviceWorkload(synth.config2(), device=dev)
    measure("varlen prefill", [d2], ["plain", "compacted"])
    del d2, scratch
    torch.cuda.empty_cache()
    log(f"[range] done in {time.time() - t0:.1f}s")
    return {"mode": "cold, median of per-call event times", "calls": args.range_steps,
            "points": out}


def oracle_timing(wl, nbytes, threads=None):
    """CPU baseline of a sweep workload: the oracle (no diagnostics) on the host cores (or on
    ``threads`` of them), on the same host inputs as the GPU run."""
    import oracle
    import synth

    threads = synth.default_threads() if threads is None else threads
    t0 = time.perf_counter()
    oracle.run(wl, threads, diagnostics=False)
    dt = time.perf_counter() - t0
    return {"kind": "oracle", "cores": threads, "seconds": round(dt, 4),
            "value": round(nbytes / dt / 1e9, 3), "unit": "GB/s",
            "sample": f"the whole workload ({wl.num_tokens} tokens), fp64"}


def sweep(args, path):
    """Per-workload timings (warm: back-to-back calls rotating over disjoint window sets;
    cold: a 1 GiB buffer is read (a sum) before each individually timed call, which evicts the
    256 MiB MALL and the L2s with clean lines)."""
    import torch

    import paged_kv_cache_fp32_amd as c128
    import synth
    from synth.device import DeviceWorkload

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sid = stream.cuda_stream
    scratch = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    sink = torch.empty((), dtype=torch.float32, device=dev)

    def flush():
        torch.sum(scratch, dim=0, out=sink)

    out = open(path, "w")
    cpu_seen = {}  # workload name -> its oracle timing (taken once per workload)

    def make_calls(dws, splits, varlen, st):
        """One call per window set, on stream handle ``st`` (None: torch's current stream, as
        graph capture needs)."""
        kw = {} if st is None else {"stream": st}
        if getattr(dws[0].wl, "indexer_fp4", False):
            return [(lambda d=d: c128.indexer_mxfp4_compress_store(*d.args(), **kw))
                    for d in dws]
        if getattr(dws[0].wl, "indexer", False):
            return [(lambda d=d: c128.indexer_compress_store(*d.args(), **kw)) for d in dws]
        if getattr(dws[0].wl, "compress_ratio", 128) == 4:
            return [(lambda d=d: c128.c4_compress_store(*d.args(), **kw)) for d in dws]
        if varlen:
            wss = [torch.empty(max(16, c128.varlen_workspace_bytes(d.wl.num_tokens)),
                               dtype=torch.uint8, device=dev) for d in dws]
            return [(lambda d=d, w=w: c128.compress_store_varlen(*d.args(), workspace=w, **kw))
                    for d, w in zip(dws, wss)]
        if splits is None:
            return [(lambda d=d: c128.compress_store(*d.args(), **kw)) for d in dws]
        wss = [c128.fanout_workspace(d.wl.num_tokens, splits, dev) for d in dws]
        return [(lambda d=d, w=w: c128.compress_store_ex(*d.args(), workspace=w, splits=splits,
                                                         **kw))
                for d, w in zip(dws, wss)]

    def graph_us_per_call(calls):
        """Per-call time of the calls captured back to back in one graph (at least 32, cycling
        over the window sets), replayed 20 times after 3 untimed replays: what a serving loop
        that captures its decode step pays, without the per-launch host cost."""
        n = max(32, len(calls))
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                calls[i % len(calls)]()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (20 * n)
        del g
        return us

    def measure(name, dws, steps, warm_only=False, splits=None, varlen=False):
        """splits None: the single-pass entry point; else compress_store_ex with that split
        count (0 = automatic) and a workspace per window set; varlen: the compacted schedule
        (compress_store_varlen) with a workspace per window set.  Batches of up to 1024 tokens
        are also timed inside a graph."""
        calls = make_calls(dws, splits, varlen, sid)
        if args.sweep_steps:
            steps = min(steps, args.sweep_steps)
        wl = dws[0].wl
        nbytes = algorithmic_bytes(wl)
        reg, per = time_calls(torch, stream, calls, steps, max(3, len(calls)))
        rec = {"workload": name, "tokens": wl.num_tokens,
               "active_tokens": int(wl.active_mask().sum()), "window_sets": len(dws),
               "entry": ("indexer mxfp4" if getattr(wl, "indexer_fp4", False) else
                         "indexer" if getattr(wl, "indexer", False) else
                         "c4" if getattr(wl, "compress_ratio", 128) == 4 else
                         "varlen (compacted)" if varlen else
                         ("staged" if wl.num_tokens >= STAGED_MIN_TOKENS else "single pass")
                         if splits is None else f"fan-out splits={splits}"),
               "algorithmic_bytes_per_call": nbytes,
               "warm_us_median": round(float(np.median(per)) * 1e3, 2),
               "warm_us_mean": round(float(np.mean(per)) * 1e3, 2)}
        rec["warm_gbs"] = round(nbytes / (rec["warm_us_median"] * 1e-6) / 1e9, 1)
        if not warm_only:
            _, percold = time_calls(torch, stream, calls, min(steps, 50), 2, flush=flush)
            rec["cold_us_median"] = round(float(np.median(percold)) * 1e3, 2)
            rec["cold_gbs"] = round(nbytes / (rec["cold_us_median"] * 1e-6) / 1e9, 1)
        rec["pct_peak_hbm_warm"] = round(100 * rec["warm_gbs"] / PEAK_GBS, 2)
        if wl.num_tokens <= 1024 and not args.sweep_no_graph:
            rec["graph_us_per_call"] = round(graph_us_per_call(make_calls(dws, splits, varlen,
                                                                          None)), 2)
        if not args.no_cpu_baseline:
            if name not in cpu_seen:
                cpu_seen[name] = oracle_timing(wl, nbytes)
                if name.startswith("cfg1"):  # the 128-token batch also on one core
                    cpu_seen[name]["one_core"] = oracle_timing(wl, nbytes, threads=1)
            rec["cpu_baseline"] = cpu_seen[name]
        out.write(json.dumps(rec) + "\n")
        out.flush()
        log(f"[sweep] {json.dumps(rec)}")

    pattern = re.compile(args.sweep_filter) if args.sweep_filter else None
    want = (lambda name: bool(pattern.search(name))) if pattern else (lambda name: True)
    if want("cfg0 single boundary token"):
        d0 = DeviceWorkload(synth.config0(), device=dev)
        measure("cfg0 single boundary token", [d0], 1000)
        measure("cfg0 single boundary token", [d0], 1000, splits=0)
        del d0
    if want("cfg1 decode batch T=128"):
        d1 = DeviceWorkload(synth.config1(), device=dev)
        measure("cfg1 decode batch T=128", [d1], 1000)
        measure("cfg1 decode batch T=128", [d1], 1000, splits=0)
        del d1
    if want("cfg2 varlen prefill"):
        d2 = DeviceWorkload(synth.config2(), device=dev)
        measure("cfg2 varlen prefill", [d2], 1000)
        measure("cfg2 varlen prefill", [d2], 1000, varlen=True)
        del d2
    if want("scattered positions T=262400"):
        d5 = DeviceWorkload(synth.scattered_batch("scattered", 61, 262400, 8, 64, 1024, kv_bs=64,
                                                  kv_blocks=64, cs_rows=8192), device=dev)
        measure("scattered positions T=262400", [d5], 200)
        measure("scattered positions T=262400", [d5], 200, varlen=True)
        del d5
    if want("large chunked prefill T=246933"):
        d6 = DeviceWorkload(synth.large_prefill(), device=dev)
        measure("large chunked prefill T=246933", [d6], 200)
        measure("large chunked prefill T=246933", [d6], 200, varlen=True)
        del d6
    pool = pool_dev = None
    for T in [1 << i for i in range(13)]:
        if not want(f"cfg3 decode sweep T={T}"):
            continue
        if pool is None:
            _, pool = synth.config3_pool()
        n_sets = min(64, 65536 // (16 * T))
        dws = []
        for s in range(n_sets):
            wl = synth.config3(T, state=pool, window_set=s)
            d = DeviceWorkload(wl, device=dev, state=pool_dev)
            pool_dev = (d.state_buf, d.state)
            dws.append(d)
        measure(f"cfg3 decode sweep T={T}", dws, 1000 if T <= 1024 else 100)
        if T in (1, 128, 4096):
            measure(f"cfg3 decode sweep T={T}", dws, 1000 if T <= 1024 else 100, varlen=True)
        if T < 1024:
            for sp in ([0, 2, 4, 8, 16] if args.sweep_splits else [0]):
                measure(f"cfg3 decode sweep T={T}", dws, 1000, splits=sp)
        del dws
    for T in (128, 256, 1024, 2048, 4096):
        if not want(f"decode step T={T}"):
            continue
        if pool is None:
            _, pool = synth.config3_pool()
        dws = []
        for s in range(min(4, 65536 // (16 * T))):
            d = DeviceWorkload(synth.decode_step(T, state=pool, window_set=s), device=dev,
                               state=pool_dev)
            pool_dev = (d.state_buf, d.state)
            dws.append(d)
        measure(f"decode step T={T}", dws, 300)
        for sp in (2, 4, 8):
            measure(f"decode step T={T}", dws, 300, splits=sp)
        measure(f"decode step T={T}", dws, 300, varlen=True)
        del dws
    del pool, pool_dev
    torch.cuda.empty_cache()
    c4_sweep(want, measure, dev)
    indexer_sweep(want, measure, dev)
    indexer_sweep(want, measure, dev, fp4=True)
    out.close()


def c4_slices(wl, T, n_sets):
    """n_sets disjoint T-token slices of a C4 decode batch (each token has its own state
    blocks and kv slot), sharing the pool."""
    import dataclasses
    out = []
    for s in range(n_sets):
        sl = slice(s * T, (s + 1) * T)
        out.append(dataclasses.replace(
            wl, block_table=wl.block_table[sl], token_to_req=np.arange(T, dtype=np.int32),
            positions=wl.positions[sl], slot_mapping=wl.slot_mapping[sl],
            kv_slot_mapping=wl.kv_slot_mapping[sl]))
    return out


def indexer_sweep(want, measure, dev, fp4=False):
    """Indexer compressor: decode batches cut from one 16384-token batch (512 MiB pool), and that
    batch with its kv slots in token order; fp4: the same inputs into the MXFP4 cache."""
    import dataclasses

    import synth
    from synth.device import DeviceWorkload
    sizes = (1, 128, 1024, 4096, 16384)
    kind = "indexer mxfp4" if fp4 else "indexer"
    names = [f"{kind} decode T={T}" for T in sizes]
    seq_name = f"{kind} decode T=16384 seq slots"
    if not any(want(n) for n in names + [seq_name]):
        return
    big = synth.indexer_decode_batch(f"{kind} decode T=16384", 1006, 16384, 16384 * 2, 1024,
                                     512, kv_bs=64, kv_blocks=256, cs_rows=4096, fp4=fp4)
    pool_dev = None
    for T, name in zip(sizes, names):
        if not want(name):
            continue
        dws = []
        for wl in c4_slices(big, T, min(64, 16384 // T)):
            d = DeviceWorkload(wl, device=dev, state=pool_dev)
            pool_dev = (d.state_buf, d.state)
            dws.append(d)
        measure(name, dws, 1000 if T <= 4096 else 400)
        del dws
    if not fp4 and want(seq_name):
        # the same batch with kv slots in token order (token t -> slot t): a cache block's
        # records, and their scales, then come from neighbouring waves
        wl = dataclasses.replace(big, kv_slot_mapping=np.arange(16384, dtype=np.int32))
        measure(seq_name, [DeviceWorkload(wl, device=dev, state=pool_dev)], 400)


def c4_sweep(want, measure, dev):
    """C4 compressor: decode batches cut from one 16384-token batch (2 GiB pool, disjoint
    windows), and a chunked prefill."""
    import synth
    from synth.device import DeviceWorkload
    names = [f"c4 decode T={T}" for T in (1, 16, 128, 1024, 4096, 16384)]
    if any(want(n) for n in names):
        big = synth.c4_decode_batch("c4 decode T=16384", 1005, 16384, 16384 * 2, 1024, 512,
                                    kv_bs=64, kv_blocks=256, cs_rows=4096)
        pool_dev = None
        for T, name in zip((1, 16, 128, 1024, 4096, 16384), names):
            if not want(name):
                continue
            dws = []
            for wl in c4_slices(big, T, min(64, 16384 // T)):
                d = DeviceWorkload(wl, device=dev, state=pool_dev)
                pool_dev = (d.state_buf, d.state)
                dws.append(d)
            measure(name, dws, 1000 if T <= 4096 else 200)
            del dws
        del big, pool_dev
    if want("c4 varlen prefill"):
        wl = synth.c4_varlen_prefill("c4 varlen prefill", 1202, 64, 1024, 4096, kv_bs=64,
                                     cs_rows=8192)
        measure("c4 varlen prefill", [DeviceWorkload(wl, device=dev)], 1000)


def read_line(args):
    """Attainable-bandwidth references on this machine (bench_support probes): a sequential
    streaming read of 4 GiB (grid-stride, best of a few launch shapes), a sequential read of the
    same 4 GiB in contiguous chunks per workgroup (best of 30 shapes), and a read of the 16-block windows
    of the 16384-token workload with the compress kernel's lane mapping but none of its
    arithmetic; each with plain loads and with the non-temporal hint."""
    import ctypes

    import torch

    import bench_support
    import synth
    from synth.device import DeviceWorkload

    L = bench_support.lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sid = stream.cuda_stream
    n = 1 << 30  # floats
    src = torch.ones(n, dtype=torch.float32, device=dev)
    out = torch.empty(1 << 16, dtype=torch.float32, device=dev)
    rec = {"mode": "read", "stream_bytes": 4 * n}
    for nt, tag in ((0, ""), (1, "_nt")):
        best = None
        for blocks, threads in ((1024, 512), (2048, 512), (4096, 256), (8192, 256), (2048, 256)):
            def call(b=blocks, t=threads, nt=nt):
                assert L.probe_stream_read(src.data_ptr(), 4 * n, out.data_ptr(), b, t, nt,
                                           sid) == 0
            _, per = time_calls(torch, stream, [call], args.steps, args.warmup)
            gbs = 4 * n / (float(np.median(per)) * 1e-3) / 1e9
            rec[f"stream{tag}_gbs_{blocks}x{threads}"] = round(gbs, 1)
            best = gbs if best is None else max(best, gbs)
        rec[f"stream{tag}_gbs_best"] = round(best, 1)
    # contiguous chunks per workgroup: grid x threads x loads per lane (chunk = loads*threads*16 B)
    out = torch.empty(1 << 16, dtype=torch.float32, device=dev)
    for nt, tag in ((0, ""), (1, "_nt")):
        best = None
        for blocks in (256, 512, 1024, 2048, 4096):
            for threads in (256, 512):
                for loads in (4, 8, 16):
                    def call(b=blocks, t=threads, u=loads, nt=nt):
                        assert L.probe_stream_chunks(src.data_ptr(), 4 * n, out.data_ptr(), b, t,
                                                     u, nt, sid) == 0
                    _, per = time_calls(torch, stream, [call], args.steps, args.warmup)
                    gbs = 4 * n / (float(np.median(per)) * 1e-3) / 1e9
                    rec[f"chunks{tag}_gbs_{blocks}x{threads}x{loads}"] = round(gbs, 1)
                    if best is None or gbs > best[0]:
                        best = (gbs, f"{blocks}x{threads}x{loads}")
        rec[f"chunks{tag}_gbs_best"] = round(best[0], 1)
        rec[f"chunks{tag}_best_shape"] = best[1]
    del src
    torch.cuda.empty_cache()
    wl = synth.config4()
    d = DeviceWorkload(wl, device=dev)
    T = wl.num_tokens
    pos = wl.positions.astype(np.int64)
    cols = (pos // 128)[:, None] * 16 + np.arange(16)[None, :]
    ids = np.ascontiguousarray(wl.block_table[np.arange(T)[:, None], cols]).astype(np.int32)
    ids_d = torch.from_numpy(ids).to(dev)
    s0 = d.state.stride(0)

    rec["gather_bytes"] = T * 128 * 4096
    for nt, tag in ((0, ""), (1, "_nt")):
        def gather(nt=nt):
            assert L.probe_block_gather_read(d.state.data_ptr(), s0, ids_d.data_ptr(), T,
                                             out.data_ptr(), nt, sid) == 0
        _, per = time_calls(torch, stream, [gather], args.steps, args.warmup)
        ms = float(np.median(per))
        rec[f"gather{tag}_us"] = round(ms * 1e3, 2)
        rec[f"gather{tag}_gbs"] = round(T * 128 * 4096 / (ms * 1e-3) / 1e9, 1)
    print(json.dumps(rec), flush=True)


def read_gather_line(args):
    """The large batch's window gather without arithmetic (the 16384-token workload's 8.59 GB
    pool, non-temporal loads; bench_support probes): the probe with the compress kernel's launch
    shape on the windows' own random block ids, on consecutive ids in pool order and on windows
    of 16 consecutive blocks in random window order; then a persistent grid over 12 launch
    shapes (workgroups x waves x loads in flight per lane) on the windows' own ids.  One JSON
    line per probe: where the gather's ceiling lies, and whether it depends on the ids or on
    the launch shape."""
    import numpy as np
    import torch

    import bench_support
    import synth
    from synth.device import DeviceWorkload

    L = bench_support.lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sid = stream.cuda_stream
    wl = synth.config4()
    d = DeviceWorkload(wl, device=dev)
    T = wl.num_tokens
    nb = d.state.shape[0]
    s0 = d.state.stride(0)
    pos = wl.positions.astype(np.int64)
    cols = (pos // 128)[:, None] * 16 + np.arange(16)[None, :]
    own = np.ascontiguousarray(wl.block_table[np.arange(T)[:, None], cols]).astype(np.int32)
    order = np.random.default_rng(wl.seed).permutation(T).astype(np.int32)
    orders = (("windows' own ids (random)", own),
              ("consecutive ids in pool order", np.arange(T * 16, dtype=np.int32).reshape(T, 16)),
              ("16 consecutive blocks a window, random window order",
               (order[:, None] * 16 + np.arange(16, dtype=np.int32)[None, :]).astype(np.int32)))
    out = torch.empty(1 << 16, dtype=torch.float32, device=dev)
    nbytes = T * 128 * 4096

    def timed(fn):
        _, per = time_calls(torch, stream, [fn], args.steps, args.warmup)
        ms = float(np.median(per))
        return round(ms * 1e3, 1), round(nbytes / (ms * 1e-3) / 1e9, 1)

    ids_dev = {}
    for name, ids in orders:
        assert ids.min() >= 0 and ids.max() < nb
        ids_dev[name] = torch.from_numpy(np.ascontiguousarray(ids)).to(dev)

        def kernel_shape(i=ids_dev[name]):
            assert L.probe_block_gather_read(d.state.data_ptr(), s0, i.data_ptr(), T,
                                             out.data_ptr(), 1, sid) == 0
        us, gbs = timed(kernel_shape)
        print(json.dumps({"mode": "read-gather", "probe": "kernel shape", "ids": name,
                          "us": us, "GBps": gbs}), flush=True)
    i = ids_dev[orders[0][0]]
    for G, W, Ld in ((256, 16, 16), (256, 16, 8), (256, 8, 16), (256, 8, 8), (256, 4, 16),
                     (256, 4, 8), (256, 4, 4), (512, 4, 8), (512, 8, 8), (256, 2, 16),
                     (512, 2, 16), (1024, 4, 8)):
        def persistent(G=G, W=W, Ld=Ld):
            assert L.probe_window_read_persistent(d.state.data_ptr(), s0, i.data_ptr(), T, G, W,
                                                  Ld, out.data_ptr(), sid) == 0
        us, gbs = timed(persistent)
        print(json.dumps({"mode": "read-gather", "probe": "persistent", "ids": orders[0][0],
                          "workgroups": G, "waves": W, "loads_in_flight": Ld,
                          "kib_in_flight_per_workgroup": W * Ld, "us": us, "GBps": gbs}),
              flush=True)


def read_small_line(args):
    """Small decode batches (1, 32, 128 and 256 tokens on the decode sweep's pool): the time of a
    pure read of exactly their windows over every launch shape of the split window-gather probe
    (S workgroups per window, W waves, L loads in flight per lane; bench_support), next to the
    plain entry point and the fan-out on the same windows.  Cold (a 1 GiB read before each call)
    and warm (4 window sets in turn); medians of the per-call event times.  One JSON line per
    batch size."""
    import ctypes

    import torch

    import bench_support
    import paged_kv_cache_fp32_amd as c128
    import synth
    from synth.device import DeviceWorkload

    L = bench_support.lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sid = stream.cuda_stream
    scratch = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    out = torch.empty(1 << 16, dtype=torch.float32, device=dev)

    def med(calls, cold):
        _, per = time_calls(torch, stream, calls, args.steps, args.warmup,
                            flush=(lambda: torch.sum(scratch, dim=0, out=sink)) if cold else None)
        return round(float(np.median(per)) * 1e3, 2)

    _, pool = synth.config3_pool()
    pool_dev = None
    for T in (1, 32, 128, 256):
        dws = []
        for s in range(4):
            d = DeviceWorkload(synth.config3(T, state=pool, window_set=s), device=dev,
                               state=pool_dev)
            pool_dev = (d.state_buf, d.state)
            dws.append(d)
        ids = []
        for d in dws:
            wl = d.wl
            cols = (wl.positions.astype(np.int64) // 128)[:, None] * 16 + np.arange(16)[None, :]
            idv = np.ascontiguousarray(wl.block_table[np.arange(T)[:, None], cols]).astype(np.int32)
            assert idv.min() >= 0 and idv.max() < wl.state.shape[0]
            ids.append(torch.from_numpy(idv).to(dev))
        s0 = dws[0].state.stride(0)
        rec = {"mode": "read-small", "tokens": T, "bytes_per_call": T * 128 * 4096}
        for cold in (False, True):
            tag = "cold" if cold else "warm"
            best = None
            for S in (1, 2, 4, 8):
                for W in (4, 8, 16):
                    for Lf in (4, 8, 16, 32):
                        n = 512 // (S * W)
                        if Lf > n or n % Lf:
                            continue
                        calls = [(lambda i=i, S=S, W=W, Lf=Lf: L.probe_window_read_split(
                            dws[0].state.data_ptr(), s0, i.data_ptr(), T, S, W, Lf,
                            out.data_ptr(), sid)) for i in ids]
                        us = med(calls, cold)
                        rec[f"read_{tag}_us_S{S}W{W}L{Lf}"] = us
                        if best is None or us < best[0]:
                            best = (us, f"S{S}W{W}L{Lf}")
            rec[f"read_{tag}_best_us"], rec[f"read_{tag}_best_shape"] = best
            rec[f"plain_{tag}_us"] = med([(lambda d=d: c128.compress_store(*d.args(), stream=sid))
                                          for d in dws], cold)
            if T <= 128:
                wss = [c128.fanout_workspace(T, 0, dev) for _ in dws]
                rec[f"fanout_{tag}_us"] = med(
                    [(lambda d=d, w=w: c128.compress_store_ex(*d.args(), workspace=w, splits=0,
                                                              stream=sid))
                     for d, w in zip(dws, wss)], cold)
        print(json.dumps(rec), flush=True)
        del dws, ids


def read_pattern_line(args, c4: bool):
    """A neighbouring compressor's 16384-token decode batch (the indexer's, or with ``c4`` the C4
    compressor's) beside read-only probes of its access pattern (bench_support idx_window_read,
    no arithmetic and no record stores): block ids resolved through the block table as the
    kernel resolves them (mode 0), row offsets precomputed on the host (mode 1: one dependent
    round trip less), and no metadata at all (mode 2: token t reads a whole hashed pool block),
    each at 1, 2, 4 and 8 tokens per wave; and a sequential read of about the batch's state bytes
    in contiguous chunks.  Cold (a 1 GiB read before each call) and warm medians of the per-call
    event times."""
    import ctypes

    import torch

    import bench_support
    import paged_kv_cache_fp32_amd as c128
    import synth
    from synth.device import DeviceWorkload

    L = bench_support.lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sid = stream.cuda_stream
    scratch = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    out = torch.empty(1 << 16, dtype=torch.float32, device=dev)

    def med(calls, cold):
        _, per = time_calls(torch, stream, calls, args.steps, args.warmup,
                            flush=(lambda: torch.sum(scratch, dim=0, out=sink)) if cold else None)
        return round(float(np.median(per)) * 1e3, 2)

    if c4:
        wl = synth.c4_decode_batch("c4 decode T=16384", 1005, 16384, 16384 * 2, 1024, 512,
                                   kv_bs=64, kv_blocks=256, cs_rows=4096)
        half, kernel, probe_fn = 512, c128.c4_compress_store, L.probe_c4_window_read
    else:
        wl = synth.indexer_decode_batch("indexer decode T=16384", 1006, 16384, 16384 * 2, 1024,
                                        512, kv_bs=64, kv_blocks=256, cs_rows=4096)
        half, kernel, probe_fn = 128, c128.indexer_compress_store, L.probe_indexer_window_read
    d = DeviceWorkload(wl, device=dev)
    st = d.state
    T = wl.num_tokens
    s0, s1 = st.stride(0), st.stride(1)
    nb = st.shape[0]
    if st.shape[1] != 8 or s1 < 4 * half or not np.array_equal(wl.token_to_req, np.arange(T)):
        raise RuntimeError("the window-read probe expects 8-row state blocks and one token a "
                           "request")
    pos = wl.positions.astype(np.int64)
    q = pos[:, None] - 7 + np.arange(8)[None, :]
    blk = wl.block_table[np.arange(T)[:, None], np.maximum(q, 0) // 8].astype(np.int64)
    offs = np.where(q >= 0, blk * s0 + (q % 8) * s1 + np.where(np.arange(8) >= 4, half, 0), -1)
    span = (nb - 1) * s0 + 7 * s1 + 4 * half
    if offs.max() + 3 * half > span or blk.min() < 0 or blk.max() >= nb or pos.max() >= 4096:
        raise RuntimeError("window-read probe offsets out of range")
    offs_dev = torch.from_numpy(np.ascontiguousarray(offs)).to(dev)
    nb_mask = (1 << (nb.bit_length() - 1)) - 1
    nbytes = algorithmic_bytes(wl)
    seq_floats = (1 << 27) if c4 else (1 << 25)  # 512 MiB / 128 MiB
    seq = torch.ones(seq_floats, dtype=torch.float32, device=dev)

    def probe(kpw):
        return bench_support.IdxProbe(
            st.data_ptr(), s0, s1, d.positions.data_ptr(), d.slot_mapping.data_ptr(),
            d.token_to_req.data_ptr(), d.block_table.data_ptr(), d.block_table.stride(0),
            d.block_table.shape[0], d.block_table.shape[1], nb, offs_dev.data_ptr(),
            d.cos_sin.data_ptr(), d.cos_sin.stride(0), d.cos_sin.shape[0], T, kpw, nb_mask)

    rec = {"mode": "read-c4" if c4 else "read-idx", "tokens": T, "algorithmic_bytes": nbytes,
           "probe_state_bytes": int((offs >= 0).sum()) * 8 * half,
           "seq_bytes": 4 * seq.numel()}
    for cold in (False, True):
        tag = "cold" if cold else "warm"
        rec[f"kernel_{tag}_us"] = med([lambda: kernel(*d.args(), stream=sid)], cold)
        for mode in (0, 1, 2):
            for kpw in (1, 2, 4, 8):
                prm = probe(kpw)

                def call(prm=prm, mode=mode):
                    assert probe_fn(ctypes.byref(prm), mode, out.data_ptr(), sid) == 0
                rec[f"probe{mode}_{tag}_us_kpw{kpw}"] = med([call], cold)
        for blocks, threads, loads in ((256, 256, 8), (512, 256, 4), (1024, 256, 8),
                                       (2048, 256, 4)):
            def call(b=blocks, t=threads, u=loads):
                assert L.probe_stream_chunks(seq.data_ptr(), 4 * seq.numel(), out.data_ptr(),
                                             b, t, u, 1, sid) == 0
            rec[f"seq_{tag}_us_{blocks}x{threads}x{loads}"] = med([call], cold)
        log(f"[{rec['mode']}] {tag} done")
    print(json.dumps(rec), flush=True)


def copy_line(args):
    """Plain device-to-device copy of 4 GiB: the streaming reference and the calibration
    kernel for the HBM counters (reads 4 GiB, writes 4 GiB per launch)."""
    import torch
    dev = torch.device("cuda:0")
    n = 1 << 30  # floats
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream(dev)
    reg, per = time_calls(torch, stream, [lambda: dst.copy_(src)], args.steps, args.warmup)
    ms = float(np.mean(per))
    nbytes = 2 * 4 * n
    print(json.dumps({"mode": "copy", "bytes_read_per_launch": 4 * n,
                      "bytes_written_per_launch": 4 * n, "kernel_avg_us": round(ms * 1e3, 2),
                      "gbs_read_plus_write": round(nbytes / (ms * 1e-3) / 1e9, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sweep", default=None, help="write per-workload JSONL to this path")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-range", action="store_true",
                    help="leave out the cold token-range points (decode 1/128/1024 tokens, a "
                         "1024-request decode step, varlen prefill) of the bench line")
    ap.add_argument("--range-steps", type=int, default=30,
                    help="cold calls per token-range point")
    ap.add_argument("--sweep-filter", default=None,
                    help="only the sweep workloads whose name matches this regular expression")
    ap.add_argument("--sweep-steps", type=int, default=0,
                    help="cap on the timed calls per sweep entry (for counter runs)")
    ap.add_argument("--sweep-no-graph", action="store_true",
                    help="with --sweep: leave out the timing inside a HIP graph (for counter runs)")
    ap.add_argument("--sweep-splits", action="store_true",
                    help="with --sweep: time every fan-out split count, not only the automatic one")
    ap.add_argument("--mode", choices=["main", "copy", "read", "read-small", "read-idx", "read-c4",
                                          "read-gather", "sweep"],
                    default="main",
                    help="main: the large-batch line (plus --sweep if given); sweep: only the "
                         "--sweep workloads; read / copy: bandwidth references and counter "
                         "calibration; read-small: pure reads of small batches' windows over "
                         "launch shapes, beside the entry points; read-gather: the large "
                         "batch's window gather over id orders and launch shapes")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the C128 compress-store path shards by request "
              "with no exchange between GPUs, so one GPU's throughput is the figure. "
              "Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        sys.exit("--steps must be >= 1")
    if args.mode == "copy":
        copy_line(args)
    elif args.mode == "read":
        read_line(args)
    elif args.mode == "read-small":
        read_small_line(args)
    elif args.mode in ("read-idx", "read-c4"):
        read_pattern_line(args, args.mode == "read-c4")
    elif args.mode == "read-gather":
        read_gather_line(args)
    elif args.mode == "sweep":
        if not args.sweep:
            sys.exit("--mode sweep needs --sweep PATH")
        sweep(args, args.sweep)
    else:
        main_line(args)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

A step is one kda_prefill_chunked call over the 8K workload (H=32, d=128,
T=8192, bf16 inputs, fp32 state, checkpoints at {2560, 6144, 8192} written into
a pool of 2 MiB pages): metadata tables, the state-independent chunk products,
the state scan and the fused checkpoint / final-state stores.  The same run
also times the decode step (256 requests x 32 heads, in place through a page
table) and the checkpoint page copies (256 x 2 MiB pages), and reports them
under "decode" and "checkpoint_copy".  Inputs are synthetic (seeded Philox
generators) and resident in HBM before timing starts.

Prints ONE JSON line (see the "roofline" and "cpu_baseline" fields).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/sec (H=32,d=128) + decode GB/s; % MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s

# Algorithmic work per (token, head) of prefill at chunk C=64, d=128, bf16 I/O:
#   bytes: q, k, v, g (4 x d x 2) + beta (2) + o (d x 2) = 1282
#   flops: 4*C*d + 6*d^2 = 131072
# plus 64 KiB per (checkpoint, head) stored.
PREFILL_BYTES_PER_TOKEN_HEAD = 1282
PREFILL_FLOPS_PER_TOKEN_HEAD = 131072


# HBM traffic per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs over this
# script, summarised by --summarize-pmc; valid only while the kernel source
# still hashes to the value recorded with the counters.
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_traffic_prefill8k_decode256_copy256_int8x256.md")
KERNEL_SOURCES = {"kda_prefill_prep": "kda_prefill.hip", "kda_prefill_scan": "kda_prefill.hip",
                  "kda_decode_step": "kda_decode.hip", "kda_page_copy": "kda_copy.hip",
                  "kda_ckpt_quant": "kda_ckpt_int8.hip", "kda_ckpt_dequant": "kda_ckpt_int8.hip",
                  "kda_short_conv": "kda_conv.hip", "kda_short_conv_update": "kda_conv.hip"}
# device kernel symbol -> library launch name
KERNEL_SYMBOLS = {"prep2_kernel": "kda_prefill_prep", "prep_kernel": "kda_prefill_prep",
                  "scan_kernel": "kda_prefill_scan", "decode_kernel": "kda_decode_step",
                  "copy_kernel": "kda_page_copy", "meta_fill_kernel": "kda_meta_fill",
                  "quant_kernel": "kda_ckpt_quant", "dequant_kernel": "kda_ckpt_dequant",
                  "conv_kernel": "kda_short_conv", "conv_update_kernel": "kda_short_conv_update"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(name):
    path = os.path.join(ROOT, "hybrid_prefix_cache_amd", "csrc", name)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def recorded_traffic(kernel):
    """HBM bytes per launch of `kernel` recorded in the counter summary, or None
    when there is none or the kernel source has changed since it was taken."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            text = f.read()
    except OSError:
        return None
    m = re.search(r"^\| " + re.escape(kernel) + r" \| ([0-9a-f]{16}) \| [^|]* \| [^|]* \| ([0-9.e+]+) \|",
                  text, re.M)
    if not m or m.group(1) != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return float(m.group(2))


def summarize_pmc(fetch_dir, write_dir, command):
    """Markdown summary of two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE, in
    KiB per dispatch) of this script.  Each counter is scaled by the factor that
    makes it read the known bytes of the page-copy kernel (256 pages of 2 MiB
    read and written per launch)."""
    def per_kernel(d, counter):
        acc = {}
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    if r["Counter_Name"] != counter:
                        continue
                    sym = r["Kernel_Name"]
                    name = next((v for k, v in KERNEL_SYMBOLS.items() if f"kda::{k}" in sym), None)
                    if name:
                        acc.setdefault(name, []).append(float(r["Counter_Value"]) * 1024.0)
        return {k: sum(v) / len(v) for k, v in acc.items()}
    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    copy_bytes = 256 * (2 << 20)
    kf, kw = copy_bytes / fetch["kda_page_copy"], copy_bytes / write["kda_page_copy"]
    lines = [
        "# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
        "Workloads: prefill 8K x 32 heads x d=128 bf16 with 3 checkpoints; decode 256 requests x",
        "32 heads; page copy 256 x 2 MiB; int8 checkpoint write / restore of 256 pages.  Commands",
        "(from /tmp, TMPDIR=/tmp, R = repository root, OUT = the profiler's output directory):", "",
        "```", *command, "```", "",
        f"Calibration against the page copy (512 MiB read + 512 MiB written per launch): "
        f"FETCH_SIZE x {kf:.3f}, WRITE_SIZE x {kw:.3f}.  Source hash = first 16 hex digits of the",
        "SHA-256 of the kernel's source file when the counters were taken; bench.py reports",
        "`roofline.traffic` only while it still matches.", "",
        "| kernel | source hash | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes per launch (calibrated) |",
        "|---|---|---|---|---|",
    ]
    for name in sorted(set(fetch) & set(write)):
        if name not in KERNEL_SOURCES:
            continue
        b = fetch[name] * kf + write[name] * kw
        lines.append(f"| {name} | {source_hash(KERNEL_SOURCES[name])} | {fetch[name] / 1024:.0f} | "
                     f"{write[name] / 1024:.0f} | {b:.6e} |")
    return "\n".join(lines) + "\n"


UTIL_COUNTERS = ("MfmaUtil", "VALUBusy", "LdsUtil", "MfmaFlopsBF16", "MfmaFlopsF32")


def summarize_util(util_dir, command):
    """Markdown summary of one rocprofv3 --pmc run of this script with the
    derived counters UTIL_COUNTERS (matrix-core busy %, vector ALU busy %, LDS
    busy %, MFMA flops per dispatch), averaged per library kernel."""
    acc = {}
    for path in glob.glob(os.path.join(util_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                sym = r["Kernel_Name"]
                name = next((v for k, v in KERNEL_SYMBOLS.items() if f"kda::{k}" in sym), None)
                if name and r["Counter_Name"] in UTIL_COUNTERS:
                    acc.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    avg = {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in acc.items()}
    lines = [
        "# Matrix-core, vector-ALU and LDS activity per launch (rocprofv3 derived counters)", "",
        "Workloads as in the kernel-trace summary (bench.py --only-core: prefill 8K x 32 heads x d=128",
        "bf16, decode 256 x 32, page copy, int8 checkpoints, verify, short conv).  Commands (from /tmp,",
        "TMPDIR=/tmp, R = repository root, OUT = the profiler's output directory):", "",
        "```", *command, "```", "",
        "MfmaUtil = matrix-core busy cycles / (GPU busy cycles x SIMDs); VALUBusy and LdsUtil likewise",
        "for vector-ALU instruction issue and LDS; MFMA flops = the counter's MOPS x 512 (dense).",
        "The prefill's algorithmic work is 131,072 flop per (token, head), 34.36 GFLOP per 8K x 32-head",
        "call; what the kernels execute on the matrix cores includes the masked halves of the",
        "triangular products and the per-slab repetition of the state products.", "",
        "| kernel | MfmaUtil % | VALUBusy % | LdsUtil % | MFMA bf16 GFLOP | MFMA fp32 GFLOP |",
        "|---|---|---|---|---|---|",
    ]
    for name in sorted(avg):
        d = avg[name]
        g = lambda c: d.get(c, float("nan"))
        lines.append(f"| {name} | {g('MfmaUtil'):.1f} | {g('VALUBusy'):.1f} | {g('LdsUtil'):.1f} | "
                     f"{g('MfmaFlopsBF16') / 1e9:.2f} | {g('MfmaFlopsF32') / 1e9:.2f} |")
    return "\n".join(lines) + "\n"


def summarize_trace(kt_dir, bench_json, command):
    """Markdown summary of a rocprofv3 --kernel-trace --stats run of this script
    (its kernel_stats.csv) next to the HIP-event figures the same run printed
    (its JSON line, saved to a file)."""
    stats = sorted(glob.glob(os.path.join(kt_dir, "**", "*kernel_stats.csv"), recursive=True))
    rows = list(csv.DictReader(open(stats[0]))) if stats else []
    with open(bench_json) as f:
        b = json.loads([ln for ln in f.read().splitlines() if ln.startswith("{")][-1])
    lines = [
        "# Kernel-trace summary: bench.py core workloads (8K prefill, 256x32 decode, 256-page copy,",
        "# int8 checkpoints, verify, short conv and its decode-shaped update)", "",
        "Commands (on an MI355X, from /tmp with TMPDIR=/tmp, R = repository root, OUT = the profiler's",
        "output directory):", "", "```", *command, "```", "",
        "Workloads: prefill H=32, d=128, T=8192, bf16 in / fp32 state, checkpoints {2560, 6144, 8192}, run",
        "as two windows of 64 chunks (two prep and two scan launches per call); decode 256 requests x 32",
        "heads in place; copy 256 x 2 MiB pages; int8 checkpoint write and restore of 256 pages x 32",
        "heads; speculative verify 128 requests x 4 tokens; short conv 8192 x 12288 bf16, width 4; conv",
        "update 256 requests x 12288 channels x 1 token.", "",
        "| Kernel | Calls | Average (us) | Min (us) | Max (us) | Share |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"]
        if len(name) > 60:
            name = name[:57] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f}% |")
    lines += ["", "Same-run HIP-event figures (library event pairs on the launch stream):", ""]
    for k, v in b.get("kernels_diagnostic", {}).items():
        lines.append(f"- {k}: {1e3 * v['avg_ms']:.1f} us per launch, {v['launches_per_call']:.0f} per call")
    r = b["roofline"]
    lines.append(f"- prefill step: {b['ms_per_step'] * 1e3:.0f} us, {b['value'] / 1e6:.2f} M tokens/s; "
                 f"{100 * r['frac']:.1f}% of HBM, {100 * r['frac_mfma_bf16']:.1f}% of bf16 MFMA "
                 f"(this run; the profiler adds a few us per launch)")
    for tag, key in (("decode", "decode"), ("copy", "checkpoint_copy"), ("verify", "verify"),
                     ("conv", "short_conv")):
        d = b.get(key)
        if d:
            lines.append(f"- {tag}: kernel {1e3 * d['kernel_avg_ms']:.1f} us ({d['kernel_gbps']:.0f} GB/s, "
                         f"{100 * d['frac_hbm']:.1f}% of 8 TB/s)")
    d = b.get("checkpoint_int8")
    if d:
        for part in ("write", "restore"):
            p = d[part]
            lines.append(f"- int8 {part}: kernel {1e3 * p['kernel_avg_ms']:.1f} us ({p['kernel_gbps']:.0f} GB/s, "
                         f"{100 * p['frac_hbm']:.1f}% of 8 TB/s)")
    d = b.get("short_conv_decode")
    if d:
        for part in ("update", "short_conv_1tok_seqs"):
            p = d[part]
            lines.append(f"- conv decode ({part}): {1e3 * p['ms_per_call']:.1f} us per call, kernel "
                         f"{1e3 * p['kernel_avg_ms']:.1f} us ({100 * p['frac_hbm']:.1f}% of 8 TB/s)")
    return "\n".join(lines) + "\n"


def to_dev(x, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()


def timed(fn, steps, warmup):
    """Run fn warmup times, then time exactly `steps` calls between two device
    synchronisations (HIP events on the current stream + host clock).  Python's
    cyclic garbage collector is paused over the timed calls, as timeit does: a
    full collection in this process takes ~35 ms of host time, which would
    stall the enqueueing of kernels."""
    import gc
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    gc.collect()
    gc.disable()
    try:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    finally:
        gc.enable()
    return e0.elapsed_time(e1) / 1e3, wall


def kernel_times(K, fn, reps):
    """Average per-launch duration of every library kernel over `reps` calls,
    from HIP events the library records around each launch on its stream."""
    import torch
    torch.cuda.synchronize()
    K.kda_profile_read(reset=True)
    K.kda_profile_enable(True)
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    K.kda_profile_enable(False)
    stats = K.kda_profile_read(reset=True)
    return {name: {"launches": n, "avg_ms": ms / max(n, 1)} for name, (n, ms) in stats.items()}


# Distinct input batches the prefill steps cycle through: repeating one batch
# would let the memory-side cache keep part of a call's inputs for the next
# call, which a stream of new requests does not offer.
PREFILL_INPUT_SETS = 4


def prefill_inputs(G, nsets=PREFILL_INPUT_SETS):
    """The 8K workload's inputs: batch 0 on the host (the CPU baseline's) and
    `nsets` distinct batches (generator streams 0 .. nsets-1) on the device."""
    w = G.PREFILL_8K
    d = G.kda_tokens(w.seed, w.H, w.D, 0, w.T, w.dtype)
    sets = [{k: to_dev(v, w.dtype) for k, v in d.items()}]
    for s in range(1, nsets):
        ds = G.kda_tokens(w.seed, w.H, w.D, 0, w.T, w.dtype, seq_id=s)
        sets.append({k: to_dev(v, w.dtype) for k, v in ds.items()})
    return w, d, sets


def bench_prefill(K, G, steps, warmup, inputs=None):
    import torch
    w, d, sets = inputs or prefill_inputs(G)
    num_pages = 8
    pool_buf = torch.zeros(num_pages * w.page_bytes // 4, dtype=torch.int32, device="cuda")
    pool = K.make_pool(pool_buf, w.page_bytes, num_pages, w.H, w.D)
    o = torch.empty((w.T, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(K.kda_prefill_workspace_bytes(pool, w.T, 1, len(w.ckpts), K.KDA_BF16),
                     dtype=torch.uint8, device="cuda")
    kw = dict(ckpt_cu=[0, len(w.ckpts)], ckpt_pos=list(w.ckpts), ckpt_page=[1, 2, 3],
              state_out_page=[0], workspace=ws)

    it = [0]

    def step():  # one call on the next input batch
        di = sets[it[0] % len(sets)]
        it[0] += 1
        K.kda_prefill_chunked(pool, di["q"], di["k"], di["v"], di["g"], di["beta"], o, [0, w.T], **kw)

    dev_s, wall_s = timed(step, steps, warmup)
    kt = kernel_times(K, step, max(steps, 5))
    graph = bench_graph(step, w.T, steps, warmup, calls=len(sets))
    return w, d, dev_s, wall_s, kt, graph


def bench_graph(step, tokens, steps, warmup, calls=1):
    """`calls` consecutive prefill calls (one per input batch) captured once in
    a HIP graph and replayed: removes the host-side validation and launch
    overhead from the timed loop.  Times are per call."""
    import torch
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(calls):
                step()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(calls):
                step()
        dev_s, _ = timed(g.replay, steps, warmup)
    except Exception as e:  # reported, never hidden
        return {"error": f"{type(e).__name__}: {e}"}
    n = steps * calls
    return {"ms_per_step": 1e3 * dev_s / n, "tokens_per_s": tokens * n / dev_s}


def device_tokens(T, H, D, seed, dtype):
    """q, k, v, g, beta drawn on the device with the generator's distributions
    (q, k unit-norm per (token, head) from N(0,1); v N(0,1); g U[-0.05, 0);
    beta sigmoid(N(0,1))), in slices so fp32 temporaries stay small.  Used where
    host generation would take minutes; the values only feed timing."""
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {n: torch.empty((T, H, D), dtype=td, device="cuda") for n in ("q", "k", "v", "g")}
    out["beta"] = torch.empty((T, H), dtype=td, device="cuda")
    sl = 1 << 16
    for t0 in range(0, T, sl):
        n = min(sl, T - t0)
        for name in ("q", "k"):
            x = torch.randn((n, H, D), generator=gen, device="cuda")
            out[name][t0:t0 + n] = (x / x.norm(dim=-1, keepdim=True)).to(td)
        out["v"][t0:t0 + n] = torch.randn((n, H, D), generator=gen, device="cuda").to(td)
        out["g"][t0:t0 + n] = (torch.rand((n, H, D), generator=gen, device="cuda") * -0.05).to(td)
        out["beta"][t0:t0 + n] = torch.sigmoid(torch.randn((n, H), generator=gen, device="cuda")).to(td)
    return out


def bench_varlen(K, G, steps=20, warmup=3):
    """Suffix prefill of the 16-sequence resume workload: each sequence restarts
    at its 512-multiple boundary B from a state page and runs to its end, all
    16 suffixes packed into one call."""
    import torch
    w = G.VARLEN_RESUME
    lens, bnd = G.varlen_plan(w)
    suf = (lens - bnd).astype(np.int64)
    total = int(suf.sum())
    d = G.kda_tokens(w.seed, w.H, w.D, 0, total, w.dtype)
    di = {k: to_dev(v, w.dtype) for k, v in d.items()}
    del d
    sb = w.H * w.D * w.D * 4
    n = w.n_seqs
    pool_buf = torch.zeros(2 * n * sb // 4, dtype=torch.int32, device="cuda")
    pool = K.make_pool(pool_buf, sb, 2 * n, w.H, w.D)
    o = torch.empty((total, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(K.kda_prefill_workspace_bytes(pool, total, n, 0, K.KDA_BF16), dtype=torch.uint8,
                     device="cuda")
    cu = np.concatenate([[0], np.cumsum(suf)]).astype(np.int64)

    def step():
        K.kda_prefill_chunked(pool, di["q"], di["k"], di["v"], di["g"], di["beta"], o, cu,
                              start_pos=bnd, state_in_page=list(range(n)),
                              state_out_page=list(range(n, 2 * n)), workspace=ws)

    dev_s, _ = timed(step, steps, warmup)
    kt = kernel_times(K, step, steps)
    return {"workload": w.name, "sequences": n, "suffix_tokens": total,
            "ms_per_call": 1e3 * dev_s / steps, "tokens_per_s": total * steps / dev_s,
            "kernels_avg_ms": {k: v["avg_ms"] for k, v in kt.items()}}


def bench_long(K, G, steps=3, warmup=1):
    """One 2^20-token sequence, 32 heads, 171 checkpoints written into the pool."""
    import torch
    w = G.LONG_1M
    di = device_tokens(w.T, w.H, w.D, w.seed, w.dtype)
    npg = len(w.ckpts) + 1
    pool_buf = torch.zeros(npg * w.page_bytes // 4, dtype=torch.int32, device="cuda")
    pool = K.make_pool(pool_buf, w.page_bytes, npg, w.H, w.D)
    o = torch.empty((w.T, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(K.kda_prefill_workspace_bytes(pool, w.T, 1, len(w.ckpts), K.KDA_BF16),
                     dtype=torch.uint8, device="cuda")

    def step():
        K.kda_prefill_chunked(pool, di["q"], di["k"], di["v"], di["g"], di["beta"], o, [0, w.T],
                              ckpt_cu=[0, len(w.ckpts)], ckpt_pos=list(w.ckpts),
                              ckpt_page=list(range(1, npg)), state_out_page=[0], workspace=ws)

    dev_s, _ = timed(step, steps, warmup)
    kt = kernel_times(K, step, steps)
    return {"workload": w.name, "tokens": w.T, "checkpoints": len(w.ckpts),
            "ms_per_call": 1e3 * dev_s / steps, "tokens_per_s": w.T * steps / dev_s,
            "kernels_avg_ms": {k: v["avg_ms"] for k, v in kt.items()},
            "inputs": "drawn on the device (seeded torch generator, the generator's distributions)"}


def bench_decode(K, G, steps=1000, warmup=10):
    """Decode workload: 256 requests x 32 heads, fp32 states in a 512-page pool
    reached through a random page table, one launch per step, `steps`
    consecutive steps each with its own token inputs (drawn on the device with
    the generator's distributions, all resident before timing)."""
    import torch
    w = G.DECODE_256
    pt = torch.from_numpy(G.decode_page_table(w)).cuda()
    pool_buf = torch.zeros(w.pool_pages * w.page_bytes // 4, dtype=torch.int32, device="cuda")
    s0 = G.random_states(w.seed, w.n_req, w.H, w.D)
    words = w.page_bytes // 4
    sb = w.H * w.D * w.D
    for r, p in enumerate(pt.cpu().numpy()):
        pool_buf[p * words:p * words + sb] = torch.from_numpy(s0[r].reshape(-1)).cuda().view(torch.int32)
    pool = K.make_pool(pool_buf, w.page_bytes, w.pool_pages, w.H, w.D)
    n_inputs = steps + warmup
    di = device_tokens(n_inputs * w.n_req, w.H, w.D, w.seed, w.dtype)
    o = torch.empty((w.n_req, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    it = [0]

    def step():
        i = it[0] % n_inputs
        it[0] += 1
        sl = slice(i * w.n_req, (i + 1) * w.n_req)
        K.kda_decode_step(pool, di["q"][sl], di["k"][sl], di["v"][sl], di["g"][sl], di["beta"][sl],
                          o, pt, pt)

    dev_s, wall_s = timed(step, steps, warmup)
    kt = kernel_times(K, step, 50)
    state_bytes = 2 * w.n_req * w.H * w.D * w.D * 4           # read + write
    io_bytes = w.n_req * w.H * (4 * w.D * 2 + 2 + w.D * 2)     # q,k,v,g,beta in; o out
    per_step = state_bytes + io_bytes
    avg = kt["kda_decode_step"]["avg_ms"] / 1e3
    del di
    return {
        "workload": w.name, "steps": steps, "distinct_input_sets": n_inputs,
        "inputs": "drawn on the device (seeded torch generator, the generator's distributions)",
        "ms_per_step": 1e3 * dev_s / steps, "bytes_per_step": per_step,
        "gbps": per_step / (dev_s / steps) / 1e9,
        "frac_hbm_step": per_step / (dev_s / steps) / 1e9 / HBM_PEAK_GBS,
        "kernel_avg_ms": 1e3 * avg, "kernel_gbps": per_step / avg / 1e9,
        "frac_hbm": per_step / avg / 1e9 / HBM_PEAK_GBS,
        "tokens_per_s": w.n_req * steps / dev_s,
    }


def bench_copy(K, steps, warmup):
    import torch
    H, D, page_bytes, n = 32, 128, 2 << 20, 256
    pool_buf = torch.zeros(2 * n * page_bytes // 4, dtype=torch.int32, device="cuda")
    pool = K.make_pool(pool_buf, page_bytes, 2 * n, H, D)
    src, dst = list(range(n)), list(range(n, 2 * n))

    def step():
        K.kda_checkpoint_write(pool, src, dst)

    dev_s, _ = timed(step, steps, warmup)
    kt = kernel_times(K, step, 20)
    moved = 2 * n * H * D * D * 4
    avg = kt["kda_page_copy"]["avg_ms"] / 1e3
    return {"pages": n, "page_bytes": page_bytes, "bytes_per_call": moved,
            "ms_per_call": 1e3 * dev_s / steps, "gbps": moved / (dev_s / steps) / 1e9,
            "kernel_avg_ms": 1e3 * avg, "kernel_gbps": moved / avg / 1e9,
            "frac_hbm": moved / avg / 1e9 / HBM_PEAK_GBS}


def bench_verify(K, G, steps=20, warmup=5, n=128, ntok=4):
    """Speculative verification: 4 draft tokens for each of 128 requests x 32
    heads in one launch, every intermediate state written to its own page."""
    import torch
    H, D = 32, 128
    sb = H * D * D * 4
    pool_buf = torch.randn((n + n * ntok) * sb // 4, device="cuda") / np.sqrt(D)
    pool = K.make_pool(pool_buf, sb, n + n * ntok, H, D)
    d = G.kda_tokens(0x4B44416, H, D, 0, n * ntok, "bf16")
    di = {k: to_dev(v, "bf16") for k, v in d.items()}
    o = torch.empty((n * ntok, H, D), dtype=torch.bfloat16, device="cuda")
    pin = torch.arange(n, dtype=torch.int32, device="cuda")
    pout = torch.arange(n, n + n * ntok, dtype=torch.int32, device="cuda")

    def step():
        K.kda_decode_verify(pool, di["q"], di["k"], di["v"], di["g"], di["beta"], o, ntok, pin, pout)

    dev_s, _ = timed(step, steps, warmup)
    kt = kernel_times(K, step, steps)
    moved = n * H * (D * D * 4 * (1 + ntok) + ntok * (4 * D * 2 + 2 + D * 2))
    avg = kt["kda_decode_verify"]["avg_ms"] / 1e3
    return {"requests": n, "tokens_per_request": ntok, "bytes_per_call": moved,
            "ms_per_call": 1e3 * dev_s / steps, "kernel_avg_ms": 1e3 * avg,
            "kernel_gbps": moved / avg / 1e9, "frac_hbm": moved / avg / 1e9 / HBM_PEAK_GBS,
            "tokens_per_s": n * ntok * steps / dev_s}


def bench_int8(K, steps=20, warmup=10):
    """int8 compressed checkpoints: quantise 256 active pages (32 heads, d=128)
    into a compressed pool, and dequantise them back into fp32 pages.  Calls
    cycle through three sets of source pages (1.5 GiB of fp32 pages, 415 MB of
    compressed ones), so that no call reads what the previous call left in
    the memory-side cache."""
    import torch
    H, D, n, R = 32, 128, 256, 3
    sb = H * D * D * 4
    pool_buf = torch.randn((R + 1) * n * sb // 4, device="cuda") / np.sqrt(D)
    pool = K.make_pool(pool_buf, sb, (R + 1) * n, H, D)
    hb = K.kda_ckpt_int8_head_bytes(D, D)
    qpb = (H * hb + 255) // 256 * 256
    qbuf = torch.zeros(R * n * qpb, dtype=torch.uint8, device="cuda")  # touched before timing
    qpool = K.make_pool(qbuf, qpb, R * n, H, D)
    sets = [list(range(r * n, (r + 1) * n)) for r in range(R)]
    dst = list(range(R * n, (R + 1) * n))
    for r in range(R):  # every compressed set holds real checkpoints before the restores
        K.kda_checkpoint_write_int8(pool, sets[r], qpool, sets[r])
    it = [0]

    def write():
        r = it[0] % R
        it[0] += 1
        K.kda_checkpoint_write_int8(pool, sets[r], qpool, sets[r])

    def restore():
        r = it[0] % R
        it[0] += 1
        K.kda_checkpoint_restore_int8(qpool, sets[r], pool, dst)
    out = {"pages": n, "page_bytes": sb, "compressed_page_bytes": H * hb, "source_sets": R}
    for name, fn, kern in (("write", write, "kda_ckpt_quant"), ("restore", restore, "kda_ckpt_dequant")):
        dev_s, _ = timed(fn, steps, warmup)
        kt = kernel_times(K, fn, steps)
        moved = n * (sb + H * hb)  # fp32 page one way, compressed page the other
        avg = kt[kern]["avg_ms"] / 1e3
        out[name] = {"ms_per_call": 1e3 * dev_s / steps, "bytes_per_call": moved,
                     "kernel_avg_ms": 1e3 * avg, "kernel_gbps": moved / avg / 1e9,
                     "frac_hbm": moved / avg / 1e9 / HBM_PEAK_GBS}
    return out


def bench_conv(K, G, steps=20, warmup=5, T=8192, C=3 * 32 * 128, W=4):
    """Short causal convolution (width 4) over the fused q|k|v projection of
    the 8192-token prefill (3 x 32 heads x 128 channels per token, bf16, one
    call), with the window checkpointed at every 512-token boundary and a
    final window page."""
    import torch
    # three distinct input batches (600 MB together, more than the memory-side
    # cache holds), so that no call finds the previous call's input cached
    xs = [to_dev(G.conv_inputs(11 + s, T, C, "bf16"), "bf16") for s in range(3)]
    wt = torch.from_numpy(G.conv_weights(11, C, W)).cuda()
    y = torch.empty(T, C, dtype=torch.bfloat16, device="cuda")
    P = list(range(512, T + 1, 512))
    win = (W - 1) * C * 2
    pb = (win + 255) // 256 * 256
    cbuf = torch.zeros((len(P) + 1) * pb, dtype=torch.uint8, device="cuda")
    cpool = K.make_conv_pool(cbuf, pb, len(P) + 1, C, W, K.KDA_BF16)
    wsb = torch.empty(K.kda_conv_workspace_bytes(1, len(P)), dtype=torch.uint8, device="cuda")

    it = [0]

    def step():
        x = xs[it[0] % len(xs)]
        it[0] += 1
        K.kda_short_conv(cpool, x, wt, y, [0, T], state_out_page=[0], ckpt_cu=[0, len(P)],
                         ckpt_pos=P, ckpt_page=list(range(1, 1 + len(P))), workspace=wsb)
    dev_s, _ = timed(step, steps, warmup)
    kt = kernel_times(K, step, steps)
    moved = 2 * T * C * 2 + (len(P) + 1) * win + C * W * 4  # x in, y out, windows, taps
    avg = kt["kda_short_conv"]["avg_ms"] / 1e3
    return {"T": T, "channels": C, "width": W, "checkpoints": len(P),
            "ms_per_call": 1e3 * dev_s / steps, "bytes_per_call": moved,
            "kernel_avg_ms": 1e3 * avg, "kernel_gbps": moved / avg / 1e9,
            "frac_hbm": moved / avg / 1e9 / HBM_PEAK_GBS}


def bench_conv_decode(K, G, steps=200, warmup=10, n=256, C=3 * 32 * 128, W=4):
    """The decode-step conv update: 256 requests x one token over the fused
    q|k|v channels (12,288, bf16), width 4, each request reading its window
    page and writing the next one (pages alternate between steps).  Timed
    through kda_short_conv_update (device page tables) and, for comparison,
    through kda_short_conv with 256 one-token sequences (host tables)."""
    import torch
    x = to_dev(G.conv_inputs(12, n, C, "bf16"), "bf16")
    wt = torch.from_numpy(G.conv_weights(12, C, W)).cuda()
    y = torch.empty(n, C, dtype=torch.bfloat16, device="cuda")
    win = (W - 1) * C * 2
    pb = (win + 255) // 256 * 256
    cbuf = torch.zeros(2 * n * pb, dtype=torch.uint8, device="cuda")
    cpool = K.make_conv_pool(cbuf, pb, 2 * n, C, W, K.KDA_BF16)
    wsb = torch.empty(K.kda_conv_workspace_bytes(n, 0), dtype=torch.uint8, device="cuda")
    cu = np.arange(n + 1, dtype=np.int64)
    pages = [list(range(n)), list(range(n, 2 * n))]
    dpages = [torch.tensor(p, dtype=torch.int32, device="cuda") for p in pages]
    moved = n * (2 * C * 2 + 2 * win) + C * W * 4  # x in, y out, window in and out, taps
    it = [0]

    def step_update():
        t = it[0]
        it[0] += 1
        K.kda_short_conv_update(cpool, x, wt, y, dpages[t % 2], dpages[(t + 1) % 2])

    def step_tables():
        t = it[0]
        it[0] += 1
        K.kda_short_conv(cpool, x, wt, y, cu, start_pos=[100 + t] * n, state_in_page=pages[t % 2],
                         state_out_page=pages[(t + 1) % 2], workspace=wsb)
    out = {"requests": n, "channels": C, "width": W, "tokens_per_request": 1, "bytes_per_call": moved}
    for name, fn, kern in (("update", step_update, "kda_short_conv_update"),
                           ("short_conv_1tok_seqs", step_tables, "kda_short_conv")):
        dev_s, _ = timed(fn, steps, warmup)
        kt = kernel_times(K, fn, steps)
        avg = kt[kern]["avg_ms"] / 1e3
        out[name] = {"ms_per_call": 1e3 * dev_s / steps, "kernel_avg_ms": 1e3 * avg,
                     "kernel_gbps": moved / avg / 1e9, "frac_hbm": moved / avg / 1e9 / HBM_PEAK_GBS,
                     "frac_hbm_call": moved / (dev_s / steps) / 1e9 / HBM_PEAK_GBS}
    return out


def index_workload(G, pb=6144):
    """Token streams of the prefix-index workload: a 2^20-token session, 64
    agentic sessions of 32,768 tokens sharing a 4096-token system prompt, and
    one request per session diverging at a random point (plus one diverging
    from the long session at 900,000 tokens)."""
    long_t = G.token_ids(21, 1 << 20)
    system = G.token_ids(22, 4096)
    sessions = [np.concatenate([system, G.token_ids(23, 32768 - 4096, seq_id=s)]) for s in range(64)]
    rng = np.random.default_rng(5)
    cuts = rng.integers(4096, 32768, 64)
    reqs = [np.concatenate([sessions[i][:cuts[i]], G.token_ids(25, 500, seq_id=i)]) for i in range(64)]
    req_long = np.concatenate([long_t[:900_000], G.token_ids(24, 1000)])
    # whole 6144-token pages match, then the deepest 4096-multiple checkpoint
    expect = [int(c) // pb * pb // 4096 * 4096 for c in cuts]
    return dict(long_t=long_t, sessions=sessions, reqs=reqs, req_long=req_long, expect=expect)


def bench_index(K, G, reps=100):
    """Host prefix index (no GPU): a 2^20-token session in 6144-token pages with
    a checkpoint every 6144 tokens in 2 KDA groups, plus 64 agentic sessions of
    32,768 tokens sharing a 4096-token system prompt (a checkpoint every 4096
    tokens).  Timed: lookup + pin + release of the long session diverging at
    900,000 tokens, and of each short session diverging at a random point; every
    boundary is checked against the closed form of the workload."""
    hb, pb, groups = 512, 6144, 2
    wl = index_workload(G, pb)
    idx = K.kda_index_create(hb, pb, groups, namespace_seed=1)
    ck = [1_000_000]

    def add(t, every, page0):
        npg = -(-len(t) // pb)
        K.kda_index_register_pages(idx, t, list(range(page0, page0 + npg)))
        for b in range(every, len(t) + 1, every):
            for g in range(groups):
                ck[0] += 1
                K.kda_index_register_ckpt(idx, t, b, g, ck[0], durable=True)
        return page0 + npg

    page = add(wl["long_t"], pb, 0)
    for t in wl["sessions"]:
        page = add(t, 4096, page)
    K.kda_index_mark_ready(idx, 0)

    def one(r):
        h = K.kda_index_lookup(idx, r, pin=True)
        if h["pin_handle"]:
            K.kda_index_release(idx, h["pin_handle"])
        return h
    hl = one(wl["req_long"])
    assert hl["boundary"] == 900_000 // pb * pb
    for r, e in zip(wl["reqs"], wl["expect"]):
        assert one(r)["boundary"] == e
    t0 = time.perf_counter()
    for _ in range(reps):
        one(wl["req_long"])
    t_long = (time.perf_counter() - t0) / reps
    t0 = time.perf_counter()
    for _ in range(reps // 10):
        for r in wl["reqs"]:
            one(r)
    t_short = (time.perf_counter() - t0) / (reps // 10 * len(wl["reqs"]))
    n_long = len(wl["req_long"])
    stats = K.kda_index_stats(idx)[:2]
    K.kda_index_destroy(idx)
    return {"long_1m": {"tokens": n_long, "boundary": hl["boundary"], "pages": len(hl["pages"]),
                        "ms_per_lookup": 1e3 * t_long,
                        "hashed_gb_per_s": n_long * 4 / t_long / 1e9},
            "sessions_32k": {"us_per_lookup": 1e6 * t_short, "lookups_per_s": 1.0 / t_short},
            "entries": stats}


def cpu_index_oracle(G, n=8):
    """The prefix-index oracle (token-prefix comparison, no hashing) on the first
    n sessions of the index workload: registration excluded, lookups timed, each
    boundary checked against the workload's closed form."""
    from oracle.prefix_index import PrefixIndexModel
    hb, pb, groups = 512, 6144, 2
    wl = index_workload(G, pb)
    model = PrefixIndexModel(hb, pb, groups)
    ck, page = 1_000_000, 0
    for t in wl["sessions"][:n]:
        npg = -(-len(t) // pb)
        model.register_pages(t, list(range(page, page + npg)), 0)
        page += npg
        for b in range(4096, len(t) + 1, 4096):
            for g in range(groups):
                ck += 1
                model.register_ckpt(t, b, g, ck, True, 0)
    model.mark_ready(0)
    t0 = time.perf_counter()
    for r, e in zip(wl["reqs"][:n], wl["expect"][:n]):
        assert model.lookup(r)["boundary"] == e
    el = (time.perf_counter() - t0) / n
    return {"value": 1.0 / el, "unit": "lookups/s", "ms_per_lookup": 1e3 * el, "cores": 1,
            "kind": "oracle", "sample": f"{n} of the 64 agentic 32K-token sessions"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(G, w, d):
    """The fp64 oracle on the same 8K workload (all 32 heads, all tokens), timed on
    this host's cores.  Generation is excluded."""
    import oracle
    # the host's CPU share (the scheduler affinity / OMP setting), not the machine total
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    # whole-workload runs repeated for about 3 s of wall time (one run is ~0.15 s)
    runs, el = 0, 0.0
    while el < 3.0 and runs < 50:
        t0 = time.perf_counter()
        oracle.run(d["q"], d["k"], d["v"], d["g"], d["beta"], [0, w.T], ckpt_cu=[0, len(w.ckpts)],
                   ckpt_pos=list(w.ckpts), threads=threads)
        el += time.perf_counter() - t0
        runs += 1
    return {"value": w.T * runs / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"whole workload ({w.T} tokens x {w.H} heads, fp64 token loop, OpenMP over "
                      f"heads), {runs} runs in {el:.2f} s"}


def rocminfo_gpu_facts():
    """Lines of `rocminfo` that describe the first GPU agent (name, compute
    units, clock, SIMDs, wave size, caches), or an explanation if it fails."""
    import subprocess
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError) as e:
        return [f"rocminfo unavailable: {e}"]
    keys = ("Marketing Name", "Compute Unit", "Max Clock Freq", "SIMDs per CU", "Wavefront Size",
            "Max Waves Per CU", "L1", "L2", "L3", "Workgroup Max Size:")
    facts, in_gpu = [], False
    for line in txt.splitlines():
        t = line.strip()
        if t.startswith("Name:") and "gfx" in t:
            if in_gpu:
                break  # the second GPU agent
            in_gpu = True
            facts.append(t)
            continue
        if in_gpu and t.startswith("Agent "):
            break
        if in_gpu and any(t.startswith(k) for k in keys):
            facts.append(" ".join(t.split()))
    return facts or ["no GPU agent found in rocminfo output"]


def measure_peaks(reps=10):
    """Measured counterparts of the roofline denominators: a copy and a fill of
    1 GiB (libkda_probe.so and torch's own kernels) and a loop of independent
    bf16 MFMAs on every CU, each the median of `reps` launches timed with HIP
    events."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "hybrid_prefix_cache_amd", "libkda_probe.so"))
    lib.kda_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.kda_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.kda_probe_fill.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p]
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def median_ms(launch):
        assert launch() == 0
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            assert launch() == 0
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    blocks, iters = 8 * cus, 20000
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    t_mfma = median_ms(lambda: lib.kda_probe_mfma_bf16(out.data_ptr(), blocks, iters, st))
    flops = blocks * 4 * iters * 16 * 16384
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    t_fill = median_ms(lambda: lib.kda_probe_fill(dst.data_ptr(), nbytes, 0x3F800000, st))
    t_copy = median_ms(lambda: lib.kda_probe_copy(dst.data_ptr(), src.data_ptr(), nbytes, st))
    assert torch.equal(dst[-4096:], src[-4096:])

    def torch_ms(fn):  # the same operations through torch's own kernels
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))
    t_tcopy = torch_ms(lambda: dst.copy_(src))
    t_tfill = torch_ms(lambda: dst.fill_(7))
    return {
        "device": props.name, "compute_units": cus, "hbm_bytes": props.total_memory,
        "rocminfo": rocminfo_gpu_facts(),
        "mfma_bf16_tflops": flops / (t_mfma / 1e3) / 1e12, "mfma_ms": t_mfma, "mfma_flop": flops,
        "copy_gbps": 2 * nbytes / (t_copy / 1e3) / 1e9, "copy_ms": t_copy,
        "fill_gbps": nbytes / (t_fill / 1e3) / 1e9, "fill_ms": t_fill,
        "torch_copy_gbps": 2 * nbytes / (t_tcopy / 1e3) / 1e9, "torch_copy_ms": t_tcopy,
        "torch_fill_gbps": nbytes / (t_tfill / 1e3) / 1e9, "torch_fill_ms": t_tfill,
    }


def summarize_peaks(p, cmd):
    """Markdown summary of measure_peaks() against the published peaks."""
    lines = ["# MI355X: device facts and measured peaks next to the published ones", "",
             f"Command (repository root, one GPU): `{cmd}`", "",
             "The benchmark's roofline fractions use the published peaks (HBM 8 TB/s, dense bf16",
             "MFMA 2.5 PFLOP/s); these probes show what simple kernels reach on the same part.", "",
             "| probe | measured | published peak | fraction |", "|---|---|---|---|",
             f"| bf16 MFMA loop ({p['mfma_flop'] / 1e12:.1f} TFLOP: 8 workgroups of 4 waves per CU, 16 "
             f"independent v_mfma_f32_16x16x32_bf16 chains per wave) | {p['mfma_bf16_tflops']:.0f} TFLOP/s "
             f"({p['mfma_ms']:.2f} ms) | {BF16_PEAK_TFLOPS:.0f} TFLOP/s | "
             f"{p['mfma_bf16_tflops'] / BF16_PEAK_TFLOPS:.3f} |",
             f"| copy, 1 GiB (read + write counted; one 16-byte non-temporal vector per thread) | "
             f"{p['copy_gbps']:.0f} GB/s ({p['copy_ms']:.3f} ms) | {HBM_PEAK_GBS:.0f} GB/s | "
             f"{p['copy_gbps'] / HBM_PEAK_GBS:.3f} |",
             f"| fill, 1 GiB (same shape) | {p['fill_gbps']:.0f} GB/s ({p['fill_ms']:.3f} ms) | "
             f"{HBM_PEAK_GBS:.0f} GB/s | {p['fill_gbps'] / HBM_PEAK_GBS:.3f} |",
             f"| torch `copy_`, 1 GiB (read + write counted) | {p['torch_copy_gbps']:.0f} GB/s "
             f"({p['torch_copy_ms']:.3f} ms) | {HBM_PEAK_GBS:.0f} GB/s | "
             f"{p['torch_copy_gbps'] / HBM_PEAK_GBS:.3f} |",
             f"| torch `fill_`, 1 GiB | {p['torch_fill_gbps']:.0f} GB/s ({p['torch_fill_ms']:.3f} ms) | "
             f"{HBM_PEAK_GBS:.0f} GB/s | {p['torch_fill_gbps'] / HBM_PEAK_GBS:.3f} |", "",
             f"Device: {p['device']}, {p['compute_units']} compute units, "
             f"{p['hbm_bytes'] / 2**30:.0f} GiB of device memory.", "", "rocminfo (first GPU agent):", ""]
    lines += [f"    {x}" for x in p["rocminfo"]]
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--only-prefill", action="store_true")
    ap.add_argument("--only-core", action="store_true",
                    help="skip the resume and 2^20-token workloads (profiling runs: one prefill shape)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the markdown traffic summary of two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("KT_DIR", "BENCH_JSON"),
                    help="print the markdown summary of a rocprofv3 --kernel-trace --stats run and exit")
    ap.add_argument("--summarize-util", metavar="UTIL_DIR",
                    help="print the markdown summary of a rocprofv3 --pmc run of UTIL_COUNTERS and exit")
    ap.add_argument("--peaks", action="store_true",
                    help="print device facts and measured copy / fill / bf16 MFMA peaks (markdown) and exit")
    args = ap.parse_args()
    if args.peaks:
        import torch
        assert torch.cuda.is_available(), "--peaks needs a GPU"
        sys.stdout.write(summarize_peaks(measure_peaks(), "python3 bench.py --peaks"))
        return
    if args.summarize_trace:
        cmd = ["rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/kt -o run -- "
               "python3 $R/bench.py --steps 20 --warmup 2 --no-cpu --only-core > $OUT/kt_bench.json",
               "python3 $R/bench.py --summarize-trace $OUT/kt $OUT/kt_bench.json"]
        sys.stdout.write(summarize_trace(*args.summarize_trace, cmd))
        return
    if args.summarize_util:
        cmd = [f"rocprofv3 --pmc {' '.join(UTIL_COUNTERS)} --output-format csv -d $OUT/pmc_util "
               f"-o run -- python3 $R/bench.py --steps 3 --warmup 1 --no-cpu --only-core",
               "python3 $R/bench.py --summarize-util $OUT/pmc_util"]
        sys.stdout.write(summarize_util(args.summarize_util, cmd))
        return
    if args.summarize_pmc:
        cmd = [f"rocprofv3 --pmc {c} --output-format csv -d $OUT/{d} -o run -- "
               f"python3 $R/bench.py --steps 3 --warmup 1 --no-cpu --only-core"
               for c, d in (("FETCH_SIZE", "pmc_fetch"), ("WRITE_SIZE", "pmc_write"))]
        cmd.append("python3 $R/bench.py --summarize-pmc $OUT/pmc_fetch $OUT/pmc_write")
        sys.stdout.write(summarize_pmc(*args.summarize_pmc, cmd))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this library has no multi-GPU path (asked for "
              f"--gpus {args.gpus}); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import hybrid_prefix_cache_amd as K
    import kda_inputs as G
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    # The GPU legs run first and the prefill right after them, with its
    # inputs already on the device, so that it is not timed on a GPU that is
    # just leaving its idle state (on one box, timed first, its first ~80
    # calls drifted from 261 to 277 and back to 255 us; after the decode leg
    # they ran at 252-254 us from the first call).  Its own W warm-up and K
    # timed calls are unchanged.
    log("prefill: generating inputs")
    pre_in = prefill_inputs(G)
    legs = {}
    if not args.only_prefill:
        log("decode: 256 requests x 32 heads")
        legs["decode"] = bench_decode(K, G)
        torch.cuda.empty_cache()
        log(f"decode: {legs['decode']}")
        legs["checkpoint_copy"] = bench_copy(K, steps=20, warmup=3)
        log(f"copy: {legs['checkpoint_copy']}")
        legs["checkpoint_int8"] = bench_int8(K)
        log(f"int8: {legs['checkpoint_int8']}")
        legs["verify"] = bench_verify(K, G)
        log(f"verify: {legs['verify']}")
        legs["short_conv"] = bench_conv(K, G)
        log(f"conv: {legs['short_conv']}")
        legs["short_conv_decode"] = bench_conv_decode(K, G)
        log(f"conv decode: {legs['short_conv_decode']}")
        torch.cuda.empty_cache()

    w, d, dev_s, wall_s, kt, graph = bench_prefill(K, G, args.steps, args.warmup, pre_in)
    del pre_in
    ms_step = 1e3 * dev_s / args.steps
    tok_s = w.T * args.steps / dev_s
    log(f"prefill: {ms_step:.3f} ms/step, {tok_s / 1e6:.2f} M tokens/s; kernels {kt}")

    # Roofline of the call (the whole hot path: prep and scan of every window,
    # metadata, checkpoint and final-state stores), counted as the method's
    # algorithmic work: 1282 B and 131072 flop per (token, head), plus 64 KiB
    # per (checkpoint, head) and per (final state, head); over the step time
    # measured with HIP events on the stream the library launches on.
    th = w.T * w.H
    ck_bytes = len(w.ckpts) * w.H * w.D * w.D * 4 + w.H * w.D * w.D * 4  # checkpoints + final state
    call_bytes = th * PREFILL_BYTES_PER_TOKEN_HEAD + ck_bytes
    call_flops = th * PREFILL_FLOPS_PER_TOKEN_HEAD
    step_s = dev_s / args.steps
    reps = max(args.steps, 5)
    per_call = {n: v["launches"] / reps for n, v in kt.items()}
    traffic = None
    tr = {n: recorded_traffic(n) for n in ("kda_prefill_prep", "kda_prefill_scan")}
    if all(v is not None for v in tr.values()):
        traffic = sum(tr[n] * per_call.get(n, 0) for n in tr)
    achieved = call_bytes / step_s / 1e9
    out = {
        "metric": METRIC, "value": tok_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "H": w.H, "d": w.D, "T": w.T, "chunk": 64,
                   "checkpoints": list(w.ckpts), "page_bytes": w.page_bytes,
                   "state_dtype": "f32", "io_dtype": "bf16",
                   "input_batches": PREFILL_INPUT_SETS},
        "roofline": {"bound": "hbm", "kernel": "kda_prefill_chunked (whole call: prep + scan per window)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_call": call_bytes, "step_ms": 1e3 * step_s,
                     "frac_mfma_bf16": call_flops / step_s / 1e12 / BF16_PEAK_TFLOPS,
                     "frac_attainable": max(call_flops / (BF16_PEAK_TFLOPS * 1e12),
                                            call_bytes / (HBM_PEAK_GBS * 1e9)) / step_s,
                     "algorithmic_flops_per_call": call_flops},
        "kernels_diagnostic": {n: {"launches_per_call": per_call[n], "avg_ms": v["avg_ms"],
                                   "ms_per_call": v["avg_ms"] * per_call[n]} for n, v in kt.items()},
        "prefill_wall_s": wall_s,
        "prefill_graph": graph,
    }
    out.update(legs)
    if not args.only_prefill:
        out["prefix_index"] = bench_index(K, G)  # host CPU work, after the GPU legs
        log(f"index: {out['prefix_index']}")
    if not args.only_prefill and not args.only_core:
        log("varlen resume: 16 sequences")
        out["varlen_resume"] = bench_varlen(K, G)
        log(f"varlen: {out['varlen_resume']}")
        torch.cuda.empty_cache()
        log("long: 2^20 tokens")
        out["long_1m"] = bench_long(K, G)
        log(f"long: {out['long_1m']}")
        torch.cuda.empty_cache()
        # what simple kernels reach on this part (the roofline keeps the
        # published peaks): copy / fill / bf16 MFMA probes, ~1 s
        try:
            pk = measure_peaks()
        except (OSError, AssertionError, RuntimeError) as e:  # the probe library is optional
            out["measured_peaks"] = {"error": str(e)}
            log(f"peaks: not measured ({e})")
        else:
            out["measured_peaks"] = {k: pk[k] for k in ("copy_gbps", "fill_gbps", "mfma_bf16_tflops",
                                                        "torch_copy_gbps", "torch_fill_gbps")}
            out["roofline"]["frac_of_measured_copy"] = achieved / pk["copy_gbps"]
            log(f"peaks: {out['measured_peaks']}")
        torch.cuda.empty_cache()
    if not args.no_cpu:
        log("cpu baseline: oracle")
        out["cpu_baseline"] = cpu_baseline(G, w, d)
        if not args.only_prefill:
            out["cpu_baseline"]["prefix_index"] = cpu_index_oracle(G)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

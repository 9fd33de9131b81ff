"""Benchmark of the INT4 KV-cache hot path on one MI355X.

One step = the whole hot path over one batch: every sequence's new token is
rotated, quantized and appended to the paged INT4 cache, and attention runs
over every sequence's context (split-K partial kernel + merge and inverse
rotation).  The step is one paged_decode_step_int4 call (two kernels: the
merge kernel also does the append); the same step as two calls
(kv_quant_append, then paged_decode_attn_int4) is reported beside it.
Workload: 256 concurrent sequences with context lengths uniform in
[1024, 8192] (seeded), 8 KV heads x 128, 32 query heads, Hadamard block 64,
page size 16, pages shuffled over a shared pool; every input is synthetic
and resident in HBM before timing starts.

Prints ONE JSON line.  `value` is whole-step throughput in algorithmic GB/s
(the bytes the method must move: the INT4 K/V tiles of every cached token,
the page-table entries, queries and outputs, and the append's fp16 input and
INT4 output).  `roofline` is for the dominant kernel (the decode partial
kernel), timed with HIP events recorded on the library's stream in a second
pass of the same K steps (the timed region itself holds no events between
kernels: each one delays the next kernel).  Secondary
measurements (append bandwidth on a 65,536-token call, rotation on/off at
128K context, per-layer latency at batch 1 and 32K context, the fp16
baseline) are reported under "extra"; `cpu_baseline` times the CPU oracle on
a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, published
INT4_BYTES_PER_TOKEN_HEAD = 2 * (64 + 2)   # K and V: 64 code bytes + 2 scale bytes each
FP16_BYTES_PER_TOKEN_HEAD = 2 * 128 * 2
APPEND_BYTES_PER_TOKEN_HEAD = 2 * (128 * 2) + INT4_BYTES_PER_TOKEN_HEAD   # read fp16 K,V; write INT4


def decode_bytes(w, int4=True):
    """Algorithmic bytes of one decode call: cached K/V of every attended token,
    page-table entries, query (fp16) and output (fp32)."""
    import numpy as np
    ctx = np.maximum(w.context_lens.astype(np.int64), 0)
    per = INT4_BYTES_PER_TOKEN_HEAD if int4 else FP16_BYTES_PER_TOKEN_HEAD
    kv = int(ctx.sum()) * w.num_kv_heads * per
    pages = int(((ctx + w.page_size - 1) // w.page_size).sum()) * 4
    q = w.batch * w.num_q_heads * w.head_dim * 2
    out = w.batch * w.num_q_heads * w.head_dim * 4
    return kv + pages + q + out


def append_bytes(T, hkv):
    """Algorithmic bytes of one append call of T tokens: fp16 K/V rows read,
    INT4 codes+scales written, (seq, pos, page-table) read."""
    return T * hkv * APPEND_BYTES_PER_TOKEN_HEAD + T * 12


def _src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "bit_kv_cache_quant_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


DECODE_KERNEL_SRC = ("decode_mfma.hip", "decode_common.h", "kvq_internal.h")
DECODE_KERNEL_NAME = "decode_int4_balanced_kernel<64, 16>"


def _traffic_from_profile(kernel_hash):
    """HBM bytes per launch of the decode partial kernel from the committed
    rocprofv3 counter summary, or None if absent or taken on other code."""
    path = os.path.join(ROOT, "profiles", "decode_int4_c4_pmc.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256_16") != kernel_hash:
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Timer:
    """Per-launch durations from torch.cuda events (hipEvents) on the current stream."""

    def __init__(self):
        import torch
        self.torch = torch
        self.pairs = []

    def mark(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e


def build_int4_cache(w, dev, layer=0, had_block=None):
    import torch
    import bit_kv_cache_quant_amd as kvq
    bh = w.had_block if had_block is None else had_block
    tb = kvq.page_tile_bytes(w.head_dim, w.page_size)
    kp = torch.zeros((w.num_pages, w.num_kv_heads, tb), dtype=torch.uint8, device=dev)
    vp = torch.zeros_like(kp)
    pt = torch.as_tensor(w.table(layer), device=dev)
    for b in range(w.batch):
        L = int(w.prefill_lens[b])
        if L <= 0:
            continue
        k, v = w.rows(layer, b, 0, L, dev)
        seq = torch.full((L,), b, dtype=torch.int32, device=dev)
        pos = torch.arange(L, dtype=torch.int32, device=dev)
        kvq.kv_quant_append(k, v, seq, pos, pt, kp, vp, w.page_size, bh)
    return kp, vp, pt


def build_fp16_cache(w, dev, layer=0):
    import torch
    import bit_kv_cache_quant_amd as kvq
    shape = (w.num_pages, w.num_kv_heads, w.page_size, w.head_dim)
    kp = torch.zeros(shape, dtype=torch.float16, device=dev)
    vp = torch.zeros_like(kp)
    pt = torch.as_tensor(w.table(layer), device=dev)
    for b in range(w.batch):
        L = int(w.prefill_lens[b])
        if L <= 0:
            continue
        k, v = w.rows(layer, b, 0, L, dev)
        seq = torch.full((L,), b, dtype=torch.int32, device=dev)
        pos = torch.arange(L, dtype=torch.int32, device=dev)
        kvq.kv_append_fp16(k, v, seq, pos, pt, kp, vp, w.page_size)
    return kp, vp, pt


def settle(fn, min_ms=60.0):
    """Runs fn back to back, untimed, for at least min_ms of GPU time: the
    GPU's clocks ramp up over the first ~100 steps of sustained work (measured:
    the first 20 c4 steps ran at 310 us each, steps 80-100 at 218 us, and
    after 1 s idle the ramp repeats), so timings start from the steady state
    a serving loop runs in."""
    import torch
    spent, n = 0.0, 4
    while spent < min_ms:
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        spent += a.elapsed_time(b)
        n = min(2 * n, 256)
    return spent


def time_calls(fn, iters, warmup):
    """GPU time (ms) of fn(): the mean over iters calls issued back to back
    between two events (no host gaps between the calls), and the median of
    iters calls timed one by one with events around each.  The GPU is
    brought to its steady clocks first (settle)."""
    import torch
    settle(fn, 20.0)
    for _ in range(warmup):
        fn()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        fn()
    b.record()
    torch.cuda.synchronize()
    mean = a.elapsed_time(b) / iters
    evs = []
    for _ in range(iters):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    ts = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    return mean, ts[len(ts) // 2]


def time_calls_cold(fn, iters, dev, flush_bytes=1 << 30):
    """Mean GPU time (ms) of fn() with the last-level cache (256 MB MALL)
    flushed before every call by reading flush_bytes of another buffer (a
    read leaves clean lines behind: a written flush buffer would leave the
    cache full of dirty lines that the timed call then pays to write back);
    events bracket fn() alone."""
    import torch
    junk = torch.ones(flush_bytes // 4, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    settle(fn, 20.0)
    evs = []
    for _ in range(iters):
        torch.sum(junk, dim=0, dtype=torch.float32, out=sink)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    del junk
    return sum(e0.elapsed_time(e1) for e0, e1 in evs) / iters


def cpu_baseline(w, budget_s=12.0):
    """The oracle, as it stands, on a bounded sample of the workload: the
    first S sequences' append + decode, timed on the host cores."""
    import numpy as np
    import oracle
    import workloads as wl

    def run(S, reps=1):
        sub_need = (w.context_lens[:S] + w.page_size - 1) // w.page_size
        npg = int(sub_need.sum())
        pt = np.full((S, int(sub_need.max())), -1, np.int32)
        off = 0
        for b in range(S):
            pt[b, :sub_need[b]] = np.arange(off, off + sub_need[b], dtype=np.int32)
            off += int(sub_need[b])
        tb = oracle.tile_bytes(w.head_dim, w.page_size)
        kp = np.zeros((npg, w.num_kv_heads, tb), np.uint8)
        vp = np.zeros_like(kp)
        for b in range(S):  # prefill (setup, not timed)
            L = int(w.prefill_lens[b])
            k, v = w.rows(0, b, 0, L, "cpu")
            oracle.kv_quant_append(k.numpy(), v.numpy(), np.full(L, b, np.int32),
                                   np.arange(L, dtype=np.int32), pt, kp, vp, w.had_block, w.page_size)
        k_new = np.stack([w.rows(0, b, int(w.append_pos[b]), 1, "cpu")[0].numpy()[0] for b in range(S)])
        v_new = np.stack([w.rows(0, b, int(w.append_pos[b]), 1, "cpu")[1].numpy()[0] for b in range(S)])
        q = w.query(0, "cpu").numpy()[:S]
        t0 = time.perf_counter()
        for _ in range(reps):   # (the append rewrites the same slots with the same bytes)
            oracle.kv_quant_append(k_new, v_new, np.arange(S, dtype=np.int32), w.append_pos[:S].copy(), pt, kp,
                                   vp, w.had_block, w.page_size)
            oracle.paged_decode_attn_int4(q, kp, vp, pt, w.context_lens[:S].copy(), w.num_kv_heads, w.page_size,
                                          w.had_block, w.softmax_scale)
        dt = time.perf_counter() - t0
        sub = wl.Workload(**{**w.__dict__, "batch": S, "context_lens": w.context_lens[:S],
                              "per_layer_page_tables": None})
        nbytes = reps * (decode_bytes(sub) + append_bytes(S, w.num_kv_heads))
        return dt, nbytes

    # one thread on a small sample first (the oracle's per-unit work is
    # sequential either way), then every host thread
    nthreads = oracle.num_threads()
    oracle.set_num_threads(1)
    dt1, nbytes1 = run(4)
    oracle.set_num_threads(nthreads)
    S, reps = 2, 1
    dt, nbytes = run(S)
    if dt < budget_s / 4:
        S = int(min(w.batch, max(S + 1, math.floor(S * budget_s / max(dt, 1e-3) * 0.8))))
        dt, nbytes = run(S)
    if S == w.batch and dt < budget_s / 2:   # the whole batch is quick: repeat it
        reps = max(2, int(budget_s * 0.8 / max(dt, 1e-3)))
        dt, nbytes = run(S, reps)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(dt, 3), "cpu_model": model, "host_cpus": os.cpu_count(),
            "single_thread_value": round(nbytes1 / dt1 / 1e9, 4),
            "single_thread_sample": "first 4 sequences, one thread",
            "sample": f"first {S} of {w.batch} sequences, {reps} time(s): append of their new tokens + fp64 "
                      f"decode over their contexts (sum {int(w.context_lens[:S].sum())} tokens), "
                      "same shapes, CPU-generated values"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--quick", action="store_true", help="main workload only (no extra measurements)")
    ap.add_argument("--append-only", action="store_true",
                    help="only the append bandwidth measurement (65,536 tokens in one call), one JSON line")
    ap.add_argument("--fp16-only", action="store_true",
                    help="only the fp16 baseline decode on the main workload, one JSON line")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the causal prefill attention over a 32,768-token prompt, one JSON line")
    ap.add_argument("--c3-only", action="store_true",
                    help="only the batch-1, 32K-context, 36-layer decode step, one JSON line")
    ap.add_argument("--no-graph", action="store_true", help="with --c3-only: no HIP-graph timing")
    ap.add_argument("--variants-only", action="store_true",
                    help="only the quantizer-variant measurements, one JSON line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB streaming kernel (counter calibration under rocprofv3 --pmc)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): the hot path is "
              "per-GPU data-parallel (each GPU serves its own sequences and caches), and this "
              "benchmark has no multi-GPU mode.", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import bit_kv_cache_quant_amd as kvq
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kvq.lib()

    if args.append_only:
        print(json.dumps({"append": append_measurements(dev, iters=args.steps, warmup=args.warmup,
                                                        with_decode_time=False)}), flush=True)
        return 0
    if args.fp16_only:
        print(json.dumps({"decode_fp16_c4": fp16_measurement(dev, iters=args.steps, warmup=args.warmup)}),
              flush=True)
        return 0

    if args.c3_only:
        print(json.dumps({"decode_b1_32k_36layers": c3_measurement(dev, iters=args.steps, warmup=args.warmup,
                                                                   with_graph=not args.no_graph)}), flush=True)
        return 0

    if args.variants_only:
        print(json.dumps({"variants": variant_measurements(dev, iters=args.steps, warmup=args.warmup)}), flush=True)
        return 0

    if args.prefill_only:
        print(json.dumps({"prefill_b1_32k": prefill_measurement(dev, iters=args.steps, warmup=args.warmup)}),
              flush=True)
        return 0

    if args.calibrate_copy:
        # a plain streaming kernel of known traffic: reads 1 GiB, writes 1 GiB
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # ---------------- main workload: decode step with append ----------------
    w = wl.c4()
    kp, vp, pt = build_int4_cache(w, dev)
    k_new, v_new = w.append_rows(0, dev)
    seq = torch.as_tensor(w.append_seq, device=dev)
    pos = torch.as_tensor(w.append_pos, device=dev)
    q = w.query(0, dev)
    cl = torch.as_tensor(w.context_lens, device=dev)
    maxctx = int(w.context_lens.max())
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    ws = torch.empty(kvq.workspace_bytes(w.batch, w.num_q_heads, w.num_kv_heads, maxctx, w.page_size),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    mid = torch.cuda.Event(enable_timing=True)
    mid.record()
    torch.cuda.synchronize()

    def step(mid_ev=None):
        # one call: the partial kernel over every cached token, whose range
        # that ends at a sequence's last cached token also rotates, quantizes,
        # stores and attends to the sequence's new token, then the merge
        kvq.paged_decode_step_int4(q, k_new, v_new, kp, vp, pt, cl, w.num_kv_heads, w.page_size, w.had_block,
                                   w.softmax_scale, maxctx, out=out, workspace=ws, phase_event=mid_ev)

    def step_two_calls():
        kvq.kv_quant_append(k_new, v_new, seq, pos, pt, kp, vp, w.page_size, w.had_block)
        kvq.paged_decode_attn_int4(q, kp, vp, pt, cl, w.num_kv_heads, w.page_size, w.had_block, w.softmax_scale,
                                   maxctx, out=out, workspace=ws)

    settle_ms = settle(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K steps back to back, bracketed by two events and nothing
    # in between.  An event recorded between two kernels holds the second
    # one back until the first has fully drained (measured: two per step
    # added ~6 us to a 216 us step), so the kernels' own durations come from
    # a second pass of the same K steps with events at every phase boundary,
    # on the library's stream (torch's current stream, which the library
    # launches on).
    def make_events(n):
        evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(n)) for _ in range(args.steps)]
        for e in evs:
            e[-1].record()                # instantiate; the decode call re-records it between its kernels
        return evs
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        step()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_per_step = ms_total / args.steps

    # phase pass: (before the call, after the partial kernel, after the merge)
    phase = make_events(3)
    torch.cuda.synchronize()
    for i in range(args.steps):
        e0, e2, em = phase[i]
        e0.record()
        step(mid_ev=em)
        e2.record()
    torch.cuda.synchronize()
    t_partial = [p[0].elapsed_time(p[2]) for p in phase]
    t_combine = [p[2].elapsed_time(p[1]) for p in phase]
    mean = lambda xs: sum(xs) / len(xs)

    dbytes = decode_bytes(w)
    abytes = append_bytes(int(w.append_seq.size), w.num_kv_heads)
    step_bytes = dbytes + abytes
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # The same step as two calls (append kernel, then partial + merge), for comparison.
    settle(step_two_calls, 20.0)
    two_mean, two_med = time_calls(step_two_calls, args.steps, 3)
    # The step with the last-level cache (256 MB) flushed before each call:
    # the 1.23 GB cache does not fit it, so this differs from the steady
    # state only by what the cache kept between steps.
    cold_ms = time_calls_cold(step, min(args.steps, 20), dev)

    # the partial kernel moves the tiles of every cached token but the new one,
    # the page table and the queries (outputs go via the workspace)
    ctx = np.maximum(w.context_lens.astype(np.int64) - 1, 0)
    partial_alg = (int(ctx.sum()) * w.num_kv_heads * INT4_BYTES_PER_TOKEN_HEAD
                   + int(((ctx + 15) // 16).sum()) * 4 + w.batch * w.num_q_heads * w.head_dim * 2)
    achieved = partial_alg / (mean(t_partial) * 1e-3) / 1e9
    khash = _src_hash(*DECODE_KERNEL_SRC)
    traffic = _traffic_from_profile(khash)

    result = {
        "metric": "INT4 paged decode-attn HBM GB/s (% of peak); rotate-quant-append tokens/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 cache x fp16 scales; int8 MFMA fixed-point q.k and p.v, fp32 softmax",
        "data": "synthetic",
        "config": {
            "workload": "decode step with append: batch 256, ctx U[1024,8192] (seeded), 8 KV heads x 128, "
                        "32 query heads, Hadamard block 64, page size 16, shuffled page pool",
            "kv_format": "INT4 codes + fp16 scale per (token, KV head)",
            "global_batch": w.batch,
            "context_tokens": int(w.context_lens.sum()),
            "bytes_per_step": step_bytes,
            "pct_of_hbm_peak": round(100 * value / PEAK_HBM_GBS, 2),
            "step_call": "paged_decode_step_int4 (the new tokens' append fused into the decode kernels)",
            "append_tokens_per_s": round(w.batch / (ms_per_step * 1e-3), 1),
            "partial_ms": round(mean(t_partial), 5),
            "merge_with_append_ms": round(mean(t_combine), 5),
            "phase_times": "partial kernel and merge: HIP events at the phase boundaries in a second pass "
                           "of the same K steps (the timed region holds no events between kernels)",
            "two_calls_ms_per_step": round(two_mean, 5),
            "two_calls_GBps": round(step_bytes / (two_mean * 1e-3) / 1e9, 2),
            "two_calls": "kv_quant_append then paged_decode_attn_int4, the same K steps back to back",
            "cold_ms_per_step": round(cold_ms, 5),
            "cold_GBps": round(step_bytes / (cold_ms * 1e-3) / 1e9, 2),
            "cold": "the step with 1 GiB of another buffer read before each call (last-level cache flushed)",
            "host_wall_s": round(wall, 4),
            "settle_ms": round(settle_ms, 1),
            "timing": "steady state: the step runs untimed for settle_ms of GPU time (clock ramp), then "
                      "the W warmup steps, then the K timed steps",
        },
        "roofline": {
            "kernel": DECODE_KERNEL_NAME,
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "alg_bytes_per_launch": partial_alg,
            "avg_launch_ms": round(mean(t_partial), 5),
            "launch_ms_p10_p50_p90": [round(float(np.percentile(t_partial, q)), 5) for q in (10, 50, 90)],
            "kernel_source_sha256_16": khash,
        },
    }
    del kp, vp, ws, k_new, v_new
    torch.cuda.empty_cache()

    if not args.quick:
        result["extra"] = extra_measurements(dev, args)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)
    return 0


def append_measurements(dev, iters=20, warmup=3, with_decode_time=True):
    """Append bandwidth: 256 sequences x 256 consecutive tokens in one call
    (Hadamard block 64 and no rotation), and (with_decode_time) the
    decode-time append of one token for each of 256 sequences."""
    import torch
    import bit_kv_cache_quant_amd as kvq
    import workloads as wl
    ex = {}
    w = wl.c2_stream()
    tb = kvq.page_tile_bytes(w.head_dim, w.page_size)
    kp = torch.zeros((w.num_pages, w.num_kv_heads, tb), dtype=torch.uint8, device=dev)
    vp = torch.zeros_like(kp)
    k, v = w.append_rows(0, dev)
    seq = torch.as_tensor(w.append_seq, device=dev)
    pos = torch.as_tensor(w.append_pos, device=dev)
    pt = torch.as_tensor(w.page_table, device=dev)
    T = int(w.append_seq.size)
    nb = append_bytes(T, w.num_kv_heads)
    for bh in (64, 0, 128, 32):
        ms, med = time_calls(lambda: kvq.kv_quant_append(k, v, seq, pos, pt, kp, vp, w.page_size, bh), iters, warmup)
        ex[f"append_65536tok_bh{bh}"] = {"ms": round(ms, 5), "tokens_per_s": round(T / (ms * 1e-3), 1),
                                         "GBps": round(nb / (ms * 1e-3) / 1e9, 2),
                                         "pct_of_hbm_peak": round(100 * nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
                                         "timing": "back to back: most of the 268 MB input can stay in the 256 MB "
                                                   "last-level cache between calls"}
    if with_decode_time:
        ms_c = time_calls_cold(lambda: kvq.kv_quant_append(k, v, seq, pos, pt, kp, vp, w.page_size, 64), iters, dev)
        ex["append_65536tok_bh64_cold"] = {
            "ms": round(ms_c, 5), "GBps": round(nb / (ms_c * 1e-3) / 1e9, 2),
            "pct_of_hbm_peak": round(100 * nb / (ms_c * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
            "timing": "1 GiB of another buffer read before each call (last-level cache flushed)"}
    if not with_decode_time:
        del kp, vp, k, v
        torch.cuda.empty_cache()
        return ex
    # prompt append: 32,768 consecutive tokens of one sequence in one call
    # (the prefill side of the same kernel), into a batch-1 32K-context cache
    w3 = wl.c3(layers=1)
    kp3 = torch.zeros((w3.num_pages, w3.num_kv_heads, kvq.page_tile_bytes(w3.head_dim, w3.page_size)),
                      dtype=torch.uint8, device=dev)
    vp3 = torch.zeros_like(kp3)
    L3 = int(w3.prefill_lens[0])
    k3, v3 = w3.rows(0, 0, 0, L3, dev)
    s3 = torch.zeros(L3, dtype=torch.int32, device=dev)
    p3 = torch.arange(L3, dtype=torch.int32, device=dev)
    pt3 = torch.as_tensor(w3.table(0), device=dev)
    ms, med = time_calls(lambda: kvq.kv_quant_append(k3, v3, s3, p3, pt3, kp3, vp3, w3.page_size, w3.had_block),
                         iters, warmup)
    nb3 = append_bytes(L3, w3.num_kv_heads)
    ex["append_prompt_32768tok_bh128"] = {"ms": round(ms, 5), "tokens_per_s": round(L3 / (ms * 1e-3), 1),
                                          "GBps": round(nb3 / (ms * 1e-3) / 1e9, 2),
                                          "pct_of_hbm_peak": round(100 * nb3 / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
                                          "timing": "back to back: the ~169 MB working set may stay in the "
                                                    "256 MB last-level cache"}
    ms_c = time_calls_cold(lambda: kvq.kv_quant_append(k3, v3, s3, p3, pt3, kp3, vp3, w3.page_size, w3.had_block),
                           iters, dev)
    ex["append_prompt_32768tok_bh128_cold"] = {
        "ms": round(ms_c, 5), "GBps": round(nb3 / (ms_c * 1e-3) / 1e9, 2),
        "pct_of_hbm_peak": round(100 * nb3 / (ms_c * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
        "timing": "1 GiB of another buffer read before each call (last-level cache flushed)"}
    del kp3, vp3, k3, v3
    # decode-time append (1 token per sequence)
    w2 = wl.c2()
    k2, v2 = w2.append_rows(0, dev)
    s2 = torch.as_tensor(w2.append_seq, device=dev)
    p2 = torch.as_tensor(w2.append_pos, device=dev)
    ms, med = time_calls(lambda: kvq.kv_quant_append(k2, v2, s2, p2, pt, kp, vp, 16, 64), 50, 5)
    ex["append_256x1tok_bh64"] = {"ms": round(ms, 5), "tokens_per_s": round(256 / (ms * 1e-3), 1),
                                  "single_call_median_ms": round(med, 5)}
    del kp, vp, k, v
    torch.cuda.empty_cache()
    return ex


def extra_measurements(dev, args):
    import numpy as np
    import torch
    import bit_kv_cache_quant_amd as kvq
    import workloads as wl
    ex = append_measurements(dev)

    # Rotation on vs off: batch 8 x 131,072 context, page size 32.
    rot = {}
    for bh in (128, 0):
        w5 = wl.c5(had_block=bh)
        kp, vp, pt = build_int4_cache(w5, dev, had_block=bh)
        q = w5.query(0, dev)
        cl = torch.as_tensor(w5.context_lens, device=dev)
        out = torch.empty((w5.batch, w5.num_q_heads, w5.head_dim), dtype=torch.float32, device=dev)
        ws = torch.empty(kvq.workspace_bytes(w5.batch, 32, 8, 131072, 32), dtype=torch.uint8, device=dev)
        ms, med = time_calls(lambda: kvq.paged_decode_attn_int4(q, kp, vp, pt, cl, 8, 32, bh, w5.softmax_scale,
                                                                131072, out=out, workspace=ws), 20, 3)
        nb = decode_bytes(w5)
        rot[bh] = ms
        ex[f"decode_8x128k_bh{bh}"] = {"ms": round(ms, 5), "GBps": round(nb / (ms * 1e-3) / 1e9, 2),
                                       "pct_of_hbm_peak": round(100 * nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)}
        del kp, vp
        torch.cuda.empty_cache()
    ex["rotation_overhead_pct"] = round(100 * (rot[128] / rot[0] - 1), 2)

    ex["decode_b1_32k_36layers"] = c3_measurement(dev)

    ex["decode_fp16_c4"] = fp16_measurement(dev, iters=10, warmup=2)
    ex["prefill_b1_32k"] = prefill_measurement(dev, iters=5, warmup=1)
    ex["variants"] = variant_measurements(dev)
    return ex


# (name, format, had_block, scale_group, scale_search, sign_mask)
VARIANT_CFGS = [
    ("int4_bh32_scale_per_block", 0, 32, 32, 0, 0),
    ("int4_bh32_scale_per_block_search", 0, 32, 32, 1, 0),
    ("int4_bh64_scale_per_block", 0, 64, 64, 0, 0),
    ("int4_bh128_token_scale_random_signs", 0, 128, 128, 0, 0x9E3779B97F4A7C15F39CC0605CEDC834),
    ("mxfp4_bh32", 1, 32, 32, 0, 0),
    ("mxfp4_bh128", 1, 128, 32, 0, 0),
]


def variant_measurements(dev, iters=10, warmup=2):
    """The quantizer variants (per-block INT4 scales, scale search, random
    signs, MXFP4): append bandwidth on 65,536 tokens (256 sequences x 256
    consecutive tokens, page size 16) and decode bandwidth at the
    long-context shape (batch 8 x 131,072, page size 32) and the batch-256
    shape, each as algorithmic bytes (codes + this format's scales)."""
    import numpy as np
    import torch
    import bit_kv_cache_quant_amd as kvq
    import workloads as wl
    res = {}
    w2 = wl.c2_stream()
    k, v = w2.append_rows(0, dev)
    seq = torch.as_tensor(w2.append_seq, device=dev)
    pos = torch.as_tensor(w2.append_pos, device=dev)
    pt2 = torch.as_tensor(w2.page_table, device=dev)
    T = int(w2.append_seq.size)
    for name, *args in VARIANT_CFGS:
        cfg = kvq.quant_config(*args)
        tb = kvq.page_tile_bytes_cfg(128, 16, cfg)
        per = 2 * tb // 16                    # K and V bytes per token-head
        kp = torch.zeros((w2.num_pages, 8, tb), dtype=torch.uint8, device=dev)
        vp = torch.zeros_like(kp)
        ms, _ = time_calls(lambda: kvq.kv_quant_append_cfg(k, v, seq, pos, pt2, kp, vp, 16, cfg), iters, warmup)
        nb = T * 8 * (2 * 256 + per) + T * 12
        res[name] = {"bytes_per_token_head": per,
                     "append_65536tok": {"ms": round(ms, 5), "GBps": round(nb / (ms * 1e-3) / 1e9, 2),
                                         "pct_of_hbm_peak": round(100 * nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)}}
        del kp, vp
    del k, v
    torch.cuda.empty_cache()
    for wname, w in (("decode_8x128k", wl.c5()), ("decode_c4", wl.c4())):
        pt = torch.as_tensor(w.table(0), device=dev)
        cl = torch.as_tensor(w.context_lens, device=dev)
        q = w.query(0, dev)
        maxctx = int(w.context_lens.max())
        out = torch.empty((w.batch, 32, 128), dtype=torch.float32, device=dev)
        ws = torch.empty(kvq.workspace_bytes(w.batch, 32, 8, maxctx, w.page_size), dtype=torch.uint8, device=dev)
        ctx = np.maximum(w.context_lens.astype(np.int64), 0)
        for name, *args in VARIANT_CFGS:
            cfg = kvq.quant_config(*args)
            tb = kvq.page_tile_bytes_cfg(128, w.page_size, cfg)
            per = 2 * tb // w.page_size
            kp = torch.zeros((w.num_pages, 8, tb), dtype=torch.uint8, device=dev)
            vp = torch.zeros_like(kp)
            for b in range(w.batch):
                L = int(w.prefill_lens[b])
                kk, vv = w.rows(0, b, 0, L, dev)
                kvq.kv_quant_append_cfg(kk, vv, torch.full((L,), b, dtype=torch.int32, device=dev),
                                        torch.arange(L, dtype=torch.int32, device=dev), pt, kp, vp, w.page_size, cfg)
            ms, _ = time_calls(lambda: kvq.paged_decode_attn_cfg(q, kp, vp, pt, cl, 8, w.page_size, cfg,
                                                                 w.softmax_scale, maxctx, out=out, workspace=ws),
                               iters, warmup)
            nb = int(ctx.sum()) * 8 * per + int(((ctx + w.page_size - 1) // w.page_size).sum()) * 4 \
                + w.batch * 32 * 128 * 6
            res[name][wname] = {"ms": round(ms, 5), "GBps": round(nb / (ms * 1e-3) / 1e9, 2),
                                "pct_of_hbm_peak": round(100 * nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)}
            del kp, vp
            torch.cuda.empty_cache()
    return res


def c3_measurement(dev, iters=10, warmup=2, with_graph=True):
    """Latency-sensitive decode: batch 1, 32K context, 36 layers with distinct
    pools and page permutations (Hadamard block 128, page size 16); the
    36-layer step timed eagerly and as one HIP graph (replays checked bit for
    bit against the eager step)."""
    import torch
    import bit_kv_cache_quant_amd as kvq
    import workloads as wl
    ex = {}
    w3 = wl.c3()
    caches = [build_int4_cache(w3, dev, layer=l) for l in range(w3.layers)]
    qs = [w3.query(l, dev) for l in range(w3.layers)]
    cl = torch.as_tensor(w3.context_lens, device=dev)
    out = torch.empty((1, 32, 128), dtype=torch.float32, device=dev)
    ws = torch.empty(kvq.workspace_bytes(1, 32, 8, 32768, 16), dtype=torch.uint8, device=dev)

    def all_layers():
        for l in range(w3.layers):
            kpl, vpl, ptl = caches[l]
            kvq.paged_decode_attn_int4(qs[l], kpl, vpl, ptl, cl, 8, 16, 128, w3.softmax_scale, 32768,
                                       out=out, workspace=ws)
    ms, med = time_calls(all_layers, iters, warmup)
    nb = decode_bytes(w3) * w3.layers
    ex["decode_b1_32k_36layers"] = {"ms_per_step": round(ms, 5), "us_per_layer": round(1000 * ms / w3.layers, 3),
                                    "GBps": round(nb / (ms * 1e-3) / 1e9, 2),
                                    "pct_of_hbm_peak": round(100 * nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)}
    if not with_graph:
        del caches
        torch.cuda.empty_cache()
        return ex["decode_b1_32k_36layers"]
    # The same 36-layer step captured once in a HIP graph and replayed; every
    # checked replay must give the eager step's output, with eager work and
    # synchronisations in between.
    torch.cuda.synchronize()
    all_layers()
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        all_layers()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        all_layers()
    for _ in range(3):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(out, eager):
            raise RuntimeError("graph replay of the batch-1 decode step differs from the eager step")
        all_layers()
        torch.cuda.synchronize()
    ms_g, _ = time_calls(graph.replay, iters, warmup)
    ex["decode_b1_32k_36layers"].update({"graph_ms_per_step": round(ms_g, 5),
                                         "graph_us_per_layer": round(1000 * ms_g / w3.layers, 3),
                                         "graph_pct_of_hbm_peak":
                                             round(100 * nb / (ms_g * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)})
    del graph
    del caches
    torch.cuda.empty_cache()

    return ex["decode_b1_32k_36layers"]


PEAK_F16_TFLOPS = 2500.0      # MI355X dense fp16 matrix rate, published
PEAK_I8_TOPS = 5000.0         # MI355X dense int8 matrix rate, published


def prefill_measurement(dev, iters, warmup):
    """Causal prefill attention of a whole 32,768-token prompt (batch 1,
    Hq 32, Hkv 8, D 128, Hadamard block 128, page size 16, shuffled pages)
    over its INT4 cache.  Useful flops: 4 D Hq per (query, visible key) pair
    (q.k and p.v, 2 each), L (L + 1) / 2 pairs.  The kernel issues more
    matrix work than that: q.k as three int8 limb products per nibble half
    (6 v_mfma_i32_16x16x64_i8 per 16 x 16 x 128 score tile) and p.v with the
    weights split into fp16 hi + lo (2 fp16 products per useful one);
    mfma_time_frac is the time those issued instructions take at the
    published dense peaks over the measured time."""
    import torch
    import bit_kv_cache_quant_amd as kvq
    import workloads as wl
    w = wl.c3(layers=1)
    kp, vp, pt = build_int4_cache(w, dev, layer=0)
    L = int(w.context_lens[0])
    g = torch.Generator(device=dev)
    g.manual_seed(3030)
    q = torch.randn((L, w.num_q_heads, w.head_dim), generator=g, device=dev).to(torch.float16)
    qs = torch.tensor([0, L], dtype=torch.int32, device=dev)
    cl = torch.as_tensor(w.context_lens, device=dev)
    out = torch.empty((L, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    call = lambda: kvq.paged_prefill_attn_int4(q, qs, kp, vp, pt, cl, w.num_kv_heads, w.page_size, w.had_block,
                                               w.softmax_scale, out=out)
    ms, med = time_calls(call, iters, warmup)
    pairs = L * (L + 1) // 2
    useful = 4.0 * w.head_dim * w.num_q_heads * pairs
    # issued work per 16 x 16 x 128 tile: q.k 6 int8 MFMAs of 16x16x64, p.v 8 fp16 MFMAs of 16x16x32
    tiles = useful / (4.0 * 16 * 16 * 128)
    t_issue = tiles * (6 * 2 * 16 * 16 * 64 / (PEAK_I8_TOPS * 1e12) + 8 * 2 * 16 * 16 * 32 / (PEAK_F16_TFLOPS * 1e12))
    res = {"ms": round(ms, 4), "median_ms": round(med, 4), "prompt_tokens": L,
           "useful_TFLOPs": round(useful / (ms * 1e-3) / 1e12, 1),
           "useful_frac_of_f16_peak": round(useful / (ms * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4),
           "mfma_time_frac": round(t_issue / (ms * 1e-3), 4),
           "prompt_tokens_per_s": round(L / (ms * 1e-3), 1)}
    del kp, vp, q, out
    torch.cuda.empty_cache()
    return res


def fp16_measurement(dev, iters, warmup):
    """The fp16 baseline decode on the main workload (batch 256, fp16 pools):
    whole call (partial kernel + merge) and the partial kernel alone (HIP
    events recorded around it through the library's timing hook)."""
    import torch
    import bit_kv_cache_quant_amd as kvq
    import workloads as wl
    w = wl.c4()
    kp, vp, pt = build_fp16_cache(w, dev)
    q = w.query(0, dev)
    cl = torch.as_tensor(w.context_lens, device=dev)
    maxctx = int(w.context_lens.max())
    out = torch.empty((w.batch, 32, 128), dtype=torch.float32, device=dev)
    ws = torch.empty(kvq.workspace_bytes(w.batch, 32, 8, maxctx, 16), dtype=torch.uint8, device=dev)
    call = lambda ev=None: kvq.paged_decode_attn_fp16(q, kp, vp, pt, cl, 8, 16, w.softmax_scale, maxctx,
                                                      out=out, workspace=ws, phase_event=ev)
    ms, med = time_calls(call, iters, warmup)
    # partial kernel alone: an event before the call and the library's event after the kernel
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for _, em in evs:
        em.record()
    torch.cuda.synchronize()
    for e0, em in evs:
        e0.record()
        call(em)
    torch.cuda.synchronize()
    part = sum(e0.elapsed_time(em) for e0, em in evs) / iters
    nb = decode_bytes(w, int4=False)
    res = {"ms": round(ms, 5), "GBps": round(nb / (ms * 1e-3) / 1e9, 2),
           "pct_of_hbm_peak": round(100 * nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
           "partial_kernel_ms": round(part, 5),
           "partial_kernel_GBps": round(nb / (part * 1e-3) / 1e9, 2),
           "partial_kernel_pct_of_hbm_peak": round(100 * nb / (part * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)}
    del kp, vp
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    sys.exit(main())

#!/usr/bin/env python3
"""Benchmark of the ring-attention hot path on one MI355X.

One step is one ``ring_attention`` call over one device's full share (every
key/value chunk, in ring order, with the causal mask if the workload has one),
with inputs already resident in HBM. The headline is the largest share that
fits one GPU: the long-context GQA share (16384 local queries, 8 query heads
on one key/value head, d = 128, against 1,048,576 keys in 64 shards). The JSON
line reports its counted throughput ``4 * d * Hq * (allowed query-key pairs)``
per second and the roofline of its attention kernel (bf16 MFMA bound); the
other bf16 shares, each timed the same way, in a ``configs`` block; the
standalone chunk-statistics and merge legs (the merge is HBM-bound, next to a
device copy of the same size) and the backward pass in ``legs``; and the fp64
CPU oracle timed on a bounded sample of the headline share.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config I]
"""

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
FP32_PEAK_TFLOPS = 157.3    # MI355X fp32 matrix, published
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
KERNEL_SOURCE = os.path.join(ROOT, "ring_attention_chunk_amd", "csrc", "attention.hip")
HEADLINE = 4                 # long_gqa_hq8_hkv1_d128_q16k_k1m: the largest share on one GPU
OTHER_CONFIGS = "1,2,3,5"    # the other bf16 shares, reported in the configs block


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed calls of the headline share")
    ap.add_argument("--warmup", type=int, default=5, help="untimed calls right before the timed ones")
    ap.add_argument("--settle-seconds", type=float, default=1.0,
                    help="untimed calls for about this long before the warm-up, so that the GPU clocks have "
                         "settled under load (reported as clock_settle; 0 turns it off)")
    ap.add_argument("--config", type=int, default=HEADLINE, help="workload index of the headline share")
    ap.add_argument("--configs", default=OTHER_CONFIGS,
                    help="comma-separated workload indices timed in the configs block ('' for none)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-legs", action="store_true", help="skip the chunk-stats, merge and backward legs")
    ap.add_argument("--profile-run", action="store_true",
                    help="launch sequence for rocprofv3 counter passes: the workload's ring_attention, a device "
                         "copy of COPY_BYTES, then the merge leg; prints what was launched")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DIR",
                    help="turn the counter CSVs of the --profile-run passes (FETCH_SIZE, WRITE_SIZE, SQ, and "
                         "optionally a second SQ pass of instruction counts) into a profiles/ summary")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "BENCH_JSON"),
                    help="turn a rocprofv3 --kernel-trace --stats run of this script and the JSON line it printed "
                         "into a profiles/ summary")
    ap.add_argument("--command", default="", help="with --summarize-*: the command lines that made the files")
    ap.add_argument("--with-backward", action="store_true",
                    help="with --profile-run: also run the backward pass of the workload")
    return ap.parse_args()


COPY_BYTES = 1 << 30      # bytes read (and written) by the calibration copy
MERGE_ROWS, MERGE_D = 32 * 8192, 128
SIMD_NUM = 256 * 4


def source_digest():
    """Digest of the kernel source with // comments and blank lines removed, so that comment edits do
    not detach the committed counter summaries from the code they were taken on."""
    import re

    with open(KERNEL_SOURCE) as f:
        lines = [re.sub(r"\s*//.*$", "", ln).rstrip() for ln in f]
    code = "\n".join(ln for ln in lines if ln)
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def timed(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps  # ms per call


def call_seconds(fn, torch):
    """Wall time of one call after one untimed call."""
    fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    return max(time.perf_counter() - t0, 1e-6)


def settle(fn, torch, seconds):
    """Untimed calls for about `seconds` (clock settling under load); returns (calls, seconds)."""
    if seconds <= 0:
        return 0, 0.0
    n = int(min(5000, max(1, round(seconds / call_seconds(fn, torch)))))
    t0 = time.perf_counter()
    for _ in range(n):
        fn()
    torch.cuda.synchronize()
    return n + 2, round(time.perf_counter() - t0, 3)


def timed_with_kernel(fn, steps, warmup, torch, api):
    """As timed(), and also the average device time of the attention kernel of the timed calls (the
    library's kernel timer, enabled only over the timed region)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    api.kernel_timer(True)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    total, n = api.kernel_timer_read()
    api.kernel_timer(False)
    if n == 0:
        raise RuntimeError("the kernel timer recorded no launch")
    return start.elapsed_time(stop) / steps, total / n


def dominant_kernel(w):
    """Name of the kernel that does a workload's attention: every bf16 workload here (aligned rows,
    whole 16-byte pieces) runs the pipelined bf16 kernel, fp32 the general one."""
    return "attention_bf16_kernel" if w.dtype == "bf16" else "attention_kernel"


def counter_summary(w):
    """The committed rocprofv3 counter summary of a workload, if it matches this source."""
    path = os.path.join(ROOT, "profiles", f"{dominant_kernel(w)}_{w.name}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha256_16") != source_digest():
        return None  # the kernel changed since the counters were taken
    return t


def traffic_for(w):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match this source."""
    t = counter_summary(w)
    return t.get("bytes_per_launch") if t else None


def clock_derived_peak(w, achieved):
    """The bf16 peak at the shader clock the counters saw while the kernel ran (CUs x sclk x 4096
    flops per clock), from the committed counter summary; the published peak assumes 2.4 GHz."""
    t = counter_summary(w)
    if not t or not t.get("sclk_ghz_under_load"):
        return None
    peak = t["clock_derived_bf16_peak_tflops"]
    return {"sclk_ghz": round(t["sclk_ghz_under_load"], 3), "peak": round(peak, 1), "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "source": "GRBM_GUI_ACTIVE over the profiled kernel duration"}


def measure_share(w, steps, warmup, settle_s, torch, ra, wl, dev="cuda:0"):
    """Time ``ring_attention`` over share ``w``: settle, warm up, then ``steps`` timed calls.

    Returns the entry of the JSON line and the device inputs (for the legs and the CPU baseline)."""
    q, k, v, kc, vc = wl.generate_torch(w, dev)
    offs = w.kv_offsets
    ws = torch.empty(ra.api.workspace_bytes(tuple(q.shape), [c.shape[2] for c in kc], len(w.q_segments)),
                     dtype=torch.uint8, device=dev)

    def step():
        return ra.ring_attention(q, kc, vc, w.q_runs, offs, causal=w.causal, scale=w.softmax_scale,
                                 workspace=ws, kv_position_strides=w.kv_strides)

    if steps is None:  # configs block: enough calls for about 0.3 s of timed work
        steps = int(min(500, max(10, math.ceil(0.3 / call_seconds(step, torch)))))
    settle_calls, settle_sec = settle(step, torch, settle_s)
    ms, kernel_ms = timed_with_kernel(step, steps, warmup, torch, ra.api)
    flops = wl.counted_flops(w)
    peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
    kernel_tflops = flops / (kernel_ms * 1e-3) / 1e12
    entry = {
        "ms": round(ms, 4),
        "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 2),
        "kernel_ms": round(kernel_ms, 4),
        "kernel_TFLOP/s": round(kernel_tflops, 2),
        "frac": round(kernel_tflops / peak, 4),
        "steps": steps,
        "warmup": warmup,
        "clock_settle_calls": settle_calls,
        "counted_flops": flops,
    }
    return entry, (q, kc, vc, offs)


def describe(w):
    return {
        "workload": w.name,
        "batch": w.batch,
        "q_heads": w.q_heads,
        "kv_heads": w.kv_heads,
        "head_dim": w.head_dim,
        "local_queries": w.lq,
        "keys": w.lk,
        "kv_chunks": len(w.chunks),
        "causal": w.causal,
        "pos_stride": w.pos_stride,
    }


def backward_leg(w, q, kc, vc, offs, args, torch, ra):
    """The backward pass of the same share (dQ, and this share's dK, dV per chunk) from the forward's out
    and lse, with a seeded bf16 upstream gradient. Counted flops: 10*d per allowed pair and query head
    (five matrix products of 2*d: S, dP, dV, dK, dQ); the kernels recompute S and dP a second time."""
    from ring_attention_chunk_amd import workloads as wl

    dev = q.device
    out, lse = ra.ring_attention(q, kc, vc, w.q_runs, offs, causal=w.causal, scale=w.softmax_scale,
                                 return_lse=True, kv_position_strides=w.kv_strides)
    g = torch.Generator(device=dev).manual_seed(7)
    dout = torch.randn(q.shape, device=dev, generator=g).to(torch.bfloat16)
    ws = torch.empty(ra.api.backward_workspace_bytes(tuple(q.shape), [c.shape[2] for c in kc], len(w.q_segments)),
                     dtype=torch.uint8, device=dev)

    def step():
        return ra.ring_attention_backward(q, kc, vc, out, lse, dout, w.q_runs, offs, causal=w.causal,
                                          scale=w.softmax_scale, kv_position_strides=w.kv_strides, workspace=ws)

    steps = max(3, min(args.steps, 10))
    ms, pair_ms = timed_with_kernel(step, steps, 2, torch, ra.api)
    kernels_ms = 2 * pair_ms  # the dK/dV kernel and the dQ kernel, each timed by its own event pair
    flops = 10 * w.head_dim * w.q_heads * w.batch * wl.unmasked_pairs_per_head(w)
    return {
        "ms": round(ms, 4),
        "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 2),
        "kernels_ms": round(kernels_ms, 4),
        "kernels_TFLOP/s": round(flops / (kernels_ms * 1e-3) / 1e12, 2),
        "frac_of_bf16_peak": round(flops / (kernels_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "counted_flops": flops,
        "shape": f"{w.name}: dq, and dk, dv of every chunk; bf16 dout",
    }


def stats_leg(q, k0, v0, scale, args, torch, ra):
    """Standalone attention_chunk_stats of one chunk (no mask): 4 * d flops per (query, key) pair."""
    B, Hq, Lq, d = q.shape
    steps = int(min(500, max(10, math.ceil(0.2 / call_seconds(lambda: ra.attention_chunk_stats(
        q, k0, v0, scale=scale), torch)))))
    ms, kernel_ms = timed_with_kernel(lambda: ra.attention_chunk_stats(q, k0, v0, scale=scale), steps, 5, torch,
                                      ra.api)
    flops = 4 * d * Hq * B * Lq * k0.shape[2]
    return {"ms": round(ms, 4), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 2),
            "kernel_ms": round(kernel_ms, 4), "kernel_TFLOP/s": round(flops / (kernel_ms * 1e-3) / 1e12, 2),
            "frac_of_bf16_peak": round(flops / (kernel_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "steps": steps, "shape": f"{Lq} queries x {k0.shape[2]} keys, {Hq} heads, d={d}"}


def block_sparse_leg(torch, ra, wl, dev="cuda:0"):
    """ring_attention_block_sparse on a non-causal share of 8 heads, d = 128, 8192 queries against 65536 keys
    in 8 shards, under random block masks of 256 x 512 positions at several densities. Counted flops: 4 * d
    per allowed (query, key) pair and query head, so equal TFLOP/s at every density means time proportional
    to density."""
    import numpy as np

    P, L = 8, 8192
    w = wl.custom("block_sparse_h8_d128_q8k_k64k", "bf16", 1, 8, 8, 128, [(0, L)],
                  [(j * L, L) for j in wl.ring_order(0, P)], False, seed=106)
    q, k, v, kc, vc = wl.generate_torch(w, dev)
    bq, bk = 256, 512
    nqb, nkb = w.seq_len // bq, w.seq_len // bk
    rows = {}
    base_ms = None
    for density in (1.0, 0.5, 0.25, 0.125):
        rng = np.random.default_rng([106, int(density * 1000)])
        m = (rng.random((nqb, nkb)) < density) if density < 1 else np.ones((nqb, nkb), bool)
        mask = torch.from_numpy(m.astype(np.uint8)).to(dev)
        qpos = np.arange(w.lq)
        allowed = int(m[qpos // bq].sum()) * bk  # every key block holds bk keys
        flops = 4 * w.head_dim * w.q_heads * w.batch * allowed
        ws = torch.empty(ra.api.load_library().ra_block_sparse_workspace_bytes(
            1, w.q_heads, w.head_dim, w.lq, w.lk, len(kc), 1, nqb, nkb), dtype=torch.uint8, device=dev)

        def step():
            return ra.ring_attention_block_sparse(q, kc, vc, mask, bq, bk, 0, w.kv_offsets, workspace=ws)

        ms, kernel_ms = timed_with_kernel(step, 20, 3, torch, ra.api)
        base_ms = base_ms or ms
        rows[f"{density:g}"] = {"block_density": round(float(m.mean()), 4), "ms": round(ms, 4),
                                "kernel_ms": round(kernel_ms, 4),
                                "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 2),
                                "kernel_TFLOP/s": round(flops / (kernel_ms * 1e-3) / 1e12, 2),
                                "ms_over_dense_ms": round(ms / base_ms, 4)}
    return {"shape": f"{w.name}: {bq} x {bk} position blocks, random masks", "by_density": rows}


def merge_leg(args, torch, ra, dev="cuda:0"):
    """Standalone merge at the 32-head, d=128, 8192-row shape with 4 rotating buffer pairs (1.6 GB, beyond
    the 256 MB last-level cache), next to a device copy of the same byte count."""
    rows, d = MERGE_ROWS, MERGE_D
    sets = [(torch.randn(rows, d, device=dev), torch.rand(rows, device=dev) + 0.5,
             torch.randn(rows, device=dev)) for _ in range(8)]
    it = [0]

    def merge_step():
        i = it[0]
        it[0] = (i + 2) % 8
        ra.merge_chunk_stats(sets[i], sets[i + 1], inplace=True)

    ms_m = timed(merge_step, 200, 20, torch)
    mbytes = 12 * (d + 2) * rows
    srcs = [torch.empty(mbytes // 8, dtype=torch.float32, device=dev) for _ in range(3)]
    dst = torch.empty_like(srcs[0])  # read + write = mbytes
    ci = [0]

    def copy_step():
        j = ci[0]
        ci[0] = (j + 1) % 3
        dst.copy_(srcs[j])

    ms_c = timed(copy_step, 200, 20, torch)
    del sets, srcs, dst
    return {
        "ms": round(ms_m, 4),
        "GB/s": round(mbytes / (ms_m * 1e-3) / 1e9, 1),
        "bytes_per_call": mbytes,
        "frac_of_hbm_peak": round(mbytes / (ms_m * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "device_copy_GB/s": round(mbytes / (ms_c * 1e-3) / 1e9, 1),
        "shape": f"{rows} rows x d={d}, fp32, 4 rotating buffer sets",
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(w, q, kc, vc, offs, seconds):
    """The fp64 oracle, as it stands, on the host cores of this process's affinity mask.

    Tasks are blocks of query rows of one head against every key, taken head by head from the first row;
    a pool of one thread per core runs them with single-threaded BLAS (numpy's element-wise work, such as
    the exponentials, is single-threaded, so one task per core keeps every core busy). New tasks start
    until ``seconds`` have passed; the tasks in flight then finish. The inputs are converted to fp64 host
    arrays before the clock starts (input preparation, like inputs resident in HBM on the GPU side).
    """
    import threading
    from concurrent.futures import FIRST_COMPLETED, ThreadPoolExecutor, wait

    import numpy as np

    import oracle
    from ring_attention_chunk_amd import workloads as wl

    cores = len(os.sched_getaffinity(0))
    workers = max(1, min(cores, 32))
    blas = {}
    try:
        from threadpoolctl import threadpool_info, threadpool_limits

        info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if info:
            blas = {"internal_api": info[0].get("internal_api"), "version": info[0].get("version"),
                    "library": os.path.basename(info[0].get("filepath", ""))}
        limiter = threadpool_limits(limits=1, user_api="blas")
    except Exception:  # pragma: no cover - threadpoolctl missing
        limiter = None
    group = w.q_heads // w.kv_heads
    qpos = wl.q_positions(w)
    kpos_sorted = np.sort(wl.k_positions(w))
    block = int(max(1, min(256, (1 << 26) // max(w.lk, 1))))
    q64 = {}
    kv64 = {}
    lock = threading.Lock()

    def head_inputs(h):
        with lock:
            if h not in q64:
                q64[h] = q[:, h:h + 1].float().cpu().double().numpy()
            hk = h // group
            if hk not in kv64:
                kv64[hk] = ([c[:, hk:hk + 1].float().cpu().double().numpy() for c in kc],
                            [c[:, hk:hk + 1].float().cpu().double().numpy() for c in vc])
            return q64[h], kv64[hk]

    tasks = [(h, r0) for h in range(w.q_heads) for r0 in range(0, w.lq, block)]
    # inputs of the heads the budget can reach, prepared before the clock starts
    for h in range(min(w.q_heads, 1 + (workers * block) // max(w.lq, 1))):
        head_inputs(h)

    def run(task):
        h, r0 = task
        r1 = min(w.lq, r0 + block)
        qh, (kh, vh) = head_inputs(h)
        oracle.attention(qh[:, :, r0:r1], kh, vh, qpos[r0:r1], offs, causal=w.causal, scale=w.softmax_scale,
                         kv_strides=w.kv_strides)
        if w.causal:
            pairs = int(np.searchsorted(kpos_sorted, qpos[r0:r1], side="right").sum())
        else:
            pairs = (r1 - r0) * w.lk
        return 4 * w.head_dim * pairs * w.batch, (r1 - r0) * w.batch, time.perf_counter()

    flops = rows = 0
    t0 = time.perf_counter()
    t_end = t0
    with ThreadPoolExecutor(max_workers=workers) as pool:
        pending = set()
        nxt = 0
        while True:
            # keep every worker busy until the budget is spent (at least one task runs)
            while len(pending) < workers and nxt < len(tasks) and (nxt == 0 or time.perf_counter() - t0 < seconds):
                pending.add(pool.submit(run, tasks[nxt]))
                nxt += 1
            if not pending:
                break
            done, pending = wait(pending, return_when=FIRST_COMPLETED)
            for f in done:
                a, b, t = f.result()
                flops, rows, t_end = flops + a, rows + b, max(t_end, t)
    if limiter is not None:
        limiter.restore_original_limits()
    wall = t_end - t0
    full = wl.counted_flops(w)
    heads_done = sorted({h for h, _ in tasks[:nxt]})
    return {
        "value": flops / wall / 1e12,
        "unit": "TFLOP/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{rows} query rows of {w.name} ({nxt} tasks of up to {block} rows of one head, heads "
                  f"{heads_done[0]}..{heads_done[-1]}, every key each); {wall:.1f} s wall on {workers} threads "
                  f"with 1 BLAS thread each",
        "affinity_cores": cores,
        "cpu_model": _cpu_model(),
        "numpy": np.__version__,
        "blas": blas,
        "rows": rows,
        "wall_s": round(wall, 2),
        "sample_flops": flops,
        "extrapolated_full_config_s": round(wall * full / max(flops, 1), 1),
    }


def profile_run(args):
    """Launches for counter collection; every kernel here is identified by name in the CSVs."""
    import torch

    import ring_attention_chunk_amd as ra
    from ring_attention_chunk_amd import workloads as wl

    dev = "cuda:0"
    w = wl.config(args.config)
    q, k, v, kc, vc = wl.generate_torch(w, dev)
    offs = [o for o, _ in w.chunks]
    for _ in range(args.warmup + args.steps):
        ra.ring_attention(q, kc, vc, w.q_runs, offs, causal=w.causal, scale=w.softmax_scale,
                          kv_position_strides=w.kv_strides)
    torch.cuda.synchronize()
    if args.with_backward:
        out, lse = ra.ring_attention(q, kc, vc, w.q_runs, offs, causal=w.causal, scale=w.softmax_scale,
                                     return_lse=True, kv_position_strides=w.kv_strides)
        g = torch.Generator(device=dev).manual_seed(7)
        dout = torch.randn(q.shape, device=dev, generator=g).to(torch.bfloat16)
        for _ in range(args.warmup + args.steps):
            ra.ring_attention_backward(q, kc, vc, out, lse, dout, w.q_runs, offs, causal=w.causal,
                                       scale=w.softmax_scale, kv_position_strides=w.kv_strides)
        torch.cuda.synchronize()
        del out, lse, dout
    del q, k, v, kc, vc
    # calibration: an elementwise kernel that reads COPY_BYTES and writes COPY_BYTES
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(args.steps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    sets = [(torch.randn(MERGE_ROWS, MERGE_D, device=dev), torch.rand(MERGE_ROWS, device=dev) + 0.5,
             torch.randn(MERGE_ROWS, device=dev)) for _ in range(2)]
    for _ in range(args.steps):
        ra.merge_chunk_stats(sets[0], sets[1], inplace=True)
    torch.cuda.synchronize()
    print(json.dumps({"workload": w.name, "ring_attention_calls": args.warmup + args.steps,
                      "copy_bytes": COPY_BYTES, "copy_calls": args.steps,
                      "merge_bytes": 12 * (MERGE_D + 2) * MERGE_ROWS, "merge_calls": args.steps}))


def _counter_rows(path):
    import csv
    import glob

    files = sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no counter_collection.csv under {path}")
    rows = []
    for fn in files:
        with open(fn) as f:
            rows += list(csv.DictReader(f))
    return rows


def _per_dispatch(rows, name_part, counter, reduce="sum"):
    """Mean over dispatches of the kernel whose name contains name_part (skipping the first one).

    Rows of one dispatch (one per hardware instance) are combined by `reduce`
    ("sum", or "max" as the counter definitions do for GRBM_GUI_ACTIVE).
    """
    vals = {}
    for r in rows:
        if name_part in r["Kernel_Name"] and r["Counter_Name"] == counter:
            key = r.get("Dispatch_Id") or r.get("Correlation_Id")
            x = float(r["Counter_Value"])
            vals[key] = (vals.get(key, 0.0) + x) if reduce == "sum" else max(vals.get(key, x), x)
    seq = [vals[k] for k in sorted(vals, key=lambda x: int(x))]
    if len(seq) > 1:
        seq = seq[1:]
    return sum(seq) / len(seq) if seq else None, len(seq)


def summarize_pmc(args):
    from ring_attention_chunk_amd import workloads as wl

    w = wl.config(args.config)
    dirs = args.summarize_pmc
    if len(dirs) not in (3, 4):
        raise SystemExit("--summarize-pmc takes the FETCH_SIZE, WRITE_SIZE and SQ directories (and optionally a "
                         "second SQ directory of instruction counts)")
    fetch, write, sq = (_counter_rows(d) for d in dirs[:3])
    copy_name = "neg_kernel"
    attn_name = dominant_kernel(w)
    f_copy, _ = _per_dispatch(fetch, copy_name, "FETCH_SIZE")
    w_copy, _ = _per_dispatch(write, copy_name, "WRITE_SIZE")
    f_attn, n_attn = _per_dispatch(fetch, attn_name, "FETCH_SIZE")
    w_attn, _ = _per_dispatch(write, attn_name, "WRITE_SIZE")
    f_merge, _ = _per_dispatch(fetch, "merge_kernel", "FETCH_SIZE")
    w_merge, _ = _per_dispatch(write, "merge_kernel", "WRITE_SIZE")
    # counters read KiB per dispatch; scale each by what it reads for the copy of known size
    fs = (COPY_BYTES / 1024) / f_copy
    ws = (COPY_BYTES / 1024) / w_copy
    attn_bytes = f_attn * 1024 * fs + w_attn * 1024 * ws
    merge_bytes = f_merge * 1024 * fs + w_merge * 1024 * ws
    busy, _ = _per_dispatch(sq, attn_name, "SQ_VALU_MFMA_BUSY_CYCLES")
    gui, _ = _per_dispatch(sq, attn_name, "GRBM_GUI_ACTIVE", reduce="max")
    gui = gui / 8 if gui else gui  # the CSV holds the sum over the 8 XCDs
    durs = {}
    for r in sq:
        if attn_name in r["Kernel_Name"]:
            durs[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    dseq = [durs[k] for k in sorted(durs, key=int)][1:] or list(durs.values())
    dur = sum(dseq) / len(dseq)
    mops, _ = _per_dispatch(sq, attn_name, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    conf, _ = _per_dispatch(sq, attn_name, "SQ_LDS_BANK_CONFLICT")
    lds_act, _ = _per_dispatch(sq, attn_name, "SQ_LDS_IDX_ACTIVE")
    B, Hq, Hkv, d = w.batch, w.q_heads, w.kv_heads, w.head_dim
    algo_bytes = 2 * (B * Hq * w.lq * d + 2 * B * Hkv * w.lk * d) + 4 * B * Hq * w.lq * d
    out = {
        "workload": w.name,
        "kernel": attn_name,
        "source_sha256_16": source_digest(),
        "bytes_per_launch": int(attn_bytes),
        "algorithmic_bytes_per_launch": algo_bytes,
        "fetch_kib_per_launch_raw": f_attn,
        "write_kib_per_launch_raw": w_attn,
        "copy_calibration": {"bytes": COPY_BYTES, "fetch_kib_raw": f_copy, "write_kib_raw": w_copy,
                             "fetch_scale": fs, "write_scale": ws},
        "mfma_busy_pct_of_gui_active": 100.0 * busy / (gui * SIMD_NUM) if busy and gui else None,
        "mfma_busy_pct_of_duration_at_2p4ghz": 100.0 * busy / (dur * 2.4e9 * SIMD_NUM) if busy else None,
        "profiled_duration_us": dur * 1e6,
        # the shader clock while the kernel ran: active cycles of one XCD over the kernel's duration
        "sclk_ghz_under_load": gui / dur / 1e9 if gui else None,
        "clock_derived_bf16_peak_tflops": 256 * (gui / dur) * 4096 / 1e12 if gui else None,
        "mfma_bf16_flops_per_launch": mops * 512 if mops else None,
        "counted_flops_per_launch": wl.counted_flops(w),
        "lds_bank_conflict_pct_of_lds_active": 100.0 * conf / lds_act if conf is not None and lds_act else None,
        "merge": {"bytes_per_call_counted": int(merge_bytes), "algorithmic_bytes_per_call": 12 * (MERGE_D + 2) *
                  MERGE_ROWS},
        "dispatches_averaged": n_attn,
        "commands": args.command,
    }
    if len(dirs) == 4:
        ins = _counter_rows(dirs[3])
        names = sorted({r["Counter_Name"] for r in ins})
        per = {}
        for c in names:
            per[c], _ = _per_dispatch(ins, attn_name, c)
        valu, mfma = per.get("SQ_INSTS_VALU"), per.get("SQ_INSTS_MFMA")
        per["valu_per_mfma"] = valu / mfma if valu and mfma else None
        out["instruction_counters_per_launch"] = per
    # the gradient kernels, when the profiled run included the backward pass
    bwd = {}
    for kname in ("dkdv_kernel", "dq_kernel"):
        b_busy, n_b = _per_dispatch(sq, kname, "SQ_VALU_MFMA_BUSY_CYCLES")
        if not b_busy:
            continue
        b_gui, _ = _per_dispatch(sq, kname, "GRBM_GUI_ACTIVE", reduce="max")
        b_mops, _ = _per_dispatch(sq, kname, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
        b_conf, _ = _per_dispatch(sq, kname, "SQ_LDS_BANK_CONFLICT")
        b_lds, _ = _per_dispatch(sq, kname, "SQ_LDS_IDX_ACTIVE")
        bwd[kname] = {"mfma_busy_pct_of_gui_active": 100.0 * b_busy / (b_gui / 8 * SIMD_NUM) if b_gui else None,
                      "mfma_bf16_flops_per_launch": b_mops * 512 if b_mops else None,
                      "lds_bank_conflict_pct_of_lds_active": 100.0 * b_conf / b_lds if b_lds else None,
                      "dispatches_averaged": n_b}
    if bwd:
        out["backward_kernels"] = bwd
    path = os.path.join(ROOT, "profiles", f"{attn_name}_{w.name}_hbm_traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


_MODES = {"0": "stats", "1": "ring full", "2": "ring causal"}
_MASKS = {"0": "no mask", "1": "mask", "2": "strided mask"}


def _kernel_label(name):
    import re

    m = re.search(r"attention_bf16_kernel<(\d+), (\d), (\d)(?:, (true|false))?>", name)
    if m:
        sp = ", block-sparse" if m.group(4) == "true" else ""
        return f"attention_bf16_kernel<{m.group(1)}, {_MODES[m.group(2)]}, {_MASKS[m.group(3)]}{sp}>"
    m = re.search(r"attention_kernel<([\w_ ]+), (\d+), (\d)(?:, (true|false))?>", name)
    if m:
        sp = ", block-sparse" if m.group(4) == "true" else ""
        return f"attention_kernel<{m.group(1)}, {m.group(2)}, {_MODES[m.group(3)]}{sp}>"
    for k in ("sparse_bits_kernel", "sparse_plan_kernel"):
        if k in name:
            return k
    m = re.search(r"(dkdv_kernel|dq_kernel)<(\d+)(?:, (true|false))?>", name)
    if m:
        return f"{m.group(1)}<{m.group(2)}{', causal' if m.group(3) == 'true' else ''}>"
    for k in ("dq_reduce_kernel", "delta_kernel", "bwd_positions_kernel", "merge_kernel", "combine_kernel",
              "upload_kernel", "__amd_rocclr_copyBuffer"):
        if k in name:
            return k
    return None


def summarize_trace(args):
    """Kernel-trace summary of one run of this script: this library's kernels from run_kernel_stats.csv,
    and, for each timed share of the JSON line, its attention kernel's average against the kernel timer."""
    import csv
    import glob
    import re

    from ring_attention_chunk_amd import workloads as wl

    tdir, jpath = args.summarize_trace
    files = sorted(glob.glob(os.path.join(tdir, "**", "*kernel_stats.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {tdir}")
    rows = list(csv.DictReader(open(files[0])))
    with open(jpath) as f:
        d = json.loads([ln for ln in f.read().splitlines() if ln.startswith("{")][-1])
    stats = {}
    for r in rows:
        lab = _kernel_label(r["Name"])
        if lab:
            prev = stats.get(lab)
            calls = int(r["Calls"])
            tot = float(r["TotalDurationNs"]) if "TotalDurationNs" in r else float(r["AverageNs"]) * calls
            if prev:
                calls += prev[0]
                tot += prev[1]
            stats[lab] = (calls, tot, min(float(r["MinNs"]), prev[2] if prev else 1e30),
                          max(float(r["MaxNs"]), prev[3] if prev else 0.0))
    head = d["config"]["workload"]
    out = [f"# attention_bf16_kernel: kernel trace of the benchmark (headline {head})", "",
           "Command (GPU box, from the repository root):", "", "```", args.command, "```", "",
           "From `kernel_stats.csv` (this library's kernels; durations in µs):", "",
           "| Kernel | Calls | Average µs | Min µs | Max µs |", "|---|---|---|---|---|"]
    for lab, (calls, tot, mn, mx) in sorted(stats.items(), key=lambda kv: -kv[1][1]):
        out.append(f"| {lab} | {calls} | {tot / calls / 1e3:.1f} | {mn / 1e3:.1f} | {mx / 1e3:.1f} |")
    out += ["", "Each share's attention kernel in the trace, averaged over the dispatches of its timed calls (taken "
            "from kernel_trace.csv in launch order), against the library's kernel timer over the same calls:", "",
            "| Share | Kernel | Trace average µs | TFLOP/s (trace) | % of 2500 | Kernel timer µs | TFLOP/s (timer) |",
            "|---|---|---|---|---|---|---|"]
    # dispatches of each kernel in launch order (kernel_trace.csv): a share's calls are the next
    # (estimate calls + settle + warm-up + steps) dispatches of its kernel variant, shares in the order the
    # benchmark runs them (the headline first, then the configs block)
    traces = sorted(glob.glob(os.path.join(tdir, "**", "*kernel_trace.csv"), recursive=True))
    disp = {}
    if traces:
        rows_t = list(csv.DictReader(open(traces[0])))
        key = "Dispatch_Id" if "Dispatch_Id" in rows_t[0] else "Correlation_Id"
        for r in sorted(rows_t, key=lambda r: int(r[key])):
            lab = _kernel_label(r["Kernel_Name"])
            if lab:
                disp.setdefault(lab, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    shares = [(head, d["roofline"]["kernel_ms"], d["config"]["counted_flops"],
               d["clock_settle"]["calls"] + d["warmup"] + d["steps"], d["steps"])]
    for name, e in d.get("configs", {}).items():
        shares.append((name, e["kernel_ms"], e["counted_flops"], 2 + e["clock_settle_calls"] + e["warmup"] + e["steps"],
                       e["steps"]))
    by_name = {wl.config(i).name: wl.config(i) for i in wl.CONFIGS}
    used = {}
    for name, kms, flops, ncalls, nsteps in shares:
        w = by_name.get(name)
        if w is None:
            continue
        mode = "2" if w.causal else "1"
        mask = ("2" if w.pos_stride != 1 else "1") if w.causal else ("1" if w.lk % (64 if w.head_dim > 64 else 128)
                                                                    else "0")
        dp = 32 if w.head_dim <= 32 else (64 if w.head_dim <= 64 else 128)
        lab = f"attention_bf16_kernel<{dp}, {_MODES[mode]}, {_MASKS[mask]}>"
        seq = disp.get(lab, [])
        first = used.get(lab, 0)
        mine = seq[first:first + ncalls]
        used[lab] = first + ncalls
        if not mine:
            continue
        timed_calls = mine[-nsteps:]  # the timed calls are the last of the share's calls
        avg = sum(timed_calls) / len(timed_calls)
        out.append(f"| {name} | {lab} | {avg:.1f} | {flops / (avg * 1e-6) / 1e12:.0f} | "
                   f"{100 * flops / (avg * 1e-6) / 1e12 / BF16_PEAK_TFLOPS:.1f} | {kms * 1e3:.1f} | "
                   f"{flops / (kms * 1e-3) / 1e12:.0f} |")
    out += ["", f"Kernel source digest {source_digest()} (sha256 of attention.hip without comments)."]
    path = os.path.join(ROOT, "profiles", f"attention_bf16_kernel_{head}_kernel_trace.md")
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(args)
        return
    if args.summarize_trace:
        summarize_trace(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build runs the whole share on a single MI355X and has no "
              "multi-GPU path; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import ring_attention_chunk_amd as ra
    from ring_attention_chunk_amd import workloads as wl

    ra.load_library()
    if args.profile_run:
        profile_run(args)
        return
    dev = "cuda:0"
    w = wl.config(args.config)
    entry, (q, kc, vc, offs) = measure_share(w, args.steps, args.warmup, args.settle_seconds, torch, ra, wl, dev)
    flops = entry["counted_flops"]
    peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
    result = {
        "metric": "ring_attention TFLOP/s at 1 GPU (counted 4*d*Hq*allowed pairs) and % of bf16 MFMA peak",
        "value": entry["TFLOP/s"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle": {"calls": entry["clock_settle_calls"], "seconds": args.settle_seconds,
                         "note": "untimed calls before the warm-up, outside the timed region"},
        "ms_per_step": entry["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": dict(describe(w), counted_flops=flops),
        "roofline": {
            "bound": "mfma",
            "kernel": dominant_kernel(w),
            "kernel_ms": entry["kernel_ms"],
            "achieved": entry["kernel_TFLOP/s"],
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": entry["frac"],
            "traffic": traffic_for(w),
        },
        "pct_of_bf16_peak": round(100 * entry["TFLOP/s"] / BF16_PEAK_TFLOPS, 2),
        "clock_derived_peak": clock_derived_peak(w, entry["kernel_TFLOP/s"]),
        "kernel_source_sha256_16": source_digest(),
    }

    legs = {}
    if not args.no_legs:
        legs["attention_chunk_stats_d128"] = stats_leg(q, kc[0], vc[0], w.softmax_scale, args, torch, ra)
        if w.dtype == "bf16" and w.head_dim % 8 == 0:
            legs["ring_attention_backward"] = backward_leg(w, q, kc, vc, offs, args, torch, ra)
    baseline = None
    if not args.no_cpu_baseline:
        baseline = cpu_baseline(w, q, kc, vc, offs, args.cpu_seconds)
    del q, kc, vc
    torch.cuda.empty_cache()

    configs = {}
    for tok in [t for t in args.configs.split(",") if t.strip()]:
        i = int(tok)
        if i == args.config:
            continue
        wi = wl.config(i)
        e, inputs = measure_share(wi, None, 3, 0.5, torch, ra, wl, dev)
        e["config"] = describe(wi)
        configs[wi.name] = e
        if i == 1 and not args.no_legs:
            qi, kci, vci, _ = inputs
            legs["attention_chunk_stats"] = stats_leg(qi, kci[0], vci[0], wi.softmax_scale, args, torch, ra)
        del inputs
        torch.cuda.empty_cache()
    if configs:
        result["configs"] = configs
    if not args.no_legs:
        legs["merge_chunk_stats"] = merge_leg(args, torch, ra, dev)
        legs["ring_attention_block_sparse"] = block_sparse_leg(torch, ra, wl, dev)
        result["legs"] = legs
    if baseline is not None:
        result["cpu_baseline"] = baseline
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

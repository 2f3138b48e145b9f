#!/usr/bin/env python3
"""Benchmark of the ring-attention hot path on one MI355X.

One step is one ``ring_attention`` call over one device's full share (every
key/value chunk, in ring order, with the causal mask if the workload has one),
with inputs already resident in HBM. The JSON line reports the counted
throughput ``4 * d * Hq * (allowed query-key pairs)`` per second, the roofline
of the attention kernel (bf16 MFMA bound), the standalone chunk-statistics and
merge legs (the merge is HBM-bound, next to a device copy of the same size),
and the fp64 CPU oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config I]
"""

import argparse
import hashlib
import json
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


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed calls first (default: as many as take about one second, so that the "
                         "GPU clocks have settled under load; a cold GPU times several percent slow)")
    ap.add_argument("--config", type=int, default=1, help="workload index (1 is the reported workload)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-legs", action="store_true", help="skip the chunk-stats and merge legs")
    ap.add_argument("--profile-run", action="store_true",
                    help="launch sequence for rocprofv3 counter passes: the workload's ring_attention, a device "
                         "copy of COPY_BYTES, then the merge leg; prints what was launched")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "SQ_DIR"),
                    help="turn the counter CSVs of the three --profile-run passes into profiles/ summaries")
    ap.add_argument("--command", default="", help="with --summarize-pmc: the command lines that made the CSVs")
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


def settle_warmup(fn, torch, seconds=1.0, cap=5000):
    """Number of untimed calls that take about `seconds` (at least 5), from one timed call."""
    fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    dt = max(time.perf_counter() - t0, 1e-6)
    return int(min(cap, max(5, round(seconds / dt))))


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
    ws = torch.empty(ra.api.backward_workspace_bytes(tuple(q.shape), [c.shape[2] for c in kc]), dtype=torch.uint8,
                     device=dev)

    def step():
        return ra.ring_attention_backward(q, kc, vc, out, lse, dout, w.q_runs, offs, causal=w.causal,
                                          scale=w.softmax_scale, kv_position_strides=w.kv_strides, workspace=ws)

    steps = max(5, min(args.steps, 20))
    ms, pair_ms = timed_with_kernel(step, steps, 3, torch, ra.api)
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


def dominant_kernel(w):
    """Name of the kernel that does a workload's attention: every bf16 workload here (aligned rows,
    whole 16-byte pieces) runs the pipelined bf16 kernel, fp32 the general one."""
    return "attention_bf16_kernel" if w.dtype == "bf16" else "attention_kernel"


def traffic_for(w):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match this source."""
    path = os.path.join(ROOT, "profiles", f"{dominant_kernel(w)}_{w.name}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha256_16") != source_digest():
        return None  # the kernel changed since the counters were taken
    return t.get("bytes_per_launch")


def cpu_baseline(w, q, kc, vc, offs, seconds):
    """The fp64 oracle on host cores over whole row blocks of the same share, for ~`seconds`."""
    import numpy as np

    import oracle
    from ring_attention_chunk_amd import workloads as wl

    try:
        from threadpoolctl import threadpool_info

        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        cores = 1
    qpos = wl.q_positions(w)
    qh = q.cpu()
    kh = [c.cpu() for c in kc]
    vh = [c.cpu() for c in vc]
    block = 256
    flops, rows, t0 = 0, 0, time.perf_counter()
    kpos = np.sort(wl.k_positions(w))
    h = 0
    r0 = 0
    while time.perf_counter() - t0 < seconds:
        r1 = min(w.lq, r0 + block)
        oracle.attention(qh[:, h:h + 1, r0:r1], [c[:, (h * w.kv_heads) // w.q_heads:][:, :1] for c in kh],
                         [c[:, (h * w.kv_heads) // w.q_heads:][:, :1] for c in vh], qpos[r0:r1], offs,
                         causal=w.causal, scale=w.softmax_scale, kv_strides=w.kv_strides)
        pairs = (r1 - r0) * w.lk if not w.causal else int(np.searchsorted(kpos, qpos[r0:r1], side="right").sum())
        flops += 4 * w.head_dim * pairs * w.batch
        rows += (r1 - r0) * w.batch
        r0 = r1
        if r0 >= w.lq:
            r0, h = 0, (h + 1) % w.q_heads
    wall = time.perf_counter() - t0
    return {
        "value": flops / wall / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{rows} query rows (blocks of {block} rows, head by head, every key) of {w.name}; "
                  f"{wall:.1f} s wall; numpy fp64 on {platform.processor() or platform.machine()}",
    }


def profile_run(args):
    """Launches for counter collection; every kernel here is identified by name in the CSVs."""
    import torch

    import ring_attention_chunk_amd as ra
    from ring_attention_chunk_amd import workloads as wl

    dev = "cuda:0"
    if args.warmup is None:
        args.warmup = 1
    w = wl.config(args.config)
    q, k, v, kc, vc = wl.generate_torch(w, dev)
    offs = [o for o, _ in w.chunks]
    for _ in range(args.warmup + args.steps):
        ra.ring_attention(q, kc, vc, w.q_runs, offs, causal=w.causal, scale=w.softmax_scale,
                          kv_position_strides=w.kv_strides)
    torch.cuda.synchronize()
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
    fetch, write, sq = (_counter_rows(d) for d in args.summarize_pmc)
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
        "mfma_bf16_flops_per_launch": mops * 512 if mops else None,
        "counted_flops_per_launch": wl.counted_flops(w),
        "lds_bank_conflict_pct_of_lds_active": 100.0 * conf / lds_act if conf is not None and lds_act else None,
        "merge": {"bytes_per_call_counted": int(merge_bytes), "algorithmic_bytes_per_call": 12 * (MERGE_D + 2) *
                  MERGE_ROWS},
        "dispatches_averaged": n_attn,
        "commands": args.command,
    }
    path = os.path.join(ROOT, "profiles", f"{attn_name}_{w.name}_hbm_traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(args)
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
    q, k, v, kc, vc = wl.generate_torch(w, dev)
    offs = [o for o, _ in w.chunks]
    flops = wl.counted_flops(w)
    ws = torch.empty(ra.api.workspace_bytes(tuple(q.shape), [c.shape[2] for c in kc], len(w.q_segments)),
                     dtype=torch.uint8, device=dev)

    def step():
        return ra.ring_attention(q, kc, vc, w.q_runs, offs, causal=w.causal, scale=w.softmax_scale,
                                 workspace=ws, kv_position_strides=w.kv_strides)

    if args.warmup is None:
        args.warmup = settle_warmup(step, torch)
    ms, kernel_ms = timed_with_kernel(step, args.steps, args.warmup, torch, ra.api)
    tflops = flops / (ms * 1e-3) / 1e12
    # the roofline is the attention kernel's: its algorithmic flops per launch over its own average
    # device time, from HIP events the library records around that launch on the call's stream
    kernel_tflops = flops / (kernel_ms * 1e-3) / 1e12
    peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
    traffic = traffic_for(w)
    result = {
        "metric": "ring_attention TFLOP/s at 1 GPU (counted 4*d*Hq*allowed pairs) and % of bf16 MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
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
            "counted_flops": flops,
        },
        "roofline": {
            "bound": "mfma",
            "kernel": dominant_kernel(w),
            "kernel_ms": round(kernel_ms, 4),
            "achieved": round(kernel_tflops, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(kernel_tflops / peak, 4),
            "traffic": traffic,
        },
        "pct_of_bf16_peak": round(100 * tflops / BF16_PEAK_TFLOPS, 2),
        "kernel_source_sha256_16": source_digest(),
    }

    if not args.no_legs:
        legs = {}
        # standalone attention_chunk_stats on one shard of the share
        k0, v0 = kc[0], vc[0]
        ms_s = timed(lambda: ra.attention_chunk_stats(q, k0, v0, scale=w.softmax_scale), args.steps,
                     args.warmup, torch)
        f_s = 4 * w.head_dim * w.q_heads * w.batch * w.lq * k0.shape[2]
        legs["attention_chunk_stats"] = {"ms": round(ms_s, 4), "TFLOP/s": round(f_s / (ms_s * 1e-3) / 1e12, 2),
                                         "shape": f"{w.lq} queries x {k0.shape[2]} keys, {w.q_heads} heads"}
        # standalone merge at the 32-head, d=128, 8192-row shape; 4 rotating buffer sets
        rows, d = 32 * 8192, 128
        sets = [(torch.randn(rows, d, device=dev), torch.rand(rows, device=dev) + 0.5,
                 torch.randn(rows, device=dev)) for _ in range(8)]
        it = [0]

        def merge_step():
            i = it[0]
            it[0] = (i + 2) % 8
            ra.merge_chunk_stats(sets[i], sets[i + 1], inplace=True)

        ms_m = timed(merge_step, max(args.steps, 20), args.warmup, torch)
        mbytes = 12 * (d + 2) * rows
        src = torch.empty(mbytes // 8, dtype=torch.float32, device=dev)  # read + write = mbytes
        dst = torch.empty_like(src)
        srcs = [torch.empty_like(src) for _ in range(3)]
        ci = [0]

        def copy_step():
            j = ci[0]
            ci[0] = (j + 1) % 3
            dst.copy_(srcs[j])

        ms_c = timed(copy_step, max(args.steps, 20), args.warmup, torch)
        legs["merge_chunk_stats"] = {
            "ms": round(ms_m, 4),
            "GB/s": round(mbytes / (ms_m * 1e-3) / 1e9, 1),
            "bytes_per_call": mbytes,
            "frac_of_hbm_peak": round(mbytes / (ms_m * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "device_copy_GB/s": round(mbytes / (ms_c * 1e-3) / 1e9, 1),
            "shape": f"{rows} rows x d={d}, fp32, 4 rotating buffer sets",
        }
        del sets, src, dst, srcs
        if w.dtype == "bf16" and w.head_dim % 8 == 0:
            legs["ring_attention_backward"] = backward_leg(w, q, kc, vc, offs, args, torch, ra)
        result["legs"] = legs

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, q, kc, vc, offs, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Paged decode attention benchmark on one MI355X.

Workload: one decode step of one layer over 32 requests x 4096-token histories
(Hq 32, Hkv 8, d 128, B 16, bf16 K/V, fp32 accumulation, 8192-block pool,
shuffled block tables), the largest single-GPU batch of the five workloads.
A step is one paged_attn_decode call: the split-K pass over every logical
block plus the merge of the partial states.  The pool is fully used by the
histories, so the step has no append.

Four copies of the pools (2 GiB) are rotated so consecutive steps do not hit
in the 256 MB Infinity Cache.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--splits 0]
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "paged decode attention KV GB/s (% of MI355X HBM peak) + tokens/s per layer"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_bf16_32x4096_traffic.txt")
KERNEL_SRCS = [os.path.join(ROOT, "paged_kv_cache_352_amd", "csrc", f) for f in ("pa_decode.hip", "pa_decode_mfma.hip")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sha():
    """sha256 over the decode kernel sources, in a fixed order."""
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current decode kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_sha():
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(b, min_seconds):
    """The float64 oracle on the host cores, over whole passes of the same batch."""
    from oracle import attention as att

    k = b.k_pool[0].float().cpu().numpy()
    v = b.v_pool[0].float().cpu().numpy()
    q = b.q[0].float().cpu().numpy()
    tab = b.block_tables.cpu().numpy()
    lens = b.seq_lens.cpu().numpy()
    rows = 0
    wall0, cpu0 = time.perf_counter(), time.process_time()
    while True:
        for s in range(b.S):
            att.paged_decode_rows(q, k, v, tab, lens, b.B, b.scale, [s])
            rows += 1
            if time.perf_counter() - wall0 >= min_seconds and rows >= 1:
                break
        if time.perf_counter() - wall0 >= min_seconds:
            break
    wall = time.perf_counter() - wall0
    cpu = time.process_time() - cpu0
    kv_bytes = rows * int(lens[0]) * 2 * b.Hkv * b.D * 2
    return {
        "value": kv_bytes / wall / 1e9,
        "unit": "GB/s",
        "cores": max(1, round(cpu / wall)),
        "kind": "oracle",
        "sample": f"{rows} of the batch's 32 requests (float64 gather + dense attention), "
                  f"{wall:.1f} s wall, {cpu:.1f} s CPU; host has {os.cpu_count()} CPUs",
    }


def calibrate_copy(torch, dev, n_bytes=1 << 30, reps=5):
    """A plain elementwise copy of known size: torch.neg over float32, n_bytes in, n_bytes out."""
    src = torch.ones(n_bytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "float32 neg copy", "bytes_read_per_dispatch": n_bytes,
                      "bytes_written_per_dispatch": n_bytes, "dispatches": reps}), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--splits", type=int, default=0, help="0 = library's choice")
    ap.add_argument("--rotate", type=int, default=4, help="pool copies cycled across steps")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB float32 negate-copy kernel (reads 1 GiB, writes 1 GiB) "
                         "a few times, to scale the HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode path has no "
              "multi-GPU mode in this build.", file=sys.stderr)
        return 2

    import torch

    import paged_kv_cache_352_amd as pa
    import workloads as W

    if not os.path.exists(pa.LIB_PATH):
        from paged_kv_cache_352_amd.build import build

        build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        return calibrate_copy(torch, dev)
    b = W.config2(device=dev)
    kv_bytes = b.valid_kv_bytes_per_layer()
    pools = [(b.k_pool[0], b.v_pool[0])]
    for _ in range(args.rotate - 1):
        pools.append((b.k_pool[0].clone(), b.v_pool[0].clone()))
    out = torch.empty((b.S, b.Hq, b.D), dtype=torch.float32, device=dev)
    first = pa.DecodeLaunch(b.q[0], pools[0][0], pools[0][1], b.block_tables, b.seq_lens, b.B, b.scale,
                            out=out, num_splits=args.splits)
    calls = [first] + [pa.DecodeLaunch(b.q[0], k, v, b.block_tables, b.seq_lens, b.B, b.scale, out=out,
                                       num_splits=args.splits, workspace=first.workspace) for k, v in pools[1:]]
    log(f"workload {b.name}: {kv_bytes / 1e6:.1f} MB valid KV per step, splits={first.splits}")

    for i in range(args.warmup):
        calls[i % len(calls)].launch()
    torch.cuda.synchronize()

    # Timed region: K steps back to back on the current stream, bracketed by
    # synchronisation; value = valid KV bytes per step / time per step.
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(args.steps):
        calls[i % len(calls)].launch()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / args.steps

    # Per-launch durations for the roofline: the same K launches, each
    # bracketed by HIP events recorded on the stream the library launches on.
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.steps):
        starts[i].record(stream)
        calls[i % len(calls)].launch()
        ends[i].record(stream)
    torch.cuda.synchronize()
    launch_ms = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    mean_launch_ms = sum(launch_ms) / len(launch_ms)
    log(f"ms/step {ms_step:.4f} (wall {wall * 1e3 / args.steps:.4f}); per-launch mean {mean_launch_ms:.4f} "
        f"p10 {launch_ms[len(launch_ms) // 10]:.4f} p90 {launch_ms[len(launch_ms) * 9 // 10]:.4f} ms")

    gbs = kv_bytes / (ms_step * 1e-3) / 1e9
    achieved = kv_bytes / (mean_launch_ms * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "accumulate": "f32",
        "data": "synthetic",
        "config": {
            "workload": "decode step, 32 requests x 4096-token history, Hq 32 / Hkv 8, d 128, B 16, bf16 K/V, "
                        "8192-block pool, shuffled tables, one layer",
            "requests": b.S, "history": 4096, "q_heads": b.Hq, "kv_heads": b.Hkv, "head_dim": b.D,
            "block_size": b.B, "pool_blocks": b.NB, "splits": first.splits, "pool_copies_rotated": len(calls),
        },
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "tokens_per_s_per_layer": round(b.S / (ms_step * 1e-3), 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "kernel": "one paged_attn_decode launch (decode kernel, plus the split merge when it splits)",
            "algorithmic_bytes_per_launch": kv_bytes,
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(b, args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

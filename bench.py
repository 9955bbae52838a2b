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
KERNEL_SRCS = [os.path.join(ROOT, "paged_kv_cache_352_amd", "csrc", f)
               for f in ("pa_decode.hip", "pa_decode_mfma.hip", "pa_mfma_common.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sha():
    """sha256 over the decode kernel sources (kernels, shared device helpers), in a fixed order."""
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current decode kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as fh:
        lines = fh.read().splitlines()
    for line in lines:
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_sha():
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def _blas_threads():
    """Threads numpy's BLAS may use in this process (threadpoolctl), else the CPUs we may run on."""
    try:
        from threadpoolctl import threadpool_info

        n = [p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:  # pragma: no cover - threadpoolctl absent
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(b, min_seconds, gpu_out=None):
    """The float64 oracle on the host cores, request by request over the same batch.

    Runs whole request passes (gather through the table, then dense attention)
    for about ``min_seconds``, cycling over the batch's requests.  When
    ``gpu_out`` (the GPU's output for the same step) is given, the rows the
    oracle computed are also compared with it."""
    import numpy as np

    from oracle import attention as att

    k = b.k_pool[0].float().cpu().numpy()
    v = b.v_pool[0].float().cpu().numpy()
    q = b.q[0].float().cpu().numpy()
    tab = b.block_tables.cpu().numpy()
    lens = b.seq_lens.cpu().numpy()
    passes = 0
    ref = {}
    wall0, cpu0 = time.perf_counter(), time.process_time()
    while time.perf_counter() - wall0 < min_seconds:
        s = passes % b.S
        ref[s] = att.paged_decode_rows(q, k, v, tab, lens, b.B, b.scale, [s])[s]
        passes += 1
    wall = time.perf_counter() - wall0
    cpu = time.process_time() - cpu0
    kv_bytes = sum(int(lens[i % b.S]) for i in range(passes)) * 2 * b.Hkv * b.D * b.elem_bytes
    res = {
        "value": kv_bytes / wall / 1e9,
        "unit": "GB/s",
        "cores": _blas_threads(),
        "kind": "oracle",
        "sample": f"{passes} request passes cycling over the {b.S}-request batch ({len(ref)} distinct requests; "
                  f"float64 gather + dense attention), {wall:.1f} s wall, {cpu:.1f} s CPU",
        "cpu_time_over_wall": round(cpu / wall, 2),
        "host_cpus": os.cpu_count(),
        "host_cpus_usable": len(os.sched_getaffinity(0)),
    }
    if gpu_out is not None:
        got = gpu_out.cpu().numpy()
        rows = sorted(ref)
        want = np.stack([ref[s] for s in rows])
        err = float(np.max(np.abs(got[rows].astype(np.float64) - want)))
        top = float(np.max(np.abs(want)))
        res["max_abs_err_vs_oracle"] = err
        res["max_err_over_max_out"] = err / top if top else 0.0
        res["tolerance"] = "5e-3 * max|out| (bf16 K/V, fp32 accumulation)"
        res["rows_compared"] = len(rows)
    return res


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


def graph_time_us(torch, enqueue, launches, replays=5, settle_s=0.25):
    """Mean GPU time per launch, in microseconds, of ``launches`` calls of
    ``enqueue()`` captured in one HIP graph and replayed back to back.

    Used for kernels too short to time one by one from Python: the graph
    keeps the GPU fed, so the time is kernel time plus the graph's own
    inter-kernel gap.  Before the timed replays the graph is replayed for
    ``settle_s`` seconds, untimed, so that the clocks have come up from the
    idle of the workload's set-up (as the headline run's settle does): timed
    straight after a set-up pause, a launch read up to 9 % slower."""
    enqueue()  # load the library and settle shapes outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(launches):
            enqueue()
    g.replay()
    torch.cuda.synchronize()
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < settle_s:
        g.replay()
        torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(replays):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / (replays * launches)
    del g
    return us


def rate(nbytes, us):
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"us": round(us, 3), "bytes": int(nbytes), "GB_s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def side_kernels(torch, pa, W, dev):
    """kv_append and kv_cow_copy at their workload shapes (one layer).

    kv_append: 256 requests x (K + V) of one token, Hkv 8, d 128, bf16: each
    launch reads 2 x 256 x 2 KiB of new K/V and writes as much into the pool.
    kv_cow_copy: the 63 copy-on-write pairs of the prefix-sharing batch, t
    valid slots each: reads and writes 63 x t x 2 KiB per pool.
    Both move about a megabyte or less, so their time is launch latency, not
    bandwidth; the fraction of peak is reported for completeness."""
    res = {}
    b = W.config3(device=dev, layers=1)
    row = b.Hkv * b.D * b.elem_bytes
    n_app = int((b.append_positions[0] >= 0).sum().item())
    us = graph_time_us(torch, lambda: pa.kv_append(b.k_pool[0], b.v_pool[0], b.k_new[0, 0], b.v_new[0, 0],
                                                    b.block_tables, b.append_positions[0], b.B), 64)
    res["kv_append"] = dict(rate(2 * 2 * n_app * row, us), workload=f"{n_app} requests, Hkv 8, d 128, bf16, one layer")
    del b
    b = W.config4(device=dev)
    t = int(b.info["t"])
    npairs = int(b.cow_src.numel())
    us = graph_time_us(torch, lambda: pa.kv_cow_copy(b.k_pool, b.v_pool, b.cow_src, b.cow_dst, b.cow_n, b.B), 64)
    res["kv_cow_copy"] = dict(rate(2 * 2 * npairs * t * row, us),
                              workload=f"{npairs} pairs x {t} valid slots, Hkv 8, d 128, bf16, one layer")
    del b
    torch.cuda.empty_cache()
    return res


def swap_time(torch, pa, b, dev, nblocks=250, reps=3):
    """Swap-out and swap-in of nblocks blocks in every layer through pinned host
    memory: 250 blocks x 32 layers x 64 KiB = 500 MiB, the amount the pages'
    recovery-cost example moves (4,000 tokens at 128 KiB per token)."""
    ids = torch.arange(nblocks, dtype=torch.int32, device=dev)
    buf = torch.empty((b.L, 2, nblocks, b.B, b.Hkv, b.D), dtype=b.dtype, pin_memory=True)
    nbytes = buf.numel() * buf.element_size()
    res = {}
    for name, fn in (("out", pa.kv_swap_out), ("in", pa.kv_swap_in)):
        fn(b.k_pool, b.v_pool, ids, buf, b.B)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            fn(b.k_pool, b.v_pool, ids, buf, b.B)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / reps
        res[f"{name}_ms"] = round(ms, 3)
        res[f"{name}_GiB_s"] = round(nbytes / (ms * 1e-3) / 2**30, 2)
    res["bytes"] = nbytes
    del buf
    return res


def suite(torch, pa, W, dev):
    """Decode (and full-step) timings of the other four workloads, one dict each."""
    out = {}

    def decode_graph(b, layers, reps=1, order=None):
        calls = [pa.DecodeLaunch(b.q[layer], b.k_pool[layer], b.v_pool[layer], b.block_tables, b.seq_lens, b.B,
                                 b.scale, order=order) for layer in layers]
        def launch_all():
            for c in calls:
                c.launch()

        us = graph_time_us(torch, launch_all, reps)
        return us / len(calls), calls[0].splits

    def full_step_graph(b, fused=False, all_layers=False, ordered=False):
        def step():
            order = pa.paged_attn_order(b.seq_lens, out=order_buf) if ordered else None  # once per step
            if b.cow_src.numel():
                pa.kv_cow_copy(b.k_pool, b.v_pool, b.cow_src, b.cow_dst, b.cow_n, b.B)
            if all_layers:  # the step's one append round, every layer in one launch, then the decodes
                pa.kv_append_layers(b.k_pool, b.v_pool, b.k_new[0], b.v_new[0], b.block_tables,
                                    b.append_positions[0], b.B)
                for layer in range(b.L):
                    pa.paged_attn_decode(b.q[layer], b.k_pool[layer], b.v_pool[layer], b.block_tables, b.seq_lens,
                                         b.B, b.scale, out=outs[layer], workspace=ws, order=order)
                return
            for layer in range(b.L):
                if fused:  # the step's one append round inside the decode launch
                    pa.paged_attn_decode_append(b.q[layer], b.k_pool[layer], b.v_pool[layer], b.k_new[0, layer],
                                                b.v_new[0, layer], b.block_tables, b.append_positions[0],
                                                b.seq_lens, b.B, b.scale, out=outs[layer], workspace=ws, order=order)
                    continue
                for r in range(b.rounds):
                    pa.kv_append(b.k_pool[layer], b.v_pool[layer], b.k_new[r, layer], b.v_new[r, layer],
                                 b.block_tables, b.append_positions[r], b.B)
                pa.paged_attn_decode(b.q[layer], b.k_pool[layer], b.v_pool[layer], b.block_tables, b.seq_lens,
                                     b.B, b.scale, out=outs[layer], workspace=ws, order=order)
        _, need = pa.paged_attn_plan(b.S, b.Hq, b.Hkv, b.D, b.MB, b.NB, b.dtype, b.B)
        order_buf = torch.empty(b.S, dtype=torch.int32, device=dev)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        outs = [torch.empty((b.S, b.Hq, b.D), dtype=torch.float32, device=dev) for _ in range(b.L)]
        return graph_time_us(torch, step, 1)

    # The block-size trade-off on the headline batch: same tokens, B = 8 .. 64,
    # four pool copies rotated as in the headline measurement.
    for B in (8, 16, 32, 64):
        b = W.config2(device=dev, B=B)
        pools = [(b.k_pool[0], b.v_pool[0])] + [(b.k_pool[0].clone(), b.v_pool[0].clone()) for _ in range(3)]
        calls = [pa.DecodeLaunch(b.q[0], k, v, b.block_tables, b.seq_lens, b.B, b.scale) for k, v in pools]

        def launch_all():
            for c in calls:
                c.launch()

        us = graph_time_us(torch, launch_all, 10) / len(calls)
        kvb = b.valid_kv_bytes_per_layer()
        out[f"bf16 32 x 4096 tokens, block size {B}"] = dict(
            rate(kvb, us), splits=calls[0].splits, layers=1, tokens_per_s_per_layer=round(b.S / (us * 1e-6), 1))
        del b, pools, calls
        torch.cuda.empty_cache()

    # Several query tokens per request ([Serving] §5): a speculative-verification
    # step with T draft tokens over the headline histories (4 rotated pool
    # copies), and one 512-token prompt chunk.  GB/s counts the history once.
    # T = 16 and 24 (the shared-tile path) also with PA_FLAG_BF16_WEIGHTS.
    for T, bf16_weights in ((2, False), (4, False), (8, False), (16, False), (16, True), (24, False), (24, True)):
        b = W.verify_batch(device=dev, T=T)
        pa.kv_append_tokens(b.k_pool, b.v_pool, b.k_new, b.v_new, b.block_tables, b.positions, b.B)
        pools = [(b.k_pool, b.v_pool)] + [(b.k_pool.clone(), b.v_pool.clone()) for _ in range(3)]
        calls = [pa.DecodeLaunch(b.q, k, v, b.block_tables, b.seq_lens, b.B, b.scale, bf16_weights=bf16_weights)
                 for k, v in pools]

        def launch_all():
            for c in calls:
                c.launch()

        us = graph_time_us(torch, launch_all, 10) / len(calls)
        tag = ", bf16 weights" if bf16_weights else ""
        out[f"bf16 verification, 32 x 4096 tokens, T = {T} query tokens{tag}"] = dict(
            rate(b.valid_kv_bytes(), us), splits=calls[0].splits, layers=1,
            query_tokens_per_s_per_layer=round(b.S * T / (us * 1e-6), 1))
        del b, pools, calls
        torch.cuda.empty_cache()
    # The prompt chunk with each softmax weight as a bf16 head plus remainder
    # (the default), and rounded once to bf16 (PA_FLAG_BF16_WEIGHTS).
    b = W.prefill_chunk_batch(device=dev)
    pa.kv_append_tokens(b.k_pool, b.v_pool, b.k_new, b.v_new, b.block_tables, b.positions, b.B)
    lens = b.seq_lens.cpu().tolist()
    # causal q.k and p.v: 4 * d flops per (query token, head, visible position)
    flops = sum(4 * b.D * b.Hq * (n - b.T + i + 1) for n in lens for i in range(b.T) if n - b.T + i >= 0)
    for bf16_weights, tag in ((False, ""), (True, ", bf16 weights")):
        call = pa.DecodeLaunch(b.q, b.k_pool, b.v_pool, b.block_tables, b.seq_lens, b.B, b.scale,
                               bf16_weights=bf16_weights)
        us = graph_time_us(torch, call.launch, 10)
        ent = dict(rate(b.valid_kv_bytes(), us), splits=call.splits, layers=1,
                   query_tokens_per_s_per_layer=round(b.S * b.T / (us * 1e-6), 1))
        ent["TFLOP_s"] = round(flops / (us * 1e-6) / 1e12, 2)
        ent["frac_bf16_mfma_peak"] = round(flops / (us * 1e-6) / 2.5e15, 4)
        out[f"bf16 prompt chunk, 8 x 4096 tokens, T = {b.T} query tokens{tag}"] = ent
        del call
    del b
    torch.cuda.empty_cache()

    # The attention part of recomputing a swapped-out request's KV instead of
    # swapping it back ([Slides] recovery-cost example: 4,000 tokens, 32
    # layers): the whole prompt again in 512-token chunks, chunk c attending
    # the request's pages up to its own last token.  The projections that
    # produce K and V are not part of this library, so this is a lower bound
    # on recomputation; one layer is timed and the 32 layers are 32 times it.
    n_re, chunk, layers_re = 4000, 512, 32
    b = W.extend_batch([n_re], n_re, seed=360, device=dev, name="reprefill_bf16_1x4000")
    pa.kv_append_tokens(b.k_pool, b.v_pool, b.k_new, b.v_new, b.block_tables, b.positions, b.B)
    for bf16_weights, tag in ((False, ""), (True, ", bf16 weights")):
        calls = []
        for c0 in range(0, n_re, chunk):
            t_c = min(chunk, n_re - c0)
            lens_c = torch.tensor([c0 + t_c], dtype=torch.int32, device=dev)
            calls.append(pa.DecodeLaunch(b.q[:, c0:c0 + t_c].contiguous(), b.k_pool, b.v_pool, b.block_tables,
                                         lens_c, b.B, b.scale, bf16_weights=bf16_weights))

        def reprefill():
            for c in calls:
                c.launch()

        us = graph_time_us(torch, reprefill, 5)
        flops = 4 * b.D * b.Hq * n_re * (n_re + 1) // 2  # position t of the prompt sees t + 1 positions
        out[f"bf16 re-prefill attention, one {n_re}-token request in {chunk}-token chunks{tag}"] = dict(
            us_per_layer=round(us, 2), chunks=len(calls), TFLOP_s=round(flops / (us * 1e-6) / 1e12, 2),
            frac_bf16_mfma_peak=round(flops / (us * 1e-6) / 2.5e15, 4),
            ms_for_32_layers=round(us * layers_re / 1e3, 3),
            note="attention only (K/V projections are outside this library): a lower bound on recomputing "
                 "the KV that swap_500MiB moves")
        del calls
    del b
    torch.cuda.empty_cache()

    for name, make, rows in (("fp32 5 requests (37..511 tokens), one layer", W.config1, None),
                             ("bf16 256 mixed-length requests, 32 layers", W.config3, None),
                             ("bf16 prefix sharing, 64 branches (COW), one layer", W.config4, None),
                             ("bf16 168 x 1025 tokens, 24 layers", W.config5, None)):
        b = make(device=dev)
        kvb = b.valid_kv_bytes_per_layer()
        layers = list(range(b.L))
        us, P = decode_graph(b, layers, reps=1 if b.L > 1 else 50)
        ent = dict(rate(kvb, us), splits=P, layers=b.L, tokens_per_s_per_layer=round(b.S / (us * 1e-6), 1))
        if b.L > 1 or b.rounds or b.cow_src.numel():
            step_us = full_step_graph(b)
            ent["full_step_us"] = round(step_us, 2)
            ent["full_step_ops"] = ("kv_cow_copy, " if b.cow_src.numel() else "") + \
                f"{b.rounds} kv_append round(s) and one decode per layer, {b.L} layer(s)"
            if b.rounds == 1 and not b.cow_src.numel():
                ent["full_step_fused_us"] = round(full_step_graph(b, fused=True), 2)
                ent["full_step_fused_ops"] = f"one paged_attn_decode_append per layer, {b.L} layer(s)"
                if b.L > 1:
                    ent["full_step_append_layers_us"] = round(full_step_graph(b, all_layers=True), 2)
                    ent["full_step_append_layers_ops"] = f"one kv_append_layers, then one decode per layer, {b.L} layers"
        if name.startswith("bf16 256 mixed"):
            # Work issued longest first (paged_attn_order once per step, passed to every layer's decode).
            order = pa.paged_attn_order(b.seq_lens)
            us_o, _ = decode_graph(b, layers, order=order)
            ent["longest_first"] = dict(rate(kvb, us_o), tokens_per_s_per_layer=round(b.S / (us_o * 1e-6), 1),
                                        full_step_fused_us=round(full_step_graph(b, fused=True, ordered=True), 2),
                                        full_step_append_layers_us=round(
                                            full_step_graph(b, all_layers=True, ordered=True), 2),
                                        ops="paged_attn_order once, then one paged_attn_decode_append per layer "
                                            "(fused) or one kv_append_layers and one decode per layer, all "
                                            "with dims->order")
            ent["swap_500MiB"] = swap_time(torch, pa, b, dev)
        if name.startswith("bf16 prefix"):
            ent["note"] = "the shared prefix is cache-resident: logical bytes, no roofline claim"
        out[name] = ent
        del b
        torch.cuda.empty_cache()
    return out


def suite_markdown(S, command):
    """The suite's JSON (``suite()``) as the markdown summary kept under profiles/:
    ``command`` is the command line that produced the JSON."""
    out = []
    w = out.append
    w("# Decode, several query tokens, block sizes, swap and full steps on the other workloads (MI355X, one GPU)\n")
    w("Command (from the repository root):\n")
    w(f"    {command}\n")
    w("(`bench.py --suite-md PATH` writes this summary from the same JSON, with `--suite-json` when the")
    w("suite has already run.)\n")
    w("Timing: each workload's launches are captured in one HIP graph and replayed back to back; the time")
    w("per launch includes the graph's inter-kernel gap.  Each graph first replays untimed for 0.25 s so")
    w("that the clocks have come up from the idle of the workload's set-up (suites taken before this")
    w("settle read 2-9 % slower).  Decode rows: per-layer decode time over all")
    w("layers (each layer has its own K/V pools, so nothing is cache-resident across layers except where")
    w("noted).  Full step: the whole decode step of all layers (copy-on-write where the workload has it,")
    w("kv_append rounds, then paged_attn_decode per layer); fused: one paged_attn_decode_append per")
    w("layer instead; all-layer append: one kv_append_layers launch for every layer, then the decodes.\n")
    w("| Workload | Decode us / layer | Valid K+V bytes / layer | GB/s | of 8 TB/s | Splits | Full step us | Fused us | All-layer append us | Tokens/s per layer |")
    w("|---|---|---|---|---|---|---|---|---|---|")
    for k in ("fp32 5 requests (37..511 tokens), one layer", "bf16 256 mixed-length requests, 32 layers",
              "bf16 prefix sharing, 64 branches (COW), one layer", "bf16 168 x 1025 tokens, 24 layers"):
        e = S[k]
        w(f"| {k} | {e['us']:.3f} | {e['bytes']:,} | {e['GB_s']:.1f} | {100*e['frac_hbm_peak']:.1f} % | {e['splits']} | "
          f"{e.get('full_step_us', '')} | {e.get('full_step_fused_us', '')} | {e.get('full_step_append_layers_us', '')} | {e['tokens_per_s_per_layer']:.0f} |")
    e = S["bf16 256 mixed-length requests, 32 layers"]
    lf = e.get("longest_first")
    if lf:
        w(f"| bf16 256 mixed-length requests, 32 layers, issued longest first | {lf['us']:.3f} | {lf['bytes']:,} | {lf['GB_s']:.1f} | "
          f"{100*lf['frac_hbm_peak']:.1f} % | {e['splits']} |  | {lf.get('full_step_fused_us', '')} | "
          f"{lf['full_step_append_layers_us']} | {lf['tokens_per_s_per_layer']:.0f} |")
        w("\nLongest first: one paged_attn_order per step (its order serves all 32 layers), then each")
        w("decode with dims->order; the fused step there is paged_attn_order and one")
        w("paged_attn_decode_append per layer, the all-layer one paged_attn_order, one kv_append_layers")
        w("and the 32 decodes.  Outputs are bitwise those of request order (tests/test_gpu_order.py).")
    w("\nThe prefix-sharing row reads the 128 shared prefix blocks 64 times, from cache after the first:")
    w("its logical rate is not an HBM figure (decode_mfma_bf16_workload_traffic.md gives its DRAM bytes).")
    w("The fp32 row is 2 MB of history: launch latency, not bandwidth.\n")
    w("## Several query tokens per request (paged_attn_extend, bf16, one layer)\n")
    w("Verification: 32 requests, 4096 positions each, the last T of them new (appended beforehand);")
    w("4 pool copies rotated.  Prompt chunk: 8 requests, 3584 positions of history plus a 512-token chunk.")
    w("GB/s counts the history once; TFLOP/s counts the causal q.k and p.v work (4 d flops per query")
    w("token, head and visible position) against the 2.5 PFLOP/s dense bf16 peak.  Rows marked \"bf16 weights\"")
    w("run with PA_FLAG_BF16_WEIGHTS (each softmax weight rounded once to bf16; see include/pagedattn.h).\n")
    w("| Workload | us | GB/s | of 8 TB/s | TFLOP/s | of bf16 peak | Splits | Query tokens/s |")
    w("|---|---|---|---|---|---|---|---|")
    for k, e in S.items():
        if k.startswith("bf16 verification") or k.startswith("bf16 prompt chunk"):
            tf = e.get("TFLOP_s", ""); fr = e.get("frac_bf16_mfma_peak")
            w(f"| {k} | {e['us']:.3f} | {e['GB_s']:.1f} | {100*e['frac_hbm_peak']:.1f} % | {tf} | {'' if fr is None else f'{100*fr:.1f} %'} | {e['splits']} | {e['query_tokens_per_s_per_layer']:.0f} |")
    w("\n## Block size on the 32 x 4096 batch (same tokens; 4 pool copies rotated)\n")
    w("| B | Decode us | GB/s | of 8 TB/s |")
    w("|---|---|---|---|")
    for B in (8, 16, 32, 64):
        e = S[f"bf16 32 x 4096 tokens, block size {B}"]
        w(f"| {B} | {e['us']:.3f} | {e['GB_s']:.1f} | {100*e['frac_hbm_peak']:.1f} % |")
    w("\nThe pages' trade-off ([Slides] \"块越小，省下的是空位，多出来的是管理\"): smaller blocks waste fewer tail")
    w("slots but need more table entries; for the read itself B = 16 to 64 are within 0.1 % here and B = 8 costs 3 %.\n")
    sw = S["bf16 256 mixed-length requests, 32 layers"].get("swap_500MiB")
    if sw:
        w("## Block swap (500 MiB through pinned host memory)\n")
        w("250 blocks x 32 layers x 64 KiB (K+V) = 524,288,000 B, the amount of the pages' recovery-cost")
        w("example (4,000 tokens at 128 KiB per token), moved by kv_swap_out / kv_swap_in directly between the")
        w("pools and pinned host memory:\n")
        w("| Direction | ms | GiB/s |")
        w("|---|---|---|")
        w(f"| out (pool -> host) | {sw['out_ms']} | {sw['out_GiB_s']} |")
        w(f"| in (host -> pool) | {sw['in_ms']} | {sw['in_GiB_s']} |\n")
        w(f"Round trip {sw['out_ms'] + sw['in_ms']:.1f} ms; the pages' teaching estimate at 25 GiB/s is 19.5 ms one")
        w("way and at least 39.1 ms for both.\n")
    re = [(k, e) for k, e in S.items() if k.startswith("bf16 re-prefill")]
    if re:
        w("## Swap or recompute ([Slides] recovery-cost example)\n")
        w("Recomputing instead of swapping means prefilling the 4,000 tokens again. The part of that which")
        w("this library runs is the attention: the whole prompt again in 512-token chunks, chunk c attending")
        w("the request's pages up to its own last token (paged_attn_extend, one request, bf16):\n")
        w("| Workload | us per layer | Chunks | TFLOP/s | of bf16 peak | ms for 32 layers |")
        w("|---|---|---|---|---|---|")
        for k, e in re:
            w(f"| {k} | {e['us_per_layer']} | {e['chunks']} | {e['TFLOP_s']} | {100*e['frac_bf16_mfma_peak']:.1f} % | {e['ms_for_32_layers']} |")
        d = re[0][1]
        w("\nThat is a lower bound on recomputation: the K/V projections and the rest of the model come on")
        w("top, and one request leaves most of the GPU idle." + (f" Recovery by swapping costs the swap-in, {sw['in_ms']} ms here,"
          f" after a {sw['out_ms']} ms swap-out at preemption time." if sw else ""))
        w(f"Recovery by recomputing costs at least the {d['ms_for_32_layers']} ms above, and 200 ms at the pages'")
        w("teaching rate of 20,000 tokens/s.")
    return "\n".join(out) + "\n"


PROFILE_WORKLOADS = {
    "decode32x4096": "bf16 32 x 4096 tokens, one layer (the headline batch, 4 rotated pool copies)",
    "mixed256": "bf16 256 mixed-length requests, 32 layers: one decode launch per layer, after the step's append",
    "mixed256o": "the same, the work issued longest first (paged_attn_order once, dims->order in every decode)",
    "prefix64": "bf16 prefix sharing, 64 branches, one layer: one decode launch, after the COW and appends",
    "long168": "bf16 168 x 1025 tokens, 24 layers: one decode launch per layer, after the step's append",
    "chunk512": "bf16 prompt chunk, 8 x 4096 tokens, T = 512, one layer (paged_attn_extend)",
    "chunk512w": "bf16 prompt chunk, 8 x 4096 tokens, T = 512, one layer, PA_FLAG_BF16_WEIGHTS",
    "verify16": "bf16 verification, 32 x 4096 tokens, T = 16 query tokens, one layer (paged_attn_extend)",
    "verify24": "bf16 verification, 32 x 4096 tokens, T = 24 query tokens, one layer (paged_attn_extend)",
}


def profile_workload(torch, pa, W, dev, name, steps, warmup):
    """Only one workload's attention launches, for rocprofv3: the step's
    copies and appends run once, untimed, then ``warmup`` + ``steps`` rounds of
    its decode (or extend) launches, one per layer per round, back to back.
    Prints the algorithmic bytes of one launch and the launches made."""
    if name == "decode32x4096":
        b = W.config2(device=dev)
        pools = [(b.k_pool[0], b.v_pool[0])] + [(b.k_pool[0].clone(), b.v_pool[0].clone()) for _ in range(3)]
        calls = [pa.DecodeLaunch(b.q[0], k, v, b.block_tables, b.seq_lens, b.B, b.scale) for k, v in pools]
        per_launch = b.valid_kv_bytes_per_layer()
        rounds = [[c] for c in calls]
    elif name in ("verify16", "verify24"):
        b = W.verify_batch(device=dev, T=int(name[-2:]))
        pa.kv_append_tokens(b.k_pool, b.v_pool, b.k_new, b.v_new, b.block_tables, b.positions, b.B)
        calls = [pa.DecodeLaunch(b.q, b.k_pool, b.v_pool, b.block_tables, b.seq_lens, b.B, b.scale)]
        per_launch = b.valid_kv_bytes()
        rounds = [calls]
    elif name in ("chunk512", "chunk512w"):
        b = W.prefill_chunk_batch(device=dev)
        pa.kv_append_tokens(b.k_pool, b.v_pool, b.k_new, b.v_new, b.block_tables, b.positions, b.B)
        calls = [pa.DecodeLaunch(b.q, b.k_pool, b.v_pool, b.block_tables, b.seq_lens, b.B, b.scale,
                                 bf16_weights=name == "chunk512w")]
        per_launch = b.valid_kv_bytes()
        rounds = [calls]
    else:
        b = {"mixed256": W.config3, "mixed256o": W.config3, "prefix64": W.config4, "long168": W.config5}[name](
            device=dev)
        if b.cow_src.numel():
            pa.kv_cow_copy(b.k_pool, b.v_pool, b.cow_src, b.cow_dst, b.cow_n, b.B)
        for r in range(b.rounds):
            for layer in range(b.L):
                pa.kv_append(b.k_pool[layer], b.v_pool[layer], b.k_new[r, layer], b.v_new[r, layer],
                             b.block_tables, b.append_positions[r], b.B)
        order = pa.paged_attn_order(b.seq_lens) if name == "mixed256o" else None
        calls = [pa.DecodeLaunch(b.q[layer], b.k_pool[layer], b.v_pool[layer], b.block_tables, b.seq_lens, b.B,
                                 b.scale, order=order) for layer in range(b.L)]
        per_launch = b.valid_kv_bytes_per_layer()
        rounds = [calls]
    torch.cuda.synchronize()
    n = 0
    for i in range(warmup + steps):
        for c in rounds[i % len(rounds)]:
            c.launch()
            n += 1
    torch.cuda.synchronize()
    print(json.dumps({"profile_workload": name, "what": PROFILE_WORKLOADS[name],
                      "algorithmic_kv_bytes_per_launch": int(per_launch), "launches": n,
                      "splits": calls[0].splits}), flush=True)
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
    ap.add_argument("--settle-seconds", type=float, default=1.0,
                    help="untimed launches before the warmup steps, so clocks settle")
    ap.add_argument("--no-side-kernels", action="store_true", help="skip the kv_append / kv_cow_copy timings")
    ap.add_argument("--suite", metavar="PATH", default=None,
                    help="also time the other four workloads and write them as JSON to PATH")
    ap.add_argument("--suite-md", metavar="PATH", default=None,
                    help="write the suite's markdown summary to PATH (with --suite, or alone with --suite-json)")
    ap.add_argument("--suite-json", metavar="PATH", default=None,
                    help="with --suite-md: format this suite JSON (written by --suite) instead of running anything")
    ap.add_argument("--profile-workload", choices=sorted(PROFILE_WORKLOADS), default=None,
                    help="only run one workload's attention launches (for rocprofv3), --warmup + --steps rounds")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB float32 negate-copy kernel (reads 1 GiB, writes 1 GiB) "
                         "a few times, to scale the HBM byte counters")
    args = ap.parse_args()

    if args.suite_md and args.suite_json:  # formatting only: no GPU
        with open(args.suite_json) as f:
            S = json.load(f)
        cmd = f"python3 bench.py --steps {args.steps} --no-cpu-baseline --no-side-kernels --suite {args.suite_json}"
        with open(args.suite_md, "w") as f:
            f.write(suite_markdown(S, cmd))
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); libpagedattn has no "
              "multi-GPU mode.", file=sys.stderr)
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
    if args.profile_workload:
        return profile_workload(torch, pa, W, dev, args.profile_workload, args.steps, args.warmup)
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

    # Untimed: let the GPU clocks settle on this load (a fresh box starts
    # slow), then the W warmup steps.
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_seconds:
        for i in range(50):
            calls[i % len(calls)].launch()
        torch.cuda.synchronize()
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

    # Per-launch spread: the same K launches, each bracketed by its own pair
    # of HIP events on the launch stream.  An event pair around every launch
    # adds about 2 us to each, so the roofline takes the mean launch time from
    # the events around the whole timed region above (one launch per step, on
    # the same stream), which is what the kernel trace's average shows.
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
    achieved = gbs  # one paged_attn_decode call per step: the mean launch time is ms_step
    # Everything a launch must touch besides the valid K/V: q, out, the table
    # rows and lengths, and the split workspace (written once, read once).
    ws_bytes = 2 * first.workspace.numel() if first.workspace is not None else 0
    other_bytes = (b.S * b.Hq * b.D * b.elem_bytes + b.S * b.Hq * b.D * 4 + b.S * b.MB * 4 + b.S * 4 + ws_bytes)
    traffic = measured_traffic()
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
        "total_GB_s": round((kv_bytes + other_bytes) / (ms_step * 1e-3) / 1e9, 2),
        "total_bytes_per_step": kv_bytes + other_bytes,
        "dram_GB_s": round(traffic / (ms_step * 1e-3) / 1e9, 2) if traffic else None,
        "launch_us_event_pairs": {"mean": round(mean_launch_ms * 1e3, 2),
                                  "p10": round(launch_ms[len(launch_ms) // 10] * 1e3, 2),
                                  "p90": round(launch_ms[len(launch_ms) * 9 // 10] * 1e3, 2)},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "one paged_attn_decode launch (decode kernel, plus the split merge when it splits)",
            "launch_us": round(ms_step * 1e3, 3),
            "timing": "HIP events on the launch stream around the K back-to-back launches of the timed region",
            "algorithmic_bytes_per_launch": kv_bytes,
        },
    }
    # The output of a step over the first pool copy (all copies hold the same
    # K/V), for the comparison with the oracle rows the CPU baseline computes.
    first.launch()
    torch.cuda.synchronize()
    host_out = out.cpu()
    del calls, first, pools
    torch.cuda.empty_cache()
    if not args.no_side_kernels:
        res["side_kernels"] = side_kernels(torch, pa, W, dev)
    if args.suite:
        st = suite(torch, pa, W, dev)
        with open(args.suite, "w") as f:
            json.dump(st, f, indent=1)
        if args.suite_md:
            with open(args.suite_md, "w") as f:
                f.write(suite_markdown(st, " ".join(["python3", "bench.py"] + sys.argv[1:])))
        for k, v in st.items():
            log(f"suite: {k}: {json.dumps(v)}")
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(b, args.cpu_seconds, gpu_out=host_out)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

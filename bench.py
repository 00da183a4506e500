#!/usr/bin/env python3
"""Benchmark of the BCQ LUT-GEMV on one MI355X.

One step = one y = W_hat x product (the whole path: table build, lookups,
scaling, accumulation, reduction, fp16 store) on device-resident inputs.
Default workload: the OPT-175B FFN-up shape, W 49152x12288 as 3 sign planes
with fp16 scales per group of 128, batch 1, fp16 x ~ N(0,1) (synthetic: the
pages' trained weights are not used).

Prints ONE JSON line on stdout. ``value`` is the achieved algorithmic HBM rate
(GB/s) over the wall-clock timed region; ``roofline.achieved`` is the same work
over the average launch duration on the GPU clock: a HIP event pair recorded on
the launch stream around the same K launches run back to back a second time,
with one untimed launch queued ahead so that the pair does not also time the
host's enqueue of the first launch (the pair around the wall-clock region is
reported as ``us_per_gemv_gpu_clock_from_sync``). ``roofline.bound`` is the larger of the two
algorithmic floors of the workload: HBM bytes at 8 TB/s, or the arithmetic of
the kernel that runs: fp32 lookups (two flops per lookup, the tables built
once) at the non-packed fp32 vector rate of 78.6 TFLOP/s for the table
kernels, fp16 products of the sign planes with x at the dense 2.5 PFLOP/s
matrix-core rate for the sign-plane MFMA kernel (batches of four rows and
more).
Before the ``--warmup`` launches, untimed launches run for at least
``--settle-s`` seconds and one full pass over the rotating weight copies, so
that clocks and caches are in their steady state however short the warm-up is
(reported as ``settle``).
``--gpus N`` with N > 1 exits: the library has no multi-GPU path.
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

METRIC = ("µs/GEMV + achieved HBM GB/s, K=12288 N=49152 3-bit BCQ g=128, batch 1")
HBM_PEAK_GBS = 8000.0
# fp32 vector arithmetic without packed math: one wave64 instruction per clock
# per compute unit, 256 CUs at 2.4 GHz, an FMA counting two flops (the 157.3
# TFLOP/s figure counts packed FMAs, which this code does not use)
ALU_PEAK_TFLOPS = 256 * 2.4e9 * 64 * 2 / 1e12
# dense fp16 matrix-core peak of MI355X (no sparsity), for the sign-plane MFMA kernel
MFMA_F16_PEAK_TFLOPS = 2500.0
KERNEL_SRCS = [os.path.join(ROOT, "lut_gemv_amd", "csrc", f)
               for f in ("lutgemv_kernel.h", "sign_mfma_kernel.h", "lutgemv_q.hip", "lutgemv.hip",
                         "layout.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lutgemv_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(N, K, q, g, m, has_offset):
    """Bytes the product must move: sign bits, scales (+ offsets), x and y."""
    G = K // g
    b = q * N * K // 8 + 2 * q * N * G + 2 * m * K + 2 * m * N
    if has_offset:
        b += 2 * N * G
    return b


def algorithmic_flops(N, K, q, g, m, has_offset):
    """fp32 operations the method must do: one multiply-add per lookup (m*N*q*K/8
    lookups), each chunk's 256-entry table built once per batch row (one add per
    entry), and one multiply-add per (batch row, row, group) for the offset."""
    f = 2 * m * N * q * (K // 8) + m * (K // 8) * 256
    if has_offset:
        f += 2 * m * N * (K // g)
    return f


def mfma_flops(N, K, q, m, has_offset):
    """Matrix-core work of the sign-plane MFMA kernel: each of the q sign planes
    (and, with an offset, an all-ones plane) times the m batch rows of x, two
    flops per product (the padding of the batch to 16 columns not counted)."""
    return 2 * m * N * K * (q + (1 if has_offset else 0))


def kernel_hash():
    """Hash of the kernel and launcher sources with their comments and blank
    lines removed (traffic counters go stale when the code changes, not when a
    comment does)."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [ln.rstrip() for ln in text.splitlines() if ln.strip()]
        h.update("\n".join(lines).encode())
    return h.hexdigest()[:16]


def stored_traffic(workload):
    """HBM bytes per launch from rocprofv3 counters (FETCH_SIZE and WRITE_SIZE,
    each scaled by what it reads for a copy of known size), if they were taken on
    this kernel source for this workload; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha256_16") != kernel_hash():
        return None
    rec = t.get("workloads", {}).get(workload)
    return rec.get("bytes_per_launch") if rec else None


def cpu_baseline(w, threads, budget_s):
    """The fp64 oracle on a bounded sample of rows, scaled to a full product.

    ``threads`` workers each run the oracle (unchanged) on their own blocks of
    256 rows with one BLAS thread, until ``budget_s`` seconds have passed or
    every row is done. Returns (seconds per full product, rows done, elapsed)."""
    import numpy as np
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    block = 256
    starts = list(range(0, w.N, block))
    t0 = time.perf_counter()

    def one(r0):
        if time.perf_counter() - t0 >= budget_s:
            return 0
        rows = np.arange(r0, min(w.N, r0 + block))
        oracle.gemv(w.bits, w.alpha, w.offset, w.x, w.g, rows=rows)
        return rows.size

    with threadpool_limits(limits=1):
        if threads == 1:
            rows_done = 0
            for r0 in starts:
                n = one(r0)
                if n == 0:
                    break
                rows_done += n
        else:
            with ThreadPoolExecutor(max_workers=threads) as ex:
                rows_done = sum(ex.map(one, starts))
    el = time.perf_counter() - t0
    return el * w.N / max(rows_done, 1), rows_done, el


def stream_peak(lg, torch, dev, nbytes=256 << 20, total=4 << 30, launches=400):
    """Achievable HBM read rate of this GPU: the library's streaming-read kernel
    over rotating buffers of nbytes (>= total bytes in all, so the last-level
    cache cannot serve repeats), non-temporal loads, event pair over `launches`
    launches after as many warm-up launches. Returns GB/s."""
    R = max(1, -(-total // nbytes))
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(R)]
    for b in bufs:
        b.fill_(1)
    sink = torch.zeros(4096, dtype=torch.int32, device=dev)
    sh = torch.cuda.current_stream(dev).cuda_stream
    for k in range(launches):
        lg.stream_read(bufs[k % R].data_ptr(), nbytes, sink.data_ptr(), sink.numel(), True, sh)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(launches):
        lg.stream_read(bufs[k % R].data_ptr(), nbytes, sink.data_ptr(), sink.numel(), True, sh)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / launches
    del bufs
    torch.cuda.empty_cache()
    return nbytes / t / 1e9


def load_workload(name):
    import workloads
    return workloads.generate(name)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="untimed launches before the warm-up, for at least this many seconds "
                         "and one pass over the rotating copies (clocks and caches settle)")
    ap.add_argument("--workload", default="opt175b_ffn_up")
    ap.add_argument("--kernel", choices=["lut", "dequant", "stream"], default="lut",
                    help="lut: the LUT-GEMV (the product); dequant: the dequantizing comparison "
                         "kernel on the same packed data; stream: the streaming-read kernel over "
                         "buffers of the workload's algorithmic bytes (the achievable ceiling)")
    ap.add_argument("--rotate", type=int, default=0,
                    help="distinct weight copies cycled through (0: enough for >= 4 GiB, at "
                         "most 4096 copies)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream-peak", action="store_true",
                    help="skip measuring the streaming-read ceiling after the timed region")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before the timed region, copy MIB MiB device to device 5 times "
                         "(a known-size reference for HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        msg = ("bench.py runs on one GPU only: the library has no multi-GPU path "
               f"(asked for --gpus {args.gpus}, WORLD_SIZE={world})")
        if int(os.environ.get("RANK", "0")) == 0:
            print(msg, file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch
    import lut_gemv_amd as lg

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t0 = time.perf_counter()
    w = load_workload(args.workload)
    log(f"workload {w.name}: N={w.N} K={w.K} q={w.q} g={w.g} m={w.m} "
        f"(generated in {time.perf_counter() - t0:.1f}s)")
    if w.is_uniform:
        pw0 = lg.PackedBCQ.from_uniform(w.codes, w.scale, w.zero, w.q, w.g, device=dev)
    else:
        pw0 = lg.PackedBCQ.from_bcq(w.bits, w.alpha, w.offset, w.g, device=dev)
    has_off = pw0.has_offset
    nbytes = algorithmic_bytes(w.N, w.K, w.q, w.g, w.m, has_off)
    nflops = algorithmic_flops(w.N, w.K, w.q, w.g, w.m, has_off)
    weight_bytes = pw0.d_bits.numel() + 2 * pw0.d_alpha.numel() + \
        (2 * pw0.d_offset.numel() if has_off else 0)
    # Enough distinct copies that no part of the weights can stay in the 256 MB
    # last-level cache between launches: the sign planes are read with a
    # non-temporal hint, so the scales of all copies (11% of the bytes at g=128)
    # must by themselves be well past the cache's size. 4 GiB of weights does
    # that at every group size here; tiny shapes, which are launch-bound, stop
    # at 4096 copies.
    R = args.rotate if args.rotate > 0 else min(4096, max(1, -(-(4 << 30) // weight_bytes)))
    x = torch.from_numpy(w.x).to(dev)
    y = torch.empty((w.m, w.N), dtype=torch.float16, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    if args.kernel == "stream":
        # the same algorithmic bytes as one contiguous buffer per copy (16-byte multiple)
        sbytes = -(-nbytes // 16) * 16
        R = args.rotate if args.rotate > 0 else min(4096, max(1, -(-(4 << 30) // sbytes)))
        del pw0
        bufs = [torch.ones(sbytes, dtype=torch.uint8, device=dev) for _ in range(R)]
        sink = torch.zeros(4096, dtype=torch.int32, device=dev)

        def launch(k):
            lg.stream_read(bufs[k % R].data_ptr(), sbytes, sink.data_ptr(), sink.numel(), True, sh)
        ws_bytes = 0
        weight_bytes = sbytes
    else:
        copies = [pw0]
        for _ in range(R - 1):
            copies.append(lg.PackedBCQ(w.N, w.K, w.q, w.g, pw0.d_bits.clone(), pw0.d_alpha.clone(),
                                       pw0.d_offset.clone() if has_off else None))
        ws_bytes = lg.workspace_size(w.N, w.K, w.q, w.g, has_off, w.m)
        ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        args_c = [(c.shape, c.d_bits.data_ptr(), c.d_alpha.data_ptr(),
                   c.d_offset.data_ptr() if has_off else None) for c in copies]
        if args.kernel == "lut":
            def launch(k):
                shape, b, a, o = args_c[k % R]
                lg.lutgemm_run(shape, w.m, b, a, o, x.data_ptr(), y.data_ptr(),
                               ws.data_ptr() if ws_bytes else None, ws_bytes, sh)
        else:
            def launch(k):
                shape, b, a, o = args_c[k % R]
                lg.bcq_dequant_gemv(shape, w.m, b, a, o, x.data_ptr(), y.data_ptr(), sh)

    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 5 device copies of {n} bytes")
        del src, dst
    torch.cuda.synchronize()
    log(f"{R} rotating copies ({R * weight_bytes / 2**30:.2f} GiB); settle >= {args.settle_s} s, "
        f"then warmup {args.warmup}")
    # settle: untimed launches in batches, for at least settle_s seconds of
    # wall clock and at least one pass over all R copies
    t_s = time.perf_counter()
    n_settle = 0
    while n_settle < R or time.perf_counter() - t_s < args.settle_s:
        for _ in range(200):
            launch(n_settle)
            n_settle += 1
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t_s
    for k in range(args.warmup):
        launch(n_settle + k)
    torch.cuda.synchronize()

    # timed region: K back-to-back products between two synchronizations; a HIP
    # event pair on the launch stream brackets the same region on the GPU clock
    K_steps = args.steps
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_begin = time.perf_counter()
    ev0.record(stream)
    for k in range(K_steps):
        launch(k)
    ev1.record(stream)
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_begin
    avg_from_sync_s = ev0.elapsed_time(ev1) * 1e-3 / K_steps
    # the kernel's launch duration on the GPU clock: the same K launches with
    # the queue kept busy (one untimed launch ahead of the first event), so the
    # event pair brackets K back-to-back products and not also the host's
    # enqueue of the first one after the synchronization (the region above
    # includes that idle gap once, which a short run divides by few steps)
    ep0 = torch.cuda.Event(enable_timing=True)
    ep1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    launch(K_steps)
    ep0.record(stream)
    for k in range(K_steps):
        launch(k)
    ep1.record(stream)
    torch.cuda.synchronize()
    avg_kernel_s = ep0.elapsed_time(ep1) * 1e-3 / K_steps
    # spread of single launches: the same K launches again, each between its own
    # event pair (the event packets add a little to each)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K_steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K_steps)]
    for k in range(K_steps):
        starts[k].record(stream)
        launch(k)
        ends[k].record(stream)
    torch.cuda.synchronize()
    durs_us = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)]) * 1e3
    p10, p50, p90 = (float(np.percentile(durs_us, v)) for v in (10, 50, 90))
    log(f"timed {K_steps} steps in {t_total * 1e3:.2f} ms wall ({avg_from_sync_s * 1e6:.2f} us per "
        f"launch between the events of that region), {avg_kernel_s * 1e6:.2f} us per launch on the "
        f"GPU clock back to back; single-launch events: p10 {p10:.2f} us, median {p50:.2f}, "
        f"p90 {p90:.2f}")

    plan = None
    if args.kernel == "lut":
        # the launch lutgemm_run makes here (after LUTGEMM_TILE, if set)
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        ws = None if cus == 256 else lg.workspace_size(w.N, w.K, w.q, w.g, bool(has_off), w.m)
        plan = lg.query_plan(w.N, w.K, w.q, w.g, bool(has_off), w.m, cus=cus, workspace_bytes=ws)
    on_mfma = plan is not None and plan["tables"] == "sign_mfma"

    ms_per_step = t_total * 1e3 / K_steps
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved_gbs = nbytes / avg_kernel_s / 1e9
    achieved_tflops = nflops / avg_kernel_s / 1e12
    hbm_frac = achieved_gbs / HBM_PEAK_GBS
    alu_frac = achieved_tflops / ALU_PEAK_TFLOPS
    # the bound is the larger of the two algorithmic floors: HBM bytes, and the
    # arithmetic of the kernel that runs (fp32 lookups and table builds on the
    # vector ALUs for the table kernels; fp16 products on the matrix cores for
    # the sign-plane MFMA kernel)
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_alu = nflops / (ALU_PEAK_TFLOPS * 1e12)
    mflops = mfma_flops(w.N, w.K, w.q, w.m, bool(has_off))
    t_mfma = mflops / (MFMA_F16_PEAK_TFLOPS * 1e12)
    mfma_frac = mflops / avg_kernel_s / 1e12 / MFMA_F16_PEAK_TFLOPS
    t_comp = t_mfma if on_mfma else t_alu
    if t_hbm >= t_comp or args.kernel == "stream":
        roof = {"bound": "hbm", "achieved": round(achieved_gbs, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(hbm_frac, 4)}
    elif on_mfma:
        roof = {"bound": "mfma", "achieved": round(mflops / avg_kernel_s / 1e12, 3),
                "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(mfma_frac, 4)}
    else:
        roof = {"bound": "alu", "achieved": round(achieved_tflops, 3),
                "peak": round(ALU_PEAK_TFLOPS, 2), "unit": "TFLOP/s", "frac": round(alu_frac, 4)}
    # counters were taken with the default rotation (weights streamed from HBM)
    roof["traffic"] = (stored_traffic(w.name) if args.kernel == "lut" and args.rotate == 0
                       else None)
    if on_mfma:
        roof["floor_us"] = {"hbm": round(t_hbm * 1e6, 3), "mfma": round(t_mfma * 1e6, 3)}
        roof["hbm_frac"] = round(hbm_frac, 4)
        roof["mfma_frac"] = round(mfma_frac, 4)
        roof["algorithmic_bytes"] = nbytes
        roof["algorithmic_flops"] = mflops
    else:
        roof["floor_us"] = {"hbm": round(t_hbm * 1e6, 3), "alu": round(t_alu * 1e6, 3)}
        roof["hbm_frac"] = round(hbm_frac, 4)
        roof["alu_frac"] = round(alu_frac, 4)
        roof["algorithmic_bytes"] = nbytes
        roof["algorithmic_flops"] = nflops

    if not args.no_stream_peak and args.kernel != "stream":
        peak_meas = stream_peak(lg, torch, dev)
        roof["hbm_peak_measured"] = round(peak_meas, 1)
        roof["hbm_frac_of_measured"] = round(achieved_gbs / peak_meas, 4)
        log(f"streaming-read ceiling: {peak_meas:.1f} GB/s (256 MiB buffers over 4 GiB, "
            f"non-temporal loads); this kernel {achieved_gbs:.1f} GB/s = "
            f"{achieved_gbs / peak_meas:.3f} of it")

    cpu = None
    if not args.no_cpu_baseline:
        cores = len(os.sched_getaffinity(0))
        full_s, rows, el = cpu_baseline(w, cores, 12.0)
        full1, rows1, el1 = cpu_baseline(w, 1, 8.0)
        cpu = {"value": round(nbytes / full_s / 1e9, 4), "unit": "GB/s", "cores": cores,
               "kind": "oracle",
               "sample": (f"fp64 oracle (reconstruct W_hat rows, direct dot) on {rows} of {w.N} "
                          f"rows in {el:.1f}s, {cores} threads each running it on its own "
                          f"256-row blocks with one BLAS thread, scaled to the full product: "
                          f"{full_s:.2f} s/GEMV; one thread: {rows1} rows in {el1:.1f}s, "
                          f"{full1:.2f} s/GEMV ({nbytes / full1 / 1e9:.4f} GB/s)")}
        log(f"cpu baseline: {cpu['sample']}")

    out = {
        "metric": (METRIC if w.name == "opt175b_ffn_up" and args.kernel == "lut"
                   else f"us/GEMV + achieved HBM GB/s, {w.name}, {args.kernel} kernel"),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "settle": {"launches": n_settle, "seconds": round(settle_s, 3)},
        "ms_per_step": round(ms_per_step, 5),
        "us_per_gemv": round(ms_per_step * 1e3, 2),
        "us_per_gemv_gpu_clock": round(avg_kernel_s * 1e6, 2),
        "us_per_gemv_gpu_clock_from_sync": round(avg_from_sync_s * 1e6, 2),
        "us_per_gemv_single_launch": {"p10": round(p10, 2), "p50": round(p50, 2),
                                      "p90": round(p90, 2)},
        "lookups_per_s": round(w.m * w.N * w.q * (w.K // 8) / avg_kernel_s, 0),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if on_mfma else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "kernel": args.kernel,
                   "N": w.N, "K": w.K, "q": w.q, "g": w.g, "m": w.m,
                   "offset": bool(has_off), "x": "fp16", "y": "fp16",
                   "weights": f"{w.q} sign planes + fp16 scales per {w.g} inputs",
                   "rotating_copies": R, "algorithmic_bytes": nbytes,
                   "plan": plan},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

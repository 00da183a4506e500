#!/usr/bin/env python3
"""Benchmark of the BCQ LUT-GEMV on one MI355X.

One step = one y = W_hat x product (the whole path: table build, lookups,
scaling, accumulation, reduction, fp16 store) on device-resident inputs.
Default workload: the OPT-175B FFN-up shape, W 49152x12288 as 3 sign planes
with fp16 scales per group of 128, batch 1, fp16 x ~ N(0,1) (synthetic: the
pages' trained weights are not used).

Prints ONE JSON line on stdout. ``value`` is the achieved algorithmic HBM rate
(GB/s) over the wall-clock timed region; ``roofline.achieved`` is the same bytes
over the average launch duration, from a HIP event pair recorded on the launch
stream around the same region.
``--gpus N`` with N > 1 exits: the library has no multi-GPU path.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("µs/GEMV + achieved HBM GB/s, K=12288 N=49152 3-bit BCQ g=128, batch 1")
HBM_PEAK_GBS = 8000.0
KERNEL_SRCS = [os.path.join(ROOT, "lut_gemv_amd", "csrc", f)
               for f in ("lutgemv_kernel.h", "lutgemv_q.hip", "lutgemv.hip", "layout.h")]
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


def kernel_hash():
    """Hash of the kernel and launcher sources (traffic counters go stale when they change)."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload):
    """HBM bytes per launch from rocprofv3 counters, if taken on this kernel source
    and this workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha256_16") != kernel_hash() or t.get("workload") != workload:
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(w, budget_s=12.0):
    """The fp64 oracle on a bounded sample of rows, one BLAS thread, scaled to a full product."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_limits
    rows_done = 0
    t0 = time.perf_counter()
    block = 256
    with threadpool_limits(limits=1):
        while rows_done < w.N and time.perf_counter() - t0 < budget_s:
            rows = np.arange(rows_done, min(w.N, rows_done + block))
            oracle.gemv(w.bits, w.alpha, w.offset, w.x, w.g, rows=rows)
            rows_done += rows.size
    el = time.perf_counter() - t0
    full_s = el * w.N / rows_done
    return full_s, rows_done, el


def load_workload(name):
    import workloads
    return workloads.generate(name)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=20000,
                    help="untimed launches first (about a second: the clocks take that long to settle)")
    ap.add_argument("--workload", default="opt175b_ffn_up")
    ap.add_argument("--kernel", choices=["lut", "dequant"], default="lut",
                    help="lut: the LUT-GEMV (the product); dequant: the dequantizing comparison "
                         "kernel on the same packed data")
    ap.add_argument("--rotate", type=int, default=0,
                    help="distinct weight copies cycled through (0: enough for >= 4 GiB, at "
                         "most 4096 copies)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    weight_bytes = pw0.d_bits.numel() + 2 * pw0.d_alpha.numel() + \
        (2 * pw0.d_offset.numel() if has_off else 0)
    # Enough distinct copies that no part of the weights can stay in the 256 MB
    # last-level cache between launches: the sign planes are read with a
    # non-temporal hint, so the scales of all copies (11% of the bytes at g=128)
    # must by themselves be well past the cache's size. 4 GiB of weights does
    # that at every group size here; tiny shapes, which are launch-bound, stop
    # at 4096 copies.
    R = args.rotate if args.rotate > 0 else min(4096, max(1, -(-(4 << 30) // weight_bytes)))
    copies = [pw0]
    for _ in range(R - 1):
        copies.append(lg.PackedBCQ(w.N, w.K, w.q, w.g, pw0.d_bits.clone(), pw0.d_alpha.clone(),
                                   pw0.d_offset.clone() if has_off else None))
    x = torch.from_numpy(w.x).to(dev)
    y = torch.empty((w.m, w.N), dtype=torch.float16, device=dev)
    ws_bytes = lg.workspace_size(w.N, w.K, w.q, w.g, has_off, w.m)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
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
    log(f"{R} rotating weight copies ({R * weight_bytes / 2**30:.2f} GiB); warmup {args.warmup}")
    for k in range(args.warmup):
        launch(k)
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
    avg_kernel_s = ev0.elapsed_time(ev1) * 1e-3 / K_steps
    # spread of single launches: the same K launches again, each between its own
    # event pair (the event packets add a little to each)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K_steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K_steps)]
    for k in range(K_steps):
        starts[k].record(stream)
        launch(k)
        ends[k].record(stream)
    torch.cuda.synchronize()
    durs_ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    log(f"timed {K_steps} steps in {t_total * 1e3:.2f} ms wall, {avg_kernel_s * 1e6:.2f} us per "
        f"launch on the GPU clock; single-launch events: median {np.median(durs_ms) * 1e3:.2f} us, "
        f"p10 {np.percentile(durs_ms, 10) * 1e3:.2f}, p90 {np.percentile(durs_ms, 90) * 1e3:.2f}")

    ms_per_step = t_total * 1e3 / K_steps
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / avg_kernel_s / 1e9
    # counters were taken with the default rotation (weights streamed from HBM)
    traffic = stored_traffic(w.name) if args.kernel == "lut" and args.rotate == 0 else None

    cpu = None
    if not args.no_cpu_baseline:
        full_s, rows, el = cpu_baseline(w)
        cpu = {"value": round(nbytes / full_s / 1e9, 4), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": (f"fp64 oracle (reconstruct W_hat rows, direct dot) on rows 0..{rows} of "
                          f"{w.N} in {el:.1f}s with one BLAS thread, scaled to the full product: "
                          f"{full_s:.1f} s/GEMV")}
        log(f"cpu baseline: {cpu['sample']}")

    out = {
        "metric": (METRIC if w.name == "opt175b_ffn_up" and args.kernel == "lut"
                   else f"us/GEMV + achieved HBM GB/s, {w.name}, {args.kernel} kernel"),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_gemv": round(ms_per_step * 1e3, 2),
        "us_per_gemv_gpu_clock": round(avg_kernel_s * 1e6, 2),
        "us_per_gemv_single_launch_median": round(float(np.median(durs_ms)) * 1e3, 2),
        "lookups_per_s": round(w.m * w.N * w.q * (w.K // 8) / avg_kernel_s, 0),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "kernel": args.kernel,
                   "N": w.N, "K": w.K, "q": w.q, "g": w.g, "m": w.m,
                   "offset": bool(has_off), "x": "fp16", "y": "fp16",
                   "rotating_copies": R, "algorithmic_bytes": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Phase timeline of one GEMV launch, per workgroup, from the phase-traced build.

Usage: ``python -m lut_gemv_amd.phases [--workload NAME] [--trials T] [--launches L]``

Runs a named synthetic workload (``workloads``) through ``liblutgemm_trace.so``
(built beside ``liblutgemm.so`` by ``python -m lut_gemv_amd.build``), with the
weights rotated over at least 4 GiB of copies as ``bench.py`` does, so that
nothing of them is cached between launches. Each trial launches L products
back to back and reads the stamps of the last one; for each phase boundary it
prints the distribution over workgroups of the time after the first
workgroup's start (µs, the median of each percentile over the trials). The
stamps come from the GPU's constant 100 MHz clock (10 ns resolution).
"""
from __future__ import annotations

import argparse
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PHASES = {0: "workgroup start", 1: "x staged in LDS", 2: "first table built",
          3: "first step done", 4: "last lookups done", 5: "workgroup end"}
TICK_US = 0.01


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--workload", default="opt175b_ffn_up")
    ap.add_argument("--trials", type=int, default=12)
    ap.add_argument("--launches", type=int, default=6)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--json", action="store_true", help="print one JSON line instead of a table")
    ap.add_argument("--rotate", type=int, default=0,
                    help="distinct weight copies cycled through (0: enough for >= 4 GiB)")
    args = ap.parse_args(argv)
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import numpy as np
    import torch

    import lut_gemv_amd as lg
    import workloads

    lg.use_traced_library()
    if not os.path.exists(lg.TRACE_LIB_PATH):
        raise SystemExit(f"{lg.TRACE_LIB_PATH} is not built; run `python -m lut_gemv_amd.build`")
    if not torch.cuda.is_available():
        raise SystemExit("a GPU is needed")
    dev = torch.device("cuda:0")
    w = workloads.generate(args.workload)
    if w.is_uniform:
        pw = lg.PackedBCQ.from_uniform(w.codes, w.scale, w.zero, w.q, w.g, device=dev)
    else:
        pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, w.offset, w.g, device=dev)
    wbytes = pw.d_bits.numel() + 2 * pw.d_alpha.numel() + (2 * pw.d_offset.numel() if pw.has_offset else 0)
    R = args.rotate if args.rotate > 0 else min(512, max(2, -(-(4 << 30) // wbytes)))
    copies = [pw] + [lg.PackedBCQ(w.N, w.K, w.q, w.g, pw.d_bits.clone(), pw.d_alpha.clone(),
                                  pw.d_offset.clone() if pw.has_offset else None)
                     for _ in range(R - 1)]
    x = torch.from_numpy(w.x).to(dev)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ws = None if cus == 256 else lg.workspace_size(w.N, w.K, w.q, w.g, pw.has_offset, w.m)
    plan = lg.query_plan(w.N, w.K, w.q, w.g, pw.has_offset, w.m, cus=cus, workspace_bytes=ws)
    nwg = plan["workgroups"]
    stamps = torch.zeros(nwg * 8, dtype=torch.int64, device=dev)
    lg.trace_attach(stamps.data_ptr(), stamps.numel() * 8)
    k = 0
    for _ in range(args.warmup):
        copies[k % R](x)
        k += 1
    torch.cuda.synchronize()
    per = {i: [] for i in PHASES}
    for _ in range(args.trials):
        stamps.zero_()
        for _ in range(args.launches):
            copies[k % R](x)
            k += 1
        torch.cuda.synchronize()
        t = stamps.cpu().numpy().reshape(nwg, 8)
        t0 = t[:, 0].min()
        for i in PHASES:
            if (t[:, i] > 0).all():
                per[i].append(np.percentile((t[:, i] - t0) * TICK_US, [0, 10, 50, 90, 100]))
    lg.trace_attach(None, 0)
    res = {PHASES[i]: [round(float(v), 2) for v in np.median(np.array(per[i]), axis=0)]
           for i in PHASES if per[i]}
    if args.json:
        print(json.dumps({"workload": w.name, "plan": plan, "rotating_copies": R,
                          "us_after_first_start_min_p10_p50_p90_max": res}))
        return 0
    print(f"{w.name}: {w.N}x{w.K} q={w.q} g={w.g} m={w.m}; plan {plan}; {R} rotating copies")
    print(f"{'phase':20s} {'min':>7s} {'p10':>7s} {'p50':>7s} {'p90':>7s} {'max':>7s}  (us after the first workgroup's start)")
    for name, v in res.items():
        print(f"{name:20s} " + " ".join(f"{u:7.2f}" for u in v))
    return 0


if __name__ == "__main__":
    sys.exit(main())

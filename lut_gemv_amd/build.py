"""Build the HIP library ``liblutgemm.so`` in-tree for gfx950.

Usage: ``python -m lut_gemv_amd.build`` (or ``__graft_entry__.build()``).
Host code (the packer) is compiled with g++, device code with hipcc, and the
two are linked into one shared library next to this file. The same sources
built with ``-DLUTGEMM_PHASE_TRACE`` give ``liblutgemm_trace.so``, the variant
whose kernels stamp their phase boundaries (``lutgemm_trace_attach``; read by
``python -m lut_gemv_amd.phases``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "liblutgemm.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
TRACE_LIB_PATH = os.path.join(PKG, "liblutgemm_trace.so")

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.environ.get("HIPCC", os.path.join(ROCM, "bin", "hipcc"))
CXX = os.environ.get("CXX", "g++")
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-mcode-object-version=5",
    # keep hipcc from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-pthread", "-ffp-contract=off"]


def _scratch_users(remarks: str):
    """Kernels whose resource-usage remarks report scratch (register spills)."""
    out, name = [], None
    for line in remarks.splitlines():
        if "Function Name:" in line:
            name = line.split("Function Name:")[1].split()[0]
        elif "ScratchSize [bytes/lane]:" in line and name:
            size = int(line.split("ScratchSize [bytes/lane]:")[1].split()[0])
            if size:
                out.append((name, size))
            name = None
    return out


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    if verbose and r.stdout.strip():
        print(r.stdout, flush=True)
    return r.stdout


def build(verbose: bool = False, extra_hip_flags=(), trace: bool = True) -> str:
    """Compile every source and link ``liblutgemm.so`` (and, with `trace`, the
    phase-traced ``liblutgemm_trace.so``); returns the regular library's path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    incs = [f"-I{INCLUDE}", f"-I{CSRC}"]
    tmp = tempfile.mkdtemp(prefix="lutgemm_build_")
    try:
        common = [os.path.join(tmp, f) for f in ("pack.o", "dequant.o", "footprint.o",
                                                  "quantize.o", "probe.o")]
        jobs = [
            [CXX, *CXX_FLAGS, *incs, "-c", os.path.join(CSRC, "pack.cpp"), "-o", common[0]],
            [HIPCC, *HIP_FLAGS, *extra_hip_flags, *incs, "-c", "-Rpass-analysis=kernel-resource-usage",
             os.path.join(CSRC, "dequant.hip"), "-o", common[1]],
            [CXX, *CXX_FLAGS, *incs, "-c", os.path.join(CSRC, "footprint.cpp"), "-o", common[2]],
            [CXX, *CXX_FLAGS, *incs, "-c", os.path.join(CSRC, "quantize.cpp"), "-o", common[3]],
            [HIPCC, *HIP_FLAGS, *extra_hip_flags, *incs, "-c",
             os.path.join(CSRC, "probe.hip"), "-o", common[4]],
        ]
        variants = {LIB_PATH: ([], "")}
        if trace:
            variants[TRACE_LIB_PATH] = (["-DLUTGEMM_PHASE_TRACE"], "_trace")
        objs = {}
        for path, (defs, tag) in variants.items():
            o = os.path.join(tmp, f"lutgemv{tag}.o")
            objs[path] = list(common) + [o]
            jobs.append([HIPCC, *HIP_FLAGS, *extra_hip_flags, *defs, *incs, "-c",
                         os.path.join(CSRC, "lutgemv.hip"), "-o", o])
            # the kernel instances of each plane count q build in their own unit
            for q in range(1, 9):
                o = os.path.join(tmp, f"lutgemv{tag}_q{q}.o")
                objs[path].append(o)
                jobs.append([HIPCC, *HIP_FLAGS, *extra_hip_flags, *defs, *incs, f"-DLUTGEMM_Q={q}",
                             "-c", "-Rpass-analysis=kernel-resource-usage",
                             os.path.join(CSRC, "lutgemv_q.hip"), "-o", o])
        workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            outs = [f.result() for f in [ex.submit(_run, j, False) for j in jobs]]
        # every kernel instance of the regular library is meant to fit its
        # register budget (the traced one may spill a little where it is tight)
        regular = [o for j, o in zip(jobs, outs) if "-DLUTGEMM_PHASE_TRACE" not in j]
        for name, size in [u for o in regular for u in _scratch_users(o)]:
            print(f"warning: {name} uses {size} bytes of scratch per lane", file=sys.stderr)
        for path, ob in objs.items():
            out_tmp = path + ".tmp"
            _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *ob,
                  "-pthread", "-o", out_tmp], verbose)
            os.replace(out_tmp, path)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)

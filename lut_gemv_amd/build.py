"""Build the HIP library ``liblutgemm.so`` in-tree for gfx950.

Usage: ``python -m lut_gemv_amd.build`` (or ``__graft_entry__.build()``).
Host code (the packer) is compiled with g++, device code with hipcc, and the
two are linked into one shared library next to this file.
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


def build(verbose: bool = False, extra_hip_flags=()) -> str:
    """Compile every source and link ``liblutgemm.so``; returns its path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    incs = [f"-I{INCLUDE}", f"-I{CSRC}"]
    tmp = tempfile.mkdtemp(prefix="lutgemm_build_")
    try:
        objs = [os.path.join(tmp, "pack.o"), os.path.join(tmp, "lutgemv.o"),
                os.path.join(tmp, "dequant.o"), os.path.join(tmp, "footprint.o"),
                os.path.join(tmp, "quantize.o"), os.path.join(tmp, "probe.o")]
        jobs = [
            [CXX, *CXX_FLAGS, *incs, "-c", os.path.join(CSRC, "pack.cpp"), "-o", objs[0]],
            [CXX, *CXX_FLAGS, *incs, "-c", os.path.join(CSRC, "footprint.cpp"), "-o", objs[3]],
            [CXX, *CXX_FLAGS, *incs, "-c", os.path.join(CSRC, "quantize.cpp"), "-o", objs[4]],
            [HIPCC, *HIP_FLAGS, *extra_hip_flags, *incs, "-c",
             os.path.join(CSRC, "lutgemv.hip"), "-o", objs[1]],
            [HIPCC, *HIP_FLAGS, *extra_hip_flags, *incs, "-c", "-Rpass-analysis=kernel-resource-usage",
             os.path.join(CSRC, "dequant.hip"), "-o", objs[2]],
            [HIPCC, *HIP_FLAGS, *extra_hip_flags, *incs, "-c",
             os.path.join(CSRC, "probe.hip"), "-o", objs[5]],
        ]
        # the kernel instances of each plane count q build in their own unit
        for q in range(1, 9):
            o = os.path.join(tmp, f"lutgemv_q{q}.o")
            objs.append(o)
            jobs.append([HIPCC, *HIP_FLAGS, *extra_hip_flags, *incs, f"-DLUTGEMM_Q={q}", "-c",
                         "-Rpass-analysis=kernel-resource-usage",
                         os.path.join(CSRC, "lutgemv_q.hip"), "-o", o])
        workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            outs = [f.result() for f in [ex.submit(_run, j, False) for j in jobs]]
        # every kernel instance is meant to fit its register budget
        spills = [u for o in outs for u in _scratch_users(o)]
        for name, size in spills:
            print(f"warning: {name} uses {size} bytes of scratch per lane", file=sys.stderr)
        out_tmp = LIB_PATH + ".tmp"
        _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs,
              "-pthread", "-o", out_tmp], verbose)
        os.replace(out_tmp, LIB_PATH)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)

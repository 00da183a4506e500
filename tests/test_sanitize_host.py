"""The library's host routines (packers, uniform rewrite, quantizer, footprint and
group search) built with AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize_host.cpp drives them on buffers sized exactly as the size
queries say, over edge shapes (ragged rows and input tiles, the smallest group,
row-wise groups, every plane count); any out-of-bounds access, leak or
undefined operation aborts the run. Its outputs must equal, byte for byte, what
the regular build of the library produces for the same inputs. CPU only.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import lut_gemv_amd as lg
from conftest import ROOT

CSRC = os.path.join(ROOT, "lut_gemv_amd", "csrc")
HOST_SOURCES = ["pack.cpp", "quantize.cpp", "footprint.cpp"]

# (kind, N, K, q, g, has_offset, iters)
CASES = [
    ("pack", 1, 8, 1, 8, 0, 0),
    ("pack", 17, 520, 3, 8, 1, 0),
    ("pack", 33, 1032, 8, 24, 1, 0),
    ("pack", 100, 4096, 4, 4096, 0, 0),
    ("pack", 0, 512, 2, 128, 0, 0),
    ("uniform", 19, 528, 4, 16, 1, 0),
    ("uniform", 5, 64, 1, 8, 1, 0),
    ("uniform", 40, 1024, 8, 128, 1, 0),
    ("quantize", 9, 256, 3, 32, 0, 3),
    ("quantize", 3, 64, 8, 8, 0, 1),
    ("quantize", 20, 512, 1, 512, 0, 0),
    ("footprint", 49152, 12288, 3, 128, 0, 26),
    ("footprint", 11008, 4096, 4, 128, 1, 40),
]


def _compiler():
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no g++")
    return cxx


def _write_inputs(d, idx, kind, N, K, q, g, off, rng):
    G = K // g if K else 0
    pre = os.path.join(d, f"c{idx}_")
    if kind == "pack":
        bits = rng.integers(0, 256, size=(q, N, K // 8), dtype=np.uint8)
        alpha = (rng.standard_normal((q, N, G)) * 0.02).astype(np.float16)
        offset = (rng.standard_normal((N, G)) * 0.02).astype(np.float16) if off else None
        bits.tofile(pre + "bits.bin")
        alpha.view(np.uint16).tofile(pre + "alpha.bin")
        if off:
            offset.view(np.uint16).tofile(pre + "offset.bin")
        return {"bits": bits, "alpha": alpha, "offset": offset}
    if kind == "uniform":
        codes = rng.integers(0, 1 << q, size=(N, K), dtype=np.uint8)
        scale = (np.abs(rng.standard_normal((N, G))) * 0.01).astype(np.float16)
        zero = rng.integers(0, 1 << q, size=(N, G), dtype=np.uint8)
        codes.tofile(pre + "codes.bin")
        scale.view(np.uint16).tofile(pre + "scale.bin")
        zero.tofile(pre + "zero.bin")
        return {"codes": codes, "scale": scale, "zero": zero}
    if kind == "quantize":
        w = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
        w.view(np.uint16).tofile(pre + "w.bin")
        return {"w": w}
    return {}


def test_host_routines_under_sanitizers(tmp_path):
    cxx = _compiler()
    exe = tmp_path / "sanitize_host"
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-pthread",
             "-ffp-contract=off", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    srcs = [os.path.join(CSRC, f) for f in HOST_SOURCES]
    r = subprocess.run([cxx, *flags, f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
                        os.path.join(ROOT, "tests", "sanitize_host.cpp"), *srcs, "-o", str(exe)],
                       capture_output=True, text=True)
    if r.returncode != 0 and "asan" in r.stderr.lower() and "cannot find" in r.stderr.lower():
        pytest.skip("sanitizer runtime not installed")
    assert r.returncode == 0, r.stderr

    d = tmp_path / "cases"
    d.mkdir()
    rng = np.random.default_rng(77)
    inputs = {}
    with open(d / "cases.txt", "w") as f:
        for idx, (kind, N, K, q, g, off, iters) in enumerate(CASES):
            inputs[idx] = _write_inputs(str(d), idx, kind, N, K, q, g, off, rng)
            f.write(f"{idx} {kind} {N} {K} {q} {g} {off} {iters}\n")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe), str(d)], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0 and r.stdout.strip() == "OK", (r.returncode, r.stdout, r.stderr[-4000:])

    def out(idx, name, dtype):
        return np.fromfile(d / f"c{idx}_{name}.bin", dtype=dtype)

    for idx, (kind, N, K, q, g, off, iters) in enumerate(CASES):
        inp = inputs[idx]
        if kind == "pack":
            pb, pa, po = lg.bcq_pack(inp["bits"], inp["alpha"], inp["offset"], g)
            assert np.array_equal(out(idx, "pbits", np.uint8), pb), idx
            assert np.array_equal(out(idx, "palpha", np.uint16), pa), idx
            if off:
                assert np.array_equal(out(idx, "poffset", np.uint16), po), idx
        elif kind == "uniform":
            pb, pa, po, nr = lg.bcq_pack_uniform(inp["codes"], inp["scale"], inp["zero"], q, g)
            assert np.array_equal(out(idx, "pbits", np.uint8), pb), idx
            assert np.array_equal(out(idx, "palpha", np.uint16), pa), idx
            assert np.array_equal(out(idx, "poffset", np.uint16), po), idx
            assert int(out(idx, "nrounded", np.uint64)[0]) == nr, idx
        elif kind == "quantize":
            bits, alpha, err = lg.bcq_quantize(inp["w"], q, g, iters=iters)
            assert np.array_equal(out(idx, "qbits", np.uint8), bits.reshape(-1)), idx
            assert np.array_equal(out(idx, "qalpha", np.uint16), alpha.view(np.uint16).reshape(-1)), idx
            assert out(idx, "qerr", np.float64)[0] == err, idx
        else:
            foot = out(idx, "foot", np.uint64)
            assert int(foot[0]) == lg.footprint_bits(N, K, q, g, bool(off)), idx
            found = lg.search_group_sizes(N, K, iters / 8.0, bool(off))
            for qq in range(1, 9):
                want = found.get(qq, (0, 0))
                assert (int(foot[qq]), int(foot[8 + qq])) == want, (idx, qq)

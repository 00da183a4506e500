"""Host-side checks of the C-ABI library: it loads, exports every declared
symbol, reports sizes, packs bit-exactly like the oracle, and rejects bad
arguments before any HIP call. No GPU needed."""
import ctypes
import os
import re

import numpy as np
import pytest

import lut_gemv_amd as lg
import oracle
import workloads
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "lutgemm.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert {"bcq_pack", "bcq_pack_uniform", "lutgemm_run"} <= set(names)
    L = lg.lib()
    for n in names:
        assert hasattr(L, n), n
    # and the shared object's dynamic symbol table agrees
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", lg.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, flags=re.M))
    assert set(names) <= exported


def _load_traced():
    if not os.path.exists(lg.TRACE_LIB_PATH):
        pytest.skip("phase-traced library not built")
    import torch  # noqa: F401  (the HIP runtime first, as the binding does)
    L = ctypes.CDLL(lg.TRACE_LIB_PATH)
    L.lutgemm_trace_attach.restype = ctypes.c_int
    L.lutgemm_trace_attach.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    return L


def test_phase_trace_entry_point():
    """The regular library refuses phase tracing; the traced build, built from
    the same sources, exports the same symbols and checks the buffer."""
    assert lg.lib().lutgemm_trace_attach(None, 0) == 6
    assert lg.lib().lutgemm_trace_attach(0x1000, 4096) == 6
    L = _load_traced()
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", lg.TRACE_LIB_PATH], capture_output=True,
                         text=True).stdout
    assert set(_declared_functions()) <= set(re.findall(r"\sT\s(\w+)$", out, flags=re.M))
    assert L.lutgemm_trace_attach(0x1004, 4096) == 5       # not 8-byte aligned
    assert L.lutgemm_trace_attach(0x1000, 4096) == 0       # host only: nothing is touched
    assert L.lutgemm_trace_attach(None, 0) == 0            # detached again


def test_abi_version_and_status_strings():
    assert lg.abi_version() == 1
    for st in range(9):
        assert lg.status_string(st)
    assert lg.status_string(123) == "unknown status"


@pytest.mark.parametrize("N,K,q,g,off", [(512, 512, 3, 128, False), (11008, 4096, 4, 128, True),
                                         (17, 520, 3, 8, True), (1, 8, 1, 8, False),
                                         (0, 512, 2, 64, False), (16, 0, 2, 8, True)])
def test_sizes_match_oracle(N, K, q, g, off):
    assert lg.packed_sizes(N, K, q, g, off) == oracle.packed_sizes(N, K, q, g, off)


@pytest.mark.parametrize("args", [
    (16, 12, 3, 8, 0),   # K % 8
    (16, 512, 0, 128, 0), (16, 512, 9, 128, 0),   # q range
    (16, 512, 3, 4, 0), (16, 512, 3, 12, 0),      # g >= 8, g % 8
    (16, 520, 3, 128, 0),                         # K % g
    (-1, 512, 3, 128, 0), (16, -8, 3, 8, 0),
    (16, 512, 3, 128, 2),                         # has_offset
    (1 << 30, 512, 3, 128, 0),
])
def test_shape_rules(args):
    assert lg.lib().lutgemm_check_shape(ctypes.byref(lg.Shape(*args))) == 2


def test_workspace_size_rules():
    assert lg.workspace_size(512, 512, 3, 128, False, 0) == 0
    assert lg.workspace_size(0, 512, 3, 128, False, 1) == 0
    assert lg.workspace_size(16, 0, 3, 8, False, 1) == 0
    with pytest.raises(lg.LutGemmError):
        lg.workspace_size(512, 512, 3, 128, False, -1)
    with pytest.raises(lg.LutGemmError):
        lg.workspace_size(512, 512, 3, 128, False, 65536)
    # few rows and a long input dimension: the reduction is split, which needs a workspace
    assert lg.workspace_size(256, 65536, 3, 128, False, 1) > 0


@pytest.mark.parametrize("q", range(1, 9))
@pytest.mark.parametrize("g", [8, 16, 24, 32, 128, 4096])
def test_every_configuration_has_a_kernel(q, g):
    """The dispatcher finds a kernel instance for every plane count, group
    class, offset flag and batch size (the workspace query reports it)."""
    for off in (False, True):
        for m in (1, 2, 3, 4, 5, 17, 64):
            for N in (16, 4096):
                lg.workspace_size(N, 4096 if 4096 % g == 0 else 24 * g, q, g, off, m)


def test_query_plan_batch_one_and_batched():
    """The launch plans of the benchmark's shapes on a full MI355X (host only)."""
    c2 = lg.query_plan(49152, 12288, 3, 128, False, 1)
    assert c2["tables"] == "single" and c2["waves"] == 16 and c2["x_in_lds"] == 1
    assert c2["split"] == 1 and c2["items"] == 256 and c2["workgroups"] == 256
    assert c2["row_tiles"] * 256 >= 49152 // 16 and c2["workspace_bytes"] == 0
    for m in (2, 4, 16, 32):
        p = lg.query_plan(12288, 12288, 3, 128, False, m)
        if m == 2:
            assert p["tables"] == "paired_mfma" and p["batch_rows"] == 2 and p["x_in_lds"] == 0, p
        elif m <= 16:   # the sign-plane MFMA kernel from 4 batch rows on
            assert p["tables"] == "sign_mfma" and p["batch_rows"] == 16 and p["waves"] == 16, p
            assert p["split"] == 5 and p["items"] == 48 * 5, p   # measured best at m = 4
            assert p["x_in_lds"] == 1, p                          # x staged once per item
        else:           # 8 waves x 32 batch rows per item past 16 rows (q <= 3)
            assert p["tables"] == "sign_mfma" and p["batch_rows"] == 32 and p["waves"] == 8, p
            assert p["split"] == 5 and p["items"] == 96 * 5, p   # measured: 42.6 us, split 2 44.1
        assert p["workspace_bytes"] == lg.workspace_size(12288, 12288, 3, 128, False, m)
        assert p["workgroups"] == min(p["items"], 256)
    # scale groups that are not whole 128-input step groups keep the tables
    assert lg.query_plan(12288, 12288, 3, 64, False, 8)["tables"] != "sign_mfma"
    # the matrix cores from 3 batch rows on for matrices of >= 6144 (row tile,
    # input tile) units, from 6 on for all; the tables below that (measured)
    for (N, K, m, mf) in ((12288, 12288, 3, True), (12288, 4096, 3, True), (4096, 14336, 4, True),
                          (4096, 4096, 3, False), (4096, 11008, 4, False), (5120, 5120, 5, False),
                          (4096, 4096, 6, True), (12288, 12288, 2, False)):
        assert (lg.query_plan(N, K, 3, 128, False, m)["tables"] == "sign_mfma") == mf, (N, K, m)
    nib = lg.query_plan(4096, 4096, 3, 128, False, 1)
    assert nib["tables"] == "nibble" and nib["split"] == 1 and nib["workgroups"] == nib["items"]
    # batch 1 with a split: row blocks of 8-16 row tiles sized so that the
    # split's items fill the 256 CUs (measured faster than 16-row blocks that
    # leave CUs idle: the one-of-eight shard, the int4 MLP, 22016 x 4096)
    for (N, K, q, g, off, ri, S) in ((6144, 12288, 3, 128, False, 12, 8),
                                     (11008, 4096, 4, 128, True, 11, 4),
                                     (22016, 4096, 3, 128, False, 11, 2)):
        p = lg.query_plan(N, K, q, g, off, 1)
        RT = N // 16
        assert p["tables"] == "single" and p["waves"] == 16 and p["x_in_lds"] == 1, p
        assert (p["row_tiles"], p["split"]) == (ri, S), p
        assert 0.9 * 256 < p["items"] == -(-RT // ri) * S <= 256, p
    # ... but not where fewer, longer steps measured faster (12288 x 12288)
    p = lg.query_plan(12288, 12288, 3, 128, False, 1)
    assert (p["row_tiles"], p["split"], p["items"]) == (16, 5, 240), p
    # scale groups not aligned to 32 inputs: single-row tables
    assert lg.query_plan(4096, 3072, 3, 24, False, 4)["tables"] == "single"
    for off in (False, True):
        for m in (0, 1, 3, 8):
            for N, K in ((0, 512), (512, 0)):
                assert lg.query_plan(N, K, 3, 128 if K else 8, off, m)["waves"] == 0


def test_query_plan_limits_and_override(monkeypatch):
    shard = lg.query_plan(6144, 12288, 3, 128, False, 1)
    assert shard["split"] > 1 and shard["workspace_bytes"] > 0
    none = lg.query_plan(6144, 12288, 3, 128, False, 1, workspace_bytes=0)
    assert none["split"] == 1 and none["workspace_bytes"] == 0
    small = lg.query_plan(6144, 12288, 3, 128, False, 1, cus=80)
    assert small["workgroups"] <= 80
    monkeypatch.setenv("LUTGEMM_TILE", "1,4,16,2,0,16,0,2")
    half = lg.query_plan(12288, 12288, 3, 128, False, 8)
    assert (half["tables"], half["split"], half["batch_rows"], half["waves"]) == ("half", 4, 2, 16)
    monkeypatch.setenv("LUTGEMM_TILE", "0,1,16,1,0,3,1,0,0,1")
    assert lg.query_plan(11008, 4096, 4, 128, True, 1)["tables"] == "nibble"
    monkeypatch.delenv("LUTGEMM_TILE")
    # the sign-plane MFMA kernel forced (PR = 5): an instance exists for every
    # plane count, offset and batch (fewer waves or batch rows per item where
    # the larger ones are not built); scale groups must be whole 128-input
    # step groups, else the override is ignored
    monkeypatch.setenv("LUTGEMM_TILE", "1,0,0,0,0,0,0,5")
    for q in range(1, 9):
        for off in (False, True):
            for m in (1, 2, 16, 17, 40):
                p = lg.query_plan(700, 2048, q, 128, off, m)
                assert p["tables"] == "sign_mfma" and p["waves"] in (8, 16), (q, off, m, p)
                assert p["batch_rows"] in (16, 32) and p["row_tiles"] == p["waves"], p
                assert p["workspace_bytes"] == (0 if p["split"] == 1 else
                                                65536 + 4 * p["split"] * m * 704)
    assert lg.query_plan(700, 2048, 3, 64, False, 4)["tables"] != "sign_mfma"
    monkeypatch.setenv("LUTGEMM_TILE", "1,3,8,32,0,0,0,5")
    p = lg.query_plan(12288, 12288, 3, 128, False, 40)
    assert (p["waves"], p["batch_rows"], p["split"], p["items"]) == (8, 32, 3, 1536 * 2 * 3 // 8 // 2)
    monkeypatch.delenv("LUTGEMM_TILE")
    L = lg.lib()
    pl = lg._Plan()
    shp = lg.Shape(512, 512, 3, 128, 0)
    assert L.lutgemm_query_plan(None, 1, 256, 0, ctypes.byref(pl)) == 1
    assert L.lutgemm_query_plan(ctypes.byref(shp), 1, 256, 0, None) == 1
    assert L.lutgemm_query_plan(ctypes.byref(shp), 1, 0, 0, ctypes.byref(pl)) == 2
    assert L.lutgemm_query_plan(ctypes.byref(shp), -1, 256, 0, ctypes.byref(pl)) == 2
    bad = lg.Shape(512, 500, 3, 128, 0)
    assert L.lutgemm_query_plan(ctypes.byref(bad), 1, 256, 0, ctypes.byref(pl)) == 2


# ---------------------------------------------------------------- packing parity

@pytest.mark.parametrize("N,K,q,g,off", [
    (17, 520, 3, 8, True), (16, 512, 1, 512, False), (40, 1024, 4, 128, True),
    (1, 8, 2, 8, False), (33, 1536, 8, 32, False), (100, 4096, 2, 4096, True),
])
def test_bcq_pack_bit_exact(N, K, q, g, off):
    w = workloads.random_bcq(N, K, q, g, seed=N * 7 + q, with_offset=off)
    pb, pa, po = lg.bcq_pack(w.bits, w.alpha, w.offset, g)
    rb, ra, ro = oracle.pack(w.bits, w.alpha, w.offset, g)
    assert np.array_equal(pb, rb)
    assert np.array_equal(pa, ra)
    if off:
        assert np.array_equal(po, ro)
    else:
        assert po is None


@pytest.mark.parametrize("name", ["tiny", "opt175b_ffn_up", "decode_m4", "subbit_q1_g32",
                                  "subbit_q2_g8192", "subbit_q4_g64"])
def test_bcq_pack_workloads_bit_exact(name):
    w = workloads.generate(name)
    pb, pa, _ = lg.bcq_pack(w.bits, w.alpha, None, w.g)
    rb, ra, _ = oracle.pack(w.bits, w.alpha, None, w.g)
    assert np.array_equal(pa, ra)
    assert np.array_equal(pb, rb)


def test_bcq_pack_uniform_llama_bit_exact():
    w = workloads.generate("llama7b_mlp_int4")
    pb, pa, po, n_r = lg.bcq_pack_uniform(w.codes, w.scale, w.zero, w.q, w.g)
    bits, alpha, off, n_ref = oracle.uniform_to_bcq(w.codes, w.scale, w.zero, w.q, w.g)
    rb, ra, ro = oracle.pack(bits, alpha, off, w.g)
    assert n_r == n_ref
    assert np.array_equal(pb, rb) and np.array_equal(pa, ra) and np.array_equal(po, ro)


@pytest.mark.parametrize("q", [1, 2, 3, 5, 8])
def test_bcq_pack_uniform_random_zero_points(q):
    w = workloads.random_uniform(37, 256, q, 32, seed=q, zero=None)
    pb, pa, po, n_r = lg.bcq_pack_uniform(w.codes, w.scale, w.zero, q, w.g)
    bits, alpha, off, n_ref = oracle.uniform_to_bcq(w.codes, w.scale, w.zero, q, w.g)
    rb, ra, ro = oracle.pack(bits, alpha, off, w.g)
    assert n_r == n_ref
    assert np.array_equal(pb, rb) and np.array_equal(pa, ra) and np.array_equal(po, ro)


@pytest.mark.parametrize("z", [0, 1, 2, 3])
def test_uniform_rounding_every_fp16_scale(z):
    """Every finite fp16 scale (q=2: values s/2, s and s*(1.5 - z)) rounds like the oracle."""
    pats = np.arange(0, 0x7C00, dtype=np.uint16)
    s = pats.view(np.float16)
    keep = np.abs(s.astype(np.float64) * max(1.0, abs(1.5 - z))) < 65504
    s = s[keep]
    N = s.size
    codes = np.zeros((N, 8), np.uint8)
    codes[:, 1] = 3
    scale = s.reshape(N, 1)
    zero = np.full((N, 1), z, np.uint8)
    pb, pa, po, n_r = lg.bcq_pack_uniform(codes, scale, zero, 2, 8)
    bits, alpha, off, n_ref = oracle.uniform_to_bcq(codes, scale, zero, 2, 8)
    rb, ra, ro = oracle.pack(bits, alpha, off, 8)
    assert n_r == n_ref
    assert np.array_equal(pa, ra) and np.array_equal(po, ro) and np.array_equal(pb, rb)


# ---------------------------------------------------------------- error paths

def _pack_call(shape, bits, alpha, offset, nb, na, no):
    ob = np.zeros(max(nb, 1), np.uint8)
    oa = np.zeros(max(na, 1), np.uint16)
    oo = np.zeros(max(no, 1), np.uint16)
    p = lambda a: None if a is None else a.ctypes.data
    return lg.lib().bcq_pack(ctypes.byref(shape), p(bits), p(alpha), p(offset), p(ob), nb,
                             p(oa), na, p(oo), no)


def test_bcq_pack_errors():
    N, K, q, g = 16, 512, 2, 128
    w = workloads.random_bcq(N, K, q, g, seed=1, with_offset=True)
    nb, na, no = lg.packed_sizes(N, K, q, g, True)
    s = lg.Shape(N, K, q, g, 1)
    a16 = w.alpha.view(np.uint16).copy()
    o16 = w.offset.view(np.uint16).copy()
    assert _pack_call(s, w.bits, a16, o16, nb, na, no) == 0
    assert _pack_call(s, w.bits, a16, None, nb, na, no) == 1            # offset missing
    assert _pack_call(s, None, a16, o16, nb, na, no) == 1
    assert _pack_call(s, w.bits, a16, o16, nb - 1, na, no) == 4         # buffer too small
    assert _pack_call(s, w.bits, a16, o16, nb, na - 1, no) == 4
    assert _pack_call(s, w.bits, a16, o16, nb, na, no - 1) == 4
    bad = a16.copy()
    bad[1, 3, 2] = 0x7C00                                               # +inf
    assert _pack_call(s, w.bits, bad, o16, nb, na, no) == 3
    bad[1, 3, 2] = 0x7E00                                               # NaN
    assert _pack_call(s, w.bits, bad, o16, nb, na, no) == 3
    bado = o16.copy()
    bado[0, 0] = 0xFC00
    assert _pack_call(s, w.bits, a16, bado, nb, na, no) == 3
    assert _pack_call(lg.Shape(N, K, q, 100, 1), w.bits, a16, o16, nb, na, no) == 2
    assert lg.lib().bcq_pack(None, None, None, None, None, 0, None, 0, None, 0) == 1


def test_bcq_pack_uniform_errors():
    w = workloads.random_uniform(16, 256, 4, 128, seed=0, zero=8)
    with pytest.raises(lg.LutGemmError) as e:
        lg.bcq_pack_uniform(w.codes | 16, w.scale, w.zero, 4, 128)
    assert e.value.status == 3
    with pytest.raises(lg.LutGemmError) as e:
        lg.bcq_pack_uniform(w.codes, w.scale, w.zero + 8, 4, 128)
    assert e.value.status == 3
    sc = w.scale.copy()
    sc[0, 0] = np.float16(np.inf)
    with pytest.raises(lg.LutGemmError) as e:
        lg.bcq_pack_uniform(w.codes, sc, w.zero, 4, 128)
    assert e.value.status == 3
    sc[0, 0] = np.float16(30000.0)      # 4 * s overflows fp16
    with pytest.raises(lg.LutGemmError) as e:
        lg.bcq_pack_uniform(w.codes, sc, w.zero, 4, 128)
    assert e.value.status == 3
    # has_offset must be 1 for the uniform rewrite
    s = lg.Shape(16, 256, 4, 128, 0)
    nb, na, no = lg.packed_sizes(16, 256, 4, 128, True)
    ob, oa, oo = np.zeros(nb, np.uint8), np.zeros(na, np.uint16), np.zeros(no, np.uint16)
    st = lg.lib().bcq_pack_uniform(ctypes.byref(s), w.codes.ctypes.data, w.scale.ctypes.data,
                                   w.zero.ctypes.data, ob.ctypes.data, nb, oa.ctypes.data, na,
                                   oo.ctypes.data, no, None)
    assert st == 2


def test_uniform_error_writes_nothing():
    w = workloads.random_uniform(16, 256, 4, 128, seed=0, zero=8)
    codes = w.codes.copy()
    codes[-1, -1] = 200
    nb, na, no = lg.packed_sizes(16, 256, 4, 128, True)
    ob = np.full(nb, 0xAB, np.uint8)
    oa = np.full(na, 0xABCD, np.uint16)
    oo = np.full(no, 0xABCD, np.uint16)
    s = lg.Shape(16, 256, 4, 128, 1)
    st = lg.lib().bcq_pack_uniform(ctypes.byref(s), codes.ctypes.data, w.scale.ctypes.data,
                                   w.zero.ctypes.data, ob.ctypes.data, nb, oa.ctypes.data, na,
                                   oo.ctypes.data, no, None)
    assert st == 3
    assert (ob == 0xAB).all() and (oa == 0xABCD).all() and (oo == 0xABCD).all()


def test_run_validates_before_any_hip_call():
    """Every argument error is reported without touching the (absent) GPU."""
    L = lg.lib()
    ok = lg.Shape(64, 512, 3, 128, 0)
    A = 0x100000     # fake, 16-byte aligned device addresses: never dereferenced
    def run(shape, m, b=A, a=A, o=None, x=A, y=A, ws=None, wsb=0):
        return L.lutgemm_run(ctypes.byref(shape) if shape is not None else None, m, b, a, o, x,
                             y, ws, wsb, None)
    assert run(None, 1) == 1
    assert run(lg.Shape(64, 12, 3, 128, 0), 1) == 2
    assert run(ok, -1) == 2
    assert run(ok, 65536) == 2
    assert run(ok, 0) == 0                       # empty batch: nothing to do
    assert run(lg.Shape(0, 512, 3, 128, 0), 1) == 0
    assert run(ok, 1, y=None) == 1
    assert run(ok, 1, b=None) == 1
    assert run(ok, 1, a=None) == 1
    assert run(ok, 1, x=None) == 1
    assert run(lg.Shape(64, 512, 3, 128, 1), 1, o=None) == 1
    assert run(ok, 1, b=A + 8) == 5
    assert run(ok, 1, x=A + 2) == 5
    assert run(ok, 1, a=A + 2) == 5
    assert run(ok, 1, y=A + 1) == 5
    assert run(lg.Shape(64, 512, 3, 128, 1), 1, o=A + 2) == 5
    big = lg.Shape(256, 65536, 3, 128, 0)
    need = lg.workspace_size(256, 65536, 3, 128, False, 1)
    assert need > 0
    assert run(big, 1, ws=None, wsb=0) == 1
    assert run(big, 1, ws=A, wsb=need - 1) == 4
    assert run(big, 1, ws=A + 4, wsb=need) == 5
    # each input buffer must be under 4 GiB (32-bit offsets in the kernel)
    huge_bits = lg.Shape(1 << 20, 1 << 13, 8, 128, 0)      # 8 GiB of sign planes
    assert run(huge_bits, 1) == 2
    assert L.lutgemm_workspace_size(ctypes.byref(huge_bits), 1, ctypes.byref(ctypes.c_size_t())) == 2
    wide = lg.Shape(64, 1 << 16, 1, 128, 0)
    assert run(wide, 32768) == 2                           # x of exactly 4 GiB: rejected


def test_dequant_validates_before_any_hip_call():
    """The dequantizing comparison kernel reports argument errors without the GPU."""
    L = lg.lib()
    ok = lg.Shape(64, 512, 3, 128, 0)
    A = 0x100000
    def run(shape, m, b=A, a=A, o=None, x=A, y=A):
        return L.bcq_dequant_gemv(ctypes.byref(shape) if shape is not None else None, m, b, a,
                                  o, x, y, None)
    assert run(None, 1) == 1
    assert run(lg.Shape(64, 12, 3, 128, 0), 1) == 2
    assert run(ok, -1) == 2
    assert run(ok, 0) == 0
    assert run(ok, 1, y=None) == 1
    assert run(ok, 1, b=None) == 1
    assert run(lg.Shape(64, 512, 3, 128, 1), 1, o=None) == 1
    assert run(ok, 1, b=A + 8) == 5
    assert run(ok, 1, x=A + 2) == 5
    assert run(ok, 1, a=A + 2) == 5


@pytest.mark.parametrize("N,K,q,g,off", [(49152, 12288, 3, 128, False), (11008, 4096, 4, 128, True),
                                         (1, 8, 8, 8, True), (7, 520, 2, 40, False)])
def test_footprint_matches_oracle(N, K, q, g, off):
    assert lg.footprint_bits(N, K, q, g, off) == oracle.footprint_bits(N * K, q, g, off)


@pytest.mark.parametrize("N,K,bpw,off", [(49152, 12288, 3.25, False), (11008, 4096, 4.5, True),
                                         (28672, 8192, 2.125, False), (3, 1000, 9.0, True),
                                         (5, 24, 1.0, False), (64, 4096, 8.0 + 1 / 3, True)])
def test_group_search_matches_oracle(N, K, bpw, off):
    assert lg.search_group_sizes(N, K, bpw, off) == oracle.search_group_sizes(N, K, bpw, off)


def test_group_search_errors():
    L = lg.lib()
    g = (ctypes.c_int32 * 8)()
    b = (ctypes.c_uint64 * 8)()
    assert L.bcq_search_group_sizes(0, 512, 0, 3.0, g, b) == 2
    assert L.bcq_search_group_sizes(4, 12, 0, 3.0, g, b) == 2
    assert L.bcq_search_group_sizes(4, 512, 2, 3.0, g, b) == 2
    assert L.bcq_search_group_sizes(4, 512, 0, 0.0, g, b) == 3
    assert L.bcq_search_group_sizes(4, 512, 0, float("nan"), g, b) == 3
    assert L.bcq_search_group_sizes(4, 512, 0, 3.0, None, b) == 1


def _quant_input(rng, N, K, dist):
    if dist == "gauss":
        w = rng.standard_normal((N, K)) * 0.02
    elif dist == "heavy":
        w = rng.standard_t(3, (N, K)) * 0.05
    elif dist == "large":
        w = rng.uniform(-60000, 60000, (N, K))
    elif dist == "tiny":
        w = rng.standard_normal((N, K)) * 1e-6          # fp16 subnormals
    else:
        raise ValueError(dist)
    w = w.astype(np.float16)
    w[0, : K // 2] = 0                                   # a zero half-row
    if N > 1:
        w[1, :] = np.float16(-0.0)                       # an all (negative) zero row
    if N > 2:
        w[2, :] = w[2, 0]                                # a constant row
    return w


@pytest.mark.parametrize("N,K,q,g,iters,dist", [
    (5, 64, 1, 8, 0, "gauss"), (4, 256, 3, 128, 0, "gauss"), (4, 256, 3, 128, 3, "gauss"),
    (3, 96, 2, 32, 2, "heavy"), (2, 4096, 4, 4096, 1, "gauss"), (3, 64, 8, 64, 2, "gauss"),
    (3, 128, 3, 64, 2, "large"), (3, 128, 2, 16, 2, "tiny"), (9, 40, 5, 8, 4, "heavy"),
])
def test_quantize_matches_oracle(N, K, q, g, iters, dist):
    """bcq_quantize and the oracle's quantizer agree bit for bit (planes and fp16
    scales); the squared errors agree up to summation order."""
    rng = np.random.default_rng(N * 1000 + K + q)
    w = _quant_input(rng, N, K, dist)
    bits, alpha, err = lg.bcq_quantize(w, q, g, iters)
    ob_, oa, oe = oracle.quantize_bcq(w, q, g, iters)
    assert np.array_equal(bits, ob_)
    assert np.array_equal(alpha.view(np.uint16), oa.view(np.uint16))
    assert err == pytest.approx(oe, rel=1e-12, abs=1e-300)


def test_quantize_then_pack_matches_oracle():
    """Quantizer output feeds bcq_pack unchanged (layouts [q][N][K/8], [q][N][K/g])."""
    rng = np.random.default_rng(7)
    N, K, q, g = 20, 520, 3, 40
    w = _quant_input(rng, N, K, "gauss")
    bits, alpha, _ = lg.bcq_quantize(w, q, g, 2)
    pb, pa, po = lg.bcq_pack(bits, alpha, None, g)
    eb, ea, eo = oracle.pack(bits, alpha, None, g)
    assert np.array_equal(pb, eb) and np.array_equal(pa.view(np.uint16), ea.view(np.uint16))


def test_quantize_errors():
    L = lg.lib()
    N, K, q, g = 4, 64, 2, 32
    w = (np.random.default_rng(0).standard_normal((N, K)) * 0.1).astype(np.float16)
    w16 = w.view(np.uint16)
    bits = np.full(q * N * K // 8, 0xAB, np.uint8)
    alpha = np.full(q * N * K // g, 0xABCD, np.uint16)
    err = ctypes.c_double(-1.0)

    def call(shape, wp=w16, it=0, nb=bits.size, na=alpha.size, b=bits, a=alpha):
        p = lambda t: None if t is None else t.ctypes.data
        return L.bcq_quantize(ctypes.byref(shape), p(wp), it, p(b), nb, p(a), na, ctypes.byref(err))

    s = lg.Shape(N, K, q, g, 0)
    assert call(lg.Shape(N, K, q, g, 1)) == 2                 # no offset term in BCQ output
    assert call(lg.Shape(N, K, q, 24, 0)) == 2                # g does not divide K
    assert call(lg.Shape(N, K, 9, g, 0)) == 2
    assert call(s, it=-1) == 3 and call(s, it=1001) == 3
    assert call(s, wp=None) == 1 and call(s, b=None) == 1 and call(s, a=None) == 1
    assert call(s, nb=bits.size - 1) == 4 and call(s, na=alpha.size - 1) == 4
    bad = w16.copy()
    bad[3, 63] = 0x7E00                                        # NaN
    assert call(s, wp=bad) == 3
    bad[3, 63] = 0xFC00                                        # -inf
    assert call(s, wp=bad) == 3
    assert (bits == 0xAB).all() and (alpha == 0xABCD).all()   # nothing written on error
    assert L.bcq_quantize(None, None, 0, None, 0, None, 0, None) == 1
    assert call(lg.Shape(0, K, q, g, 0), wp=None, b=None, a=None) == 0
    assert err.value == 0.0
    assert call(s) == 0 and err.value > 0


def test_header_is_plain_c_and_links(tmp_path):
    """include/lutgemm.h compiles as strict C99 and a C program links against the
    library and calls its host entry points (no torch, no Python)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "abi.c"
    src.write_text(r'''
#include <stdio.h>
#include <string.h>
#include "lutgemm.h"
int main(void) {
  lutgemm_shape s;
  size_t nb = 0, na = 0, no = 0;
  uint8_t bits[2 * 16 * 512 / 8];
  uint16_t alpha[2 * 16 * 4];
  static uint8_t pb[2 * 1024];
  static uint16_t pa[2 * 16 * 4];
  uint64_t fb = 0;
  int32_t gs[8];
  uint64_t bs[8];
  memset(&s, 0, sizeof s);
  s.N = 16; s.K = 512; s.q = 2; s.g = 128; s.has_offset = 0;
  if (lutgemm_abi_version() != LUTGEMM_ABI_VERSION) return 1;
  if (lutgemm_check_shape(&s) != LUTGEMM_OK) return 2;
  if (lutgemm_packed_sizes(&s, &nb, &na, &no) != LUTGEMM_OK) return 3;
  if (nb != sizeof pb || na != sizeof pa / sizeof pa[0] || no != 0) return 4;
  memset(bits, 0xA5, sizeof bits);
  for (size_t i = 0; i < sizeof alpha / sizeof alpha[0]; ++i) alpha[i] = 0x3C00; /* 1.0 */
  if (bcq_pack(&s, bits, alpha, NULL, pb, nb, pa, na, NULL, 0) != LUTGEMM_OK) return 5;
  if (bcq_footprint_bits(&s, &fb) != LUTGEMM_OK || fb != 2u * 16 * 512 + 16u * 2 * 16 * 4) return 6;
  if (bcq_search_group_sizes(16, 512, 0, 3.0, gs, bs) != LUTGEMM_OK) return 7;
  if (lutgemm_run(NULL, 1, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) != LUTGEMM_ERR_NULL) return 8;
  printf("%s\n", lutgemm_status_string(LUTGEMM_ERR_SHAPE));
  return 0;
}
''')
    exe = tmp_path / "abi"
    libdir = os.path.dirname(lg.LIB_PATH)
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                        f"-I{os.path.join(ROOT, 'include')}", str(src), f"-L{libdir}",
                        "-l:" + os.path.basename(lg.LIB_PATH), f"-Wl,-rpath,{libdir}", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stderr)
    assert r.stdout.strip() == lg.status_string(2)


def test_stream_read_validates_before_any_hip_call():
    """The streaming-read measurement kernel reports argument errors without the GPU."""
    L = lg.lib()
    A = 0x100000
    assert L.lutgemm_stream_read(A, 0, A, 1, 1, None) == 0           # nothing to read
    assert L.lutgemm_stream_read(None, 64, A, 1, 1, None) == 1
    assert L.lutgemm_stream_read(A, 64, None, 1, 1, None) == 1
    assert L.lutgemm_stream_read(A + 8, 64, A, 1, 1, None) == 5
    assert L.lutgemm_stream_read(A, 64, A + 2, 1, 1, None) == 5
    assert L.lutgemm_stream_read(A, 64, A, 1, 2, None) == 3
    assert L.lutgemm_stream_read(A, 64, A, 0, 1, None) == 4
    assert L.lutgemm_stream_read(A, 1 << 32, A, 1, 1, None) == 2


def test_packed_workspace_is_kept_per_stream(monkeypatch):
    """PackedBCQ keeps one workspace per stream (calls that overlap in time must
    not share one): the same stream gets the same buffer back, another stream its
    own, and a larger need replaces only that stream's buffer. CPU tensors and
    stand-in streams; no GPU."""
    import contextlib

    import torch

    class FakeStream:
        def __init__(self, h):
            self.cuda_stream = h

    sizes = {1: 1000, 4: 3000}
    inits = []
    monkeypatch.setattr(lg, "workspace_size", lambda N, K, q, g, off, m: sizes.get(m, 0))
    monkeypatch.setattr(lg, "workspace_init", lambda p, n, s: inits.append((n, s)))
    monkeypatch.setattr(torch.cuda, "stream", lambda s: contextlib.nullcontext())
    pw = lg.PackedBCQ(64, 512, 3, 128, torch.zeros(16, dtype=torch.uint8),
                      torch.zeros(16, dtype=torch.int16))
    s1, s2 = FakeStream(11), FakeStream(22)
    a, na = pw.workspace(1, s1)
    b, nb = pw.workspace(1, s1)
    c, nc = pw.workspace(1, s2)
    assert a is b and na == nb == 1000
    assert c is not a and nc == 1000
    assert inits == [(1000, 11), (1000, 22)]
    d, nd = pw.workspace(4, s1)                    # grows on s1 only
    assert nd == 3000 and d is not a
    assert pw.workspace(1, s2)[0] is c
    assert pw.workspace(1, s1)[0] is d            # a larger buffer serves smaller needs
    assert inits[-1] == (3000, 11)
    assert pw.workspace(2, s1) == (None, 0)       # no split: no workspace


def test_run_noalloc_validates_before_any_hip_call(monkeypatch):
    """lutgemm_run_noalloc reports argument errors, and refuses a forced split
    whose partial sums would not fit its scratch, without touching the GPU."""
    L = lg.lib()
    assert L.lutgemm_noalloc_scratch_bytes() == 4 << 20
    ok = lg.Shape(64, 512, 3, 128, 0)
    A = 0x100000

    def run(shape, m, b=A, a=A, o=None, x=A, y=A):
        return L.lutgemm_run_noalloc(ctypes.byref(shape) if shape is not None else None, m, b, a,
                                     o, x, y, None)
    assert run(None, 1) == 1
    assert run(lg.Shape(64, 12, 3, 128, 0), 1) == 2
    assert run(ok, -1) == 2 and run(ok, 65536) == 2
    assert run(ok, 0) == 0 and run(lg.Shape(0, 512, 3, 128, 0), 1) == 0
    assert run(ok, 1, y=None) == 1 and run(ok, 1, b=None) == 1
    assert run(lg.Shape(64, 512, 3, 128, 1), 1, o=None) == 1
    assert run(ok, 1, b=A + 8) == 5 and run(ok, 1, x=A + 2) == 5
    # 64 splits x 8 batch rows x 4096 rows x 4 bytes = 8 MiB of partial sums
    big = lg.Shape(4096, 32768, 3, 128, 0)
    monkeypatch.setenv("LUTGEMM_TILE", "1,64,16,1")
    assert run(big, 8) == 4
    monkeypatch.setenv("LUTGEMM_TILE", "1,8,16,1")      # 1 MiB: fits, so it reaches the device check
    assert run(big, 8) == 7
    monkeypatch.delenv("LUTGEMM_TILE")

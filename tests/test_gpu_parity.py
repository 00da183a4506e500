"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Acceptance per output (the tolerance the GEMV is specified to): |y_gpu - y_ref|
<= 1e-3 * sum_k |W_hat[j,k] x[k]| + 1e-4. The full-size workloads run in the
launch configuration the benchmark times; the OPT-175B FFN-up shape, its row
shard, the int4 MLP and the 12288-wide batches are checked on every output, the
28672x8192 sweep on sampled rows the oracle computes one by one. Small problems
are checked on every output.
"""
import os
import sys

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import lut_gemv_amd as lg  # noqa: E402

DEV = "cuda:0"


def _say(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


def _gpu_y(pw, x_np):
    x = torch.from_numpy(np.ascontiguousarray(x_np)).to(DEV)
    y = pw(x)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _sample_rows(N, n, seed=0):
    if N <= n:
        return np.arange(N)
    rng = np.random.default_rng(seed)
    edge = np.r_[np.arange(min(32, N)), np.arange(max(0, N - 32), N)]
    return np.unique(np.r_[edge, rng.choice(N, size=n, replace=False)])


def _check(y_gpu, w, rows=None, ref=None):
    if ref is None:
        ref, bound = oracle.gemv(w.bits, w.alpha, w.offset, w.x, w.g, rows=rows)
    else:
        ref, bound = ref
    yg = y_gpu if rows is None else y_gpu[:, rows]
    ok, worst = oracle.parity_ok(yg.astype(np.float64), ref, bound)
    _say(f"{w.name}: worst err/tol = {worst:.3f} over {yg.size} outputs")
    assert ok, f"{w.name}: worst err/tol {worst}"
    return worst


@pytest.fixture(scope="module", autouse=True)
def _device():
    _say(f"device {torch.cuda.get_device_name(0)}")
    assert lg.abi_version() == 1
    yield


# ---------------------------------------------------------------- named workloads

def test_tiny_all_outputs():
    w = workloads.generate("tiny")
    _say("tiny 512x512 q3 g128")
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, None, w.g)
    _check(_gpu_y(pw, w.x), w)


def test_opt175b_ffn_up_all_outputs():
    """The benchmark's workload in the launch configuration it times, every output."""
    w = workloads.generate("opt175b_ffn_up")
    _say("opt175b_ffn_up 49152x12288 q3 g128 m1")
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, None, w.g)
    y = _gpu_y(pw, w.x)
    assert np.isfinite(y).all()
    _check(y, w)


def test_opt175b_ffn_up_shard_all_outputs():
    """One of eight row shards of the FFN-up matrix, every output."""
    w = workloads.generate("opt175b_ffn_up_shard8")
    _say("opt175b_ffn_up_shard8 6144x12288 q3 g128 m1")
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, None, w.g)
    _check(_gpu_y(pw, w.x), w)


def test_linearity():
    """y(x1 + x2) = y(x1) + y(x2) within the tolerance of the two sides (x1, x2
    and their sum exact in fp16: multiples of 1/4 below 64)."""
    rng = np.random.default_rng(21)
    w = workloads.random_bcq(3000, 4096, 3, 128, m=1, seed=21, with_offset=True)
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, w.offset, w.g)
    x1 = (rng.integers(-64, 64, size=(1, w.K)) / 4).astype(np.float16)
    x2 = (rng.integers(-64, 64, size=(1, w.K)) / 4).astype(np.float16)
    xs = (x1.astype(np.float64) + x2.astype(np.float64)).astype(np.float16)
    assert np.array_equal(xs.astype(np.float64), x1.astype(np.float64) + x2.astype(np.float64))
    _say("linearity")
    y1, y2, ys = (_gpu_y(pw, v).astype(np.float64) for v in (x1, x2, xs))
    _, b1 = oracle.gemv(w.bits, w.alpha, w.offset, x1, w.g)
    _, b2 = oracle.gemv(w.bits, w.alpha, w.offset, x2, w.g)
    _, bs = oracle.gemv(w.bits, w.alpha, w.offset, xs, w.g)
    lim = 1e-3 * (b1 + b2 + bs) + 3e-4
    assert np.all(np.abs(ys - (y1 + y2)) <= lim)


def test_llama7b_int4_uniform_all_outputs():
    w = workloads.generate("llama7b_mlp_int4")
    _say("llama7b_mlp_int4 11008x4096 int4 zero 8 -> BCQ q4 + offset")
    pw = lg.PackedBCQ.from_uniform(w.codes, w.scale, w.zero, w.q, w.g)
    y = _gpu_y(pw, w.x)
    # against the uniform matrix by definition: s * (c - z)
    Wd = oracle.dequant_uniform(w.codes, w.scale, w.zero, w.g)
    x64 = w.x.astype(np.float64)
    ref = x64 @ Wd.T
    bound = np.abs(x64) @ np.abs(Wd).T
    ok, worst = oracle.parity_ok(y.astype(np.float64), ref, bound)
    _say(f"llama7b vs dequantized definition: worst {worst:.3f}; n_rounded={pw.n_rounded}")
    assert ok
    # and against the BCQ form the rewrite produced
    bits, alpha, off, _ = oracle.uniform_to_bcq(w.codes, w.scale, w.zero, w.q, w.g)
    wb = workloads.Workload(w.name, w.N, w.K, w.q, w.g, w.m, w.x, bits, alpha, off)
    _check(y, wb, rows=_sample_rows(w.N, 1024))


@pytest.mark.parametrize("m", [8, 24])
def test_llama7b_int4_uniform_batched(m):
    """The int4 MLP at batch 8 and 24: the sign-plane MFMA kernel at 8 waves with
    the offset plane (x per item at 8), against the dequantized definition."""
    w0 = workloads.generate("llama7b_mlp_int4")
    x = np.random.default_rng(60 + m).standard_normal((m, w0.K)).astype(np.float16)
    plan = lg.query_plan(w0.N, w0.K, w0.q, w0.g, True, m)
    assert plan["tables"] == "sign_mfma" and plan["waves"] == 8, plan
    _say(f"llama7b int4 at m={m}: plan={plan}")
    pw = lg.PackedBCQ.from_uniform(w0.codes, w0.scale, w0.zero, w0.q, w0.g)
    y = _gpu_y(pw, x)
    Wd = oracle.dequant_uniform(w0.codes, w0.scale, w0.zero, w0.g)
    x64 = x.astype(np.float64)
    ok, worst = oracle.parity_ok(y.astype(np.float64), x64 @ Wd.T, np.abs(x64) @ np.abs(Wd).T)
    _say(f"llama7b int4 at m={m} vs dequantized definition: worst {worst:.3f}")
    assert ok


@pytest.mark.parametrize("m", [4, 16, 32])
def test_decode_batch_all_outputs(m):
    w = workloads.generate(f"decode_m{m}")
    _say(f"decode m={m} 12288x12288 q3 g128")
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, None, w.g)
    y = _gpu_y(pw, w.x)
    _check(y, w)


@pytest.mark.parametrize("q", [1, 2, 4])
@pytest.mark.parametrize("g", [32, 64, 128, 8192])
def test_subbit_sweep_sampled(q, g):
    w = workloads.generate(f"subbit_q{q}_g{g}")
    _say(f"subbit q={q} g={g} 28672x8192")
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, None, w.g)
    y = _gpu_y(pw, w.x)
    _check(y, w, rows=_sample_rows(w.N, 1024, seed=q * 1000 + g))


# ---------------------------------------------------------------- edge cases

@pytest.mark.parametrize("N,K,q,g,m,off", [
    (1, 512, 3, 128, 1, False),       # one row
    (17, 520, 3, 8, 1, True),         # ragged rows and a ragged 1-chunk input tile, g=8
    (1000, 4104, 2, 24, 3, True),     # g not a multiple of 32; ragged everything
    (64, 8, 1, 8, 2, False),          # K = 8: one chunk
    (300, 1536, 5, 64, 5, True),      # q=5, batch not a multiple of 4
    (129, 2048, 6, 256, 2, False),
    (77, 1024, 7, 32, 1, True),
    (48, 1024, 8, 16, 4, True),       # q=8, g=16
    (4096, 512, 4, 512, 7, False),
    (20000, 1024, 3, 128, 1, False),  # many row blocks, short K
])
def test_edge_shapes_all_outputs(N, K, q, g, m, off):
    w = workloads.random_bcq(N, K, q, g, m=m, seed=N + K + q, with_offset=off, name=f"edge_{N}x{K}q{q}g{g}m{m}")
    _say(f"edge N={N} K={K} q={q} g={g} m={m} offset={off}")
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, w.offset, w.g)
    _check(_gpu_y(pw, w.x), w)


def test_zero_input_gives_exact_zero():
    w = workloads.random_bcq(256, 1024, 3, 128, m=2, seed=3, with_offset=True, x_dist="zeros")
    _say("x = 0")
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, w.offset, w.g)
    y = _gpu_y(pw, w.x)
    assert (y.view(np.uint16) & 0x7FFF == 0).all()


def test_integer_case_is_exact():
    """q=1, alpha=1, integer x: every partial sum is an integer below 2^11, so
    the fp32 path and the fp16 output are exact: y = B x in integers."""
    rng = np.random.default_rng(9)
    N, K = 200, 1024
    bits = rng.integers(0, 256, size=(1, N, K // 8), dtype=np.uint8)
    alpha = np.ones((1, N, K // 128), np.float16)
    xi = rng.integers(-1, 2, size=(1, K))
    _say("integer exactness q=1")
    pw = lg.PackedBCQ.from_bcq(bits, alpha, None, 128)
    y = _gpu_y(pw, xi.astype(np.float16))
    signs = oracle.signs(bits)[0].astype(np.int64)          # [N][K]
    expect = xi @ signs.T
    assert np.array_equal(y.astype(np.int64), expect)


def test_unit_vector_probes():
    """x = e_k returns column k of W_hat: probes the layout column by column."""
    w = workloads.random_bcq(40, 1024, 3, 64, seed=4, with_offset=True)
    Wh = oracle.reconstruct_rows(w.bits, w.alpha, w.offset, w.g, np.arange(w.N))
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, w.offset, w.g)
    ks = [0, 1, 7, 8, 63, 64, 511, 512, 513, 1023]
    X = np.zeros((len(ks), w.K), np.float16)
    for r, k in enumerate(ks):
        X[r, k] = 1
    _say("unit-vector probes")
    y = _gpu_y(pw, X)
    for r, k in enumerate(ks):
        col = Wh[:, k]
        assert np.allclose(y[r].astype(np.float64), col, rtol=1e-3, atol=1e-4), k


def test_empty_shapes():
    _say("empty shapes")
    w = workloads.random_bcq(32, 512, 2, 128, m=1, seed=1)
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, None, w.g)
    x0 = torch.zeros((0, 512), dtype=torch.float16, device=DEV)
    assert pw(x0).shape == (0, 32)
    # K = 0: the empty sum, y = 0
    pk = lg.PackedBCQ(32, 0, 2, 8, torch.zeros(16, dtype=torch.uint8, device=DEV),
                      torch.zeros(16, dtype=torch.int16, device=DEV))
    y = torch.full((3, 32), 7.0, dtype=torch.float16, device=DEV)
    pk(torch.zeros((3, 0), dtype=torch.float16, device=DEV), out=y)
    torch.cuda.synchronize()
    assert (y == 0).all()


def test_bitwise_deterministic_and_split_consistent(monkeypatch):
    w = workloads.random_bcq(4096, 8192, 3, 128, m=1, seed=5)
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, None, w.g)
    x = torch.from_numpy(w.x).to(DEV)
    _say("determinism")
    ys = [pw(x).clone() for _ in range(5)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y, ys[0])
    # other splits of the reduction give results within tolerance of the oracle
    # "RPW,S,W,MC,ring,RI": RI < W*RPW leaves waves without rows in a row block
    for tile in ["4,1", "4,3", "2,16", "1,2", "1,1,16,1,3,12", "2,2,16,1,2,13", "1,3,8,1,0,5"]:
        monkeypatch.setenv("LUTGEMM_TILE", tile)
        _say(f"split override {tile}")
        y = pw(x)
        torch.cuda.synchronize()
        _check(y.cpu().numpy(), w, rows=_sample_rows(w.N, 512))
    monkeypatch.delenv("LUTGEMM_TILE")


# "RPW,S,W,MC,ring,RI,XL,PR": paired tables (two batch rows per table entry)
@pytest.mark.parametrize("tile", ["1,1,8,2,0,8,0,1", "2,1,8,4,0,16,0,1", "1,3,8,4,0,5,0,1",
                                  "2,2,8,2,0,13,0,1", "1,2,16,2,0,16,0,1", "1,1,16,2,0,11,0,1"])
@pytest.mark.parametrize("N,K,q,g,m,off", [
    (1000, 4128, 3, 32, 3, True),      # ragged rows and input tiles, odd batch
    (300, 1536, 5, 64, 5, False),
    (1024, 12288, 3, 128, 4, False),
    (129, 2048, 8, 256, 7, True),
])
def test_paired_tables_all_outputs(monkeypatch, tile, N, K, q, g, m, off):
    w = workloads.random_bcq(N, K, q, g, m=m, seed=N + q + m, with_offset=off,
                             name=f"paired_{N}x{K}q{q}g{g}m{m}")
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, w.offset, w.g)
    monkeypatch.setenv("LUTGEMM_TILE", tile)
    _say(f"paired tables {tile}: N={N} K={K} q={q} g={g} m={m} offset={off}")
    _check(_gpu_y(pw, w.x), w)
    monkeypatch.delenv("LUTGEMM_TILE")


# PR = 2: half paired tables (entries with bit 7 clear, double-buffered); the
# bytes with bit 7 set read the complementary entry negated
@pytest.mark.parametrize("tile", ["1,1,16,2,0,16,0,2", "1,3,16,2,0,11,0,2", "1,1,8,4,0,8,0,2",
                                  "1,2,8,2,0,5,0,2", "1,4,8,4,0,7,0,2"])
@pytest.mark.parametrize("N,K,q,g,m,off", [
    (1000, 4128, 3, 32, 3, True),      # ragged rows and input tiles, odd batch
    (300, 1536, 5, 64, 5, False),
    (1024, 12288, 3, 128, 4, False),
    (129, 2048, 8, 256, 7, True),
    (700, 1024, 2, 32, 1, True),       # one batch row: the pair's second row is zero
    (513, 3072, 1, 512, 10, False),
])
def test_half_tables_all_outputs(monkeypatch, tile, N, K, q, g, m, off):
    w = workloads.random_bcq(N, K, q, g, m=m, seed=N + q + m + 7, with_offset=off,
                             name=f"half_{N}x{K}q{q}g{g}m{m}")
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, w.offset, w.g)
    monkeypatch.setenv("LUTGEMM_TILE", tile)
    _say(f"half tables {tile}: N={N} K={K} q={q} g={g} m={m} offset={off}")
    _check(_gpu_y(pw, w.x), w)
    monkeypatch.delenv("LUTGEMM_TILE")


# PR = 3: split paired tables (half an input tile per table, double-buffered;
# 16 waves, one row tile per wave, two batch rows: built for q <= 3)
@pytest.mark.parametrize("tile", ["1,1,16,2,0,16,0,3", "1,3,16,2,0,11,0,3", "1,2,16,2,0,5,0,3"])
@pytest.mark.parametrize("N,K,q,g,m,off", [
    (1000, 4128, 3, 32, 3, True),      # ragged rows and input tiles, odd batch
    (300, 1536, 2, 64, 5, False),
    (1024, 12288, 3, 128, 4, False),
    (129, 2048, 1, 256, 7, True),
    (700, 1024, 2, 32, 1, True),       # one batch row: the pair's second row is zero
    (513, 3072, 1, 512, 10, False),
    (2000, 1536, 3, 1536, 2, True),    # one scale group per row
])
def test_split_paired_tables_all_outputs(monkeypatch, tile, N, K, q, g, m, off):
    w = workloads.random_bcq(N, K, q, g, m=m, seed=N + q + m + 11, with_offset=off,
                             name=f"split_{N}x{K}q{q}g{g}m{m}")
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, w.offset, w.g)
    monkeypatch.setenv("LUTGEMM_TILE", tile)
    assert lg.query_plan(N, K, q, g, off, m)["tables"] == "split"
    _say(f"split paired tables {tile}: N={N} K={K} q={q} g={g} m={m} offset={off}")
    _check(_gpu_y(pw, w.x), w)
    monkeypatch.delenv("LUTGEMM_TILE")


# PR = 4: paired tables built by MFMA (the sign matrix times the activations;
# 16 waves, one row tile per wave, two batch rows: built for q <= 3)
@pytest.mark.parametrize("tile", ["1,1,16,2,0,16,0,4", "1,3,16,2,0,11,0,4", "1,2,16,2,0,5,0,4"])
@pytest.mark.parametrize("N,K,q,g,m,off", [
    (1000, 4128, 3, 32, 3, True),      # ragged rows and input tiles, odd batch
    (300, 1536, 2, 64, 5, False),
    (1024, 12288, 3, 128, 4, False),
    (129, 2048, 1, 256, 7, True),
    (700, 1056, 2, 32, 1, True),       # one batch row; the last input tile holds 4 chunks
    (513, 3072, 1, 512, 10, False),
    (2000, 1536, 3, 1536, 2, True),    # one scale group per row
])
def test_mfma_built_tables_all_outputs(monkeypatch, tile, N, K, q, g, m, off):
    w = workloads.random_bcq(N, K, q, g, m=m, seed=N + q + m + 13, with_offset=off,
                             name=f"mfma_{N}x{K}q{q}g{g}m{m}")
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, w.offset, w.g)
    monkeypatch.setenv("LUTGEMM_TILE", tile)
    if g % 32 == 0:
        assert lg.query_plan(N, K, q, g, off, m)["tables"] == "paired_mfma"
    _say(f"MFMA-built tables {tile}: N={N} K={K} q={q} g={g} m={m} offset={off}")
    _check(_gpu_y(pw, w.x), w)
    monkeypatch.delenv("LUTGEMM_TILE")


# PR = 5: the sign-plane MFMA kernel ("RPW,S,W,MC,...,PR": split S, W waves and
# MC = 16 or 32 batch rows per item, 0 for the kernel's own choice): ragged
# rows, input tiles with fewer than four step groups, several batch groups,
# offsets, scale groups of 128..512 inputs, every plane count
@pytest.mark.parametrize("tile", ["1,0,0,0,0,0,0,5", "1,1,0,16,0,0,0,5", "1,3,8,0,0,0,0,5",
                                  "1,7,0,16,0,0,0,5"])
@pytest.mark.parametrize("N,K,q,g,m,off", [
    (1000, 4224, 3, 128, 4, False),    # the last input tile holds one step group
    (300, 1536, 2, 256, 17, True),     # two groups of 16 batch rows
    (1024, 12288, 3, 128, 32, False),
    (129, 3072, 1, 384, 7, True),      # groups straddle input tiles
    (700, 1536, 4, 512, 2, True),
    (513, 4096, 8, 128, 40, False),    # three batch groups of 16
    (250, 2560, 6, 128, 33, True),
    (64, 512, 3, 128, 3, False),
    (700, 1024, 5, 128, 1, False),     # one batch row
])
def test_sign_mfma_all_outputs(monkeypatch, tile, N, K, q, g, m, off):
    w = workloads.random_bcq(N, K, q, g, m=m, seed=N + 7 * q + m, with_offset=off,
                             name=f"signmfma_{N}x{K}q{q}g{g}m{m}")
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, w.offset, w.g)
    monkeypatch.setenv("LUTGEMM_TILE", tile)
    plan = lg.query_plan(N, K, q, g, off, m)
    assert plan["tables"] == "sign_mfma", plan
    _say(f"sign MFMA {tile}: N={N} K={K} q={q} g={g} m={m} offset={off} plan={plan}")
    _check(_gpu_y(pw, w.x), w)
    monkeypatch.delenv("LUTGEMM_TILE")


# The sign-plane MFMA kernel with x staged once per item (XL = 1 where its
# conditions hold: one group of 16 batch rows, no more items than CUs, at most
# five input tiles per item): ragged rows and batches, a last input tile of one
# step group, offsets, groups straddling input tiles, 8-wave instances (q = 5)
@pytest.mark.parametrize("tile,N,K,q,g,m,off", [
    ("1,3,16,16,0,0,1,5", 1000, 4224, 3, 128, 4, False),
    ("1,2,0,0,0,0,1,5", 1000, 4224, 3, 128, 4, False),     # five tiles per item
    ("1,0,0,0,0,0,1,5", 300, 1536, 2, 256, 12, True),
    ("1,2,16,16,0,0,1,5", 513, 4096, 3, 128, 16, False),
    ("1,4,0,0,0,0,1,5", 129, 3072, 1, 384, 7, True),
    ("1,1,0,0,0,0,1,5", 64, 512, 3, 128, 3, False),
    ("1,3,8,0,0,0,1,5", 2048, 2560, 5, 128, 9, False),
    ("", 4096, 12288, 3, 128, 5, False),                    # the default launch
])
def test_sign_mfma_x_per_item_all_outputs(monkeypatch, tile, N, K, q, g, m, off):
    w = workloads.random_bcq(N, K, q, g, m=m, seed=3 * N + q + m, with_offset=off,
                             name=f"signmfma_xi_{N}x{K}q{q}g{g}m{m}")
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, w.offset, w.g)
    monkeypatch.setenv("LUTGEMM_TILE", tile)
    plan = lg.query_plan(N, K, q, g, off, m)
    assert plan["tables"] == "sign_mfma" and plan["x_in_lds"] == 1, plan
    _say(f"sign MFMA, x per item {tile}: N={N} K={K} q={q} g={g} m={m} offset={off} plan={plan}")
    _check(_gpu_y(pw, w.x), w)
    # and the same product with x staged per input tile
    monkeypatch.setenv("LUTGEMM_TILE", (tile or "1,0,0,0,0,0,1,5").replace(",1,5", ",0,5"))
    assert lg.query_plan(N, K, q, g, off, m)["x_in_lds"] == 0
    _check(_gpu_y(pw, w.x), w)
    monkeypatch.delenv("LUTGEMM_TILE")


# The dispatcher's own batched launches: the sign-plane MFMA kernel from 3 batch
# rows on larger matrices (x per item), 8 waves x 32 batch rows per item past 16
# rows (with an offset, scale groups of 256), the tables for a small matrix at 3
@pytest.mark.parametrize("N,K,q,g,m,off,tables,batch_rows", [
    (12288, 4096, 3, 128, 3, False, "sign_mfma", 16),
    (6144, 8192, 3, 128, 5, False, "sign_mfma", 16),
    (4096, 12288, 3, 256, 20, False, "sign_mfma", 32),
    (3072, 8192, 2, 128, 64, True, "sign_mfma", 32),
    (4096, 4096, 3, 128, 3, False, "single", 1),
])
def test_batched_default_launches_all_outputs(N, K, q, g, m, off, tables, batch_rows):
    w = workloads.random_bcq(N, K, q, g, m=m, seed=N + K + m, with_offset=off,
                             name=f"batched_{N}x{K}q{q}g{g}m{m}")
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, w.offset, w.g)
    plan = lg.query_plan(N, K, q, g, off, m)
    assert plan["tables"] == tables and plan["batch_rows"] == batch_rows, plan
    _say(f"batched default launch: N={N} K={K} q={q} g={g} m={m} offset={off} plan={plan}")
    _check(_gpu_y(pw, w.x), w)


# "RPW,S,W,MC,ring,RI,XL,PR,EI": x in LDS with the early-issue ring (EI = 1), forced
# onto single-item, split and many-item launches, and the plain ring beside it (EI = 0)
@pytest.mark.parametrize("tile", ["1,1,16,1,0,12,1,0,1", "1,1,16,1,0,12,1,0,0", "1,3,16,1,0,5,1,0,1",
                                  "2,2,16,1,0,20,1,0,1"])
@pytest.mark.parametrize("N,K,q,g,m,off", [
    (3000, 4128, 3, 32, 1, True),      # ragged rows and input tiles
    (2000, 12288, 3, 128, 1, False),
    (777, 15360, 4, 64, 1, True),      # the largest x staged in LDS
    (64, 512, 1, 32, 1, False),        # one input tile: fewer tiles than ring steps
])
def test_early_issue_ring_all_outputs(monkeypatch, tile, N, K, q, g, m, off):
    w = workloads.random_bcq(N, K, q, g, m=m, seed=N + K + q, with_offset=off,
                             name=f"early_issue_{N}x{K}q{q}g{g}")
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, w.offset, w.g)
    monkeypatch.setenv("LUTGEMM_TILE", tile)
    _say(f"early-issue ring {tile}: N={N} K={K} q={q} g={g} offset={off}")
    _check(_gpu_y(pw, w.x), w)
    monkeypatch.delenv("LUTGEMM_TILE")


# batch 1 with x too long for LDS: read-once (non-temporal) sign-plane loads, in the
# dispatcher's configuration and in forced ones (split, two row tiles per wave, 3-deep ring)
@pytest.mark.parametrize("tile", ["", "1,3,16,1,0,16", "2,2,16,1,0,20", "1,4,16,1,3,12"])
@pytest.mark.parametrize("N,K,q,g,off", [(2000, 20480, 3, 128, False), (333, 16896, 4, 64, True)])
def test_read_once_batch1_long_x_all_outputs(monkeypatch, tile, N, K, q, g, off):
    w = workloads.random_bcq(N, K, q, g, m=1, seed=N + K, with_offset=off,
                             name=f"read_once_{N}x{K}q{q}g{g}")
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, w.offset, w.g)
    if tile:
        monkeypatch.setenv("LUTGEMM_TILE", tile)
    _say(f"read-once loads {tile or 'default'}: N={N} K={K} q={q} g={g} offset={off}")
    _check(_gpu_y(pw, w.x), w)
    monkeypatch.delenv("LUTGEMM_TILE", raising=False)


# 2 or 3 batch groups of one-row items, items per batch group a multiple of 8: the batch
# groups of one weight block run side by side on one XCD, split reductions included
@pytest.mark.parametrize("tile,N,K,m", [("1,3,16,1,0,16", 2048, 12288, 3), ("1,2,16,1,0,16", 1000, 8192, 2),
                                        ("1,1,16,1,0,16", 2048, 4096, 2), ("2,4,16,1,0,32", 4096, 4096, 3)])
def test_xcd_grouped_batch_groups_all_outputs(monkeypatch, tile, N, K, m):
    w = workloads.random_bcq(N, K, 3, 128, m=m, seed=N + K + m, with_offset=True,
                             name=f"xcd_groups_{N}x{K}m{m}")
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, w.offset, w.g)
    monkeypatch.setenv("LUTGEMM_TILE", tile)
    _say(f"batch groups on one XCD {tile}: N={N} K={K} m={m}")
    _check(_gpu_y(pw, w.x), w)
    monkeypatch.delenv("LUTGEMM_TILE")


def test_workspace_reuse_across_shapes():
    """One workspace (through the C ABI) serves a large split call, then a smaller
    one, then the large again: each completed call leaves its counters zero."""
    big = workloads.random_bcq(8192, 12288, 3, 128, m=2, seed=6)
    small = workloads.random_bcq(1024, 4096, 2, 64, m=3, seed=7)
    pb = lg.PackedBCQ.from_bcq(big.bits, big.alpha, None, big.g)
    ps = lg.PackedBCQ.from_bcq(small.bits, small.alpha, None, small.g)
    nb = lg.workspace_size(big.N, big.K, big.q, big.g, False, 2)
    ns = lg.workspace_size(small.N, small.K, small.q, small.g, False, 3)
    assert nb > 0 and ns > 0
    ws = torch.empty(max(nb, ns), dtype=torch.uint8, device=DEV)
    sh = torch.cuda.current_stream().cuda_stream
    lg.workspace_init(ws.data_ptr(), ws.numel(), sh)
    _say("workspace reuse")
    for w, p in [(big, pb), (small, ps), (big, pb), (small, ps)]:
        x = torch.from_numpy(w.x).to(DEV)
        y = torch.empty((w.m, w.N), dtype=torch.float16, device=DEV)
        lg.lutgemm_run(p.shape, w.m, p.d_bits.data_ptr(), p.d_alpha.data_ptr(), None,
                       x.data_ptr(), y.data_ptr(), ws.data_ptr(), ws.numel(), sh)
        torch.cuda.synchronize()
        _check(y.cpu().numpy(), w, rows=_sample_rows(w.N, 256))


def test_large_batch_and_many_rows():
    w = workloads.random_bcq(64, 512, 2, 128, m=300, seed=8)
    _say("m=300")
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, None, w.g)
    _check(_gpu_y(pw, w.x), w)
    w = workloads.random_bcq(200000, 512, 1, 512, m=1, seed=9)
    _say("N=200000")
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, None, w.g)
    _check(_gpu_y(pw, w.x), w, rows=_sample_rows(w.N, 2048))


def test_quantized_fp16_matrix_end_to_end():
    """fp16 W -> bcq_quantize -> bcq_pack -> lutgemm_run, against the oracle's
    product of the oracle's own quantization of the same W (bit-identical)."""
    rng = np.random.default_rng(12)
    N, K, q, g, m = 700, 2048, 3, 64, 3
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    x = rng.standard_normal((m, K)).astype(np.float16)
    bits, alpha, _ = lg.bcq_quantize(W, q, g, iters=2)
    ob, oa, _ = oracle.quantize_bcq(W[:64], q, g, 2)            # a slice, for time
    assert np.array_equal(bits[:, :64], ob) and np.array_equal(alpha[:, :64].view(np.uint16),
                                                               oa.view(np.uint16))
    _say("quantize -> pack -> run")
    pw = lg.PackedBCQ.from_bcq(bits, alpha, None, g)
    w = workloads.Workload("quantized", N, K, q, g, m, x, bits, alpha, None)
    _check(_gpu_y(pw, x), w)


def test_cancelling_planes_with_activation_outliers():
    """Planes that cancel plus activation outliers: in every chunk the first input
    is 1000 and its two plane bits are opposite with equal scales, so its weight
    is exactly 0; the outlier then enters both table entries of a row but not the
    bound sum_k |W_hat x|. fp16 table entries fail this input (the worst output
    at about 11x the tolerance, in an exact simulation of such entries); the fp32
    tables must pass it on every output."""
    rng = np.random.default_rng(31)
    N, K, q, g = 256, 4096, 2, 128
    x = rng.standard_normal((1, K))
    x[0, ::8] = 1000.0
    x = x.astype(np.float16)
    bits = rng.integers(0, 256, size=(q, N, K // 8), dtype=np.uint8)
    bits[1] = bits[0] ^ 0x01                      # bit 0 (input 8c) opposite in the two planes
    a0 = (np.abs(rng.standard_normal((N, K // g))) * 0.02).astype(np.float16)
    alpha = np.stack([a0, a0])                    # equal scales: the outlier's weight is 0
    w = workloads.Workload("cancel_outlier", N, K, q, g, 1, x, bits, alpha, None)
    Wh = oracle.reconstruct_rows(bits, alpha, None, g, np.arange(N))
    assert (Wh[:, ::8] == 0).all()
    _say("cancelling planes + outliers")
    pw = lg.PackedBCQ.from_bcq(bits, alpha, None, g)
    _check(_gpu_y(pw, x), w)


@pytest.mark.parametrize("kind", ["nan", "inf"])
def test_non_finite_x_propagates(kind):
    """x is not checked: a NaN or an infinity in x makes every output non-finite,
    as in the exact product (every row reads every input). The kind may differ:
    an infinite input can give NaN where the exact product is infinite, because
    the table entries are built as differences (IEEE inf - inf)."""
    w = workloads.random_bcq(500, 2048, 3, 128, m=2, seed=41, with_offset=True)
    x = w.x.copy()
    x[0, 777] = np.float16(np.nan) if kind == "nan" else np.float16(np.inf)
    x[1, 5] = np.float16(np.nan) if kind == "nan" else -np.float16(np.inf)
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, w.offset, w.g)
    _say(f"non-finite x ({kind})")
    y = _gpu_y(pw, x).astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        ref, _ = oracle.gemv(w.bits, w.alpha, w.offset, x, w.g)
    assert (~np.isfinite(ref)).all()
    assert (~np.isfinite(y)).all()
    if kind == "nan":
        assert np.isnan(y).all()


def test_maximum_split_all_outputs(monkeypatch):
    """The input dimension split 64 ways (the most the dispatcher uses) on a shape
    with 16 row blocks and 4 items per workgroup: 1024 partial-sum items meet in
    the fused reduction. Three runs, each checked on every output and bitwise
    equal to the first; the loop stops at its first failure."""
    w = workloads.random_bcq(4096, 32768, 3, 128, m=1, seed=43, name="split64_4096x32768")
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, None, w.g)
    ref = oracle.gemv(w.bits, w.alpha, None, w.x, w.g)
    x = torch.from_numpy(w.x).to(DEV)
    monkeypatch.setenv("LUTGEMM_TILE", "1,64,16,1")
    first = None
    for rep in range(3):
        _say(f"split 64, run {rep}")
        y = pw(x)
        torch.cuda.synchronize()
        yn = y.cpu().numpy()
        _check(yn, w, ref=ref)
        if first is None:
            first = yn
        else:
            assert np.array_equal(yn.view(np.uint16), first.view(np.uint16))
    monkeypatch.delenv("LUTGEMM_TILE")


def test_two_streams_share_a_weight():
    """Split launches of one weight on two streams at once: each stream has its
    own workspace, and both results match the oracle."""
    w = workloads.random_bcq(6144, 12288, 3, 128, m=2, seed=44)
    assert lg.workspace_size(w.N, w.K, w.q, w.g, False, 2) > 0
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, None, w.g)
    x = torch.from_numpy(w.x).to(DEV)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    _say("two streams")
    ys = []
    for _ in range(4):
        with torch.cuda.stream(s1):
            ys.append(pw(x))
        with torch.cuda.stream(s2):
            ys.append(pw(x))
    torch.cuda.synchronize()
    assert len(pw._ws) >= 2
    ref = oracle.gemv(w.bits, w.alpha, None, w.x, w.g)
    for y in ys:
        _check(y.cpu().numpy(), w, ref=ref)


def test_fake_arch_is_refused_before_launch(monkeypatch):
    """LUTGEMM_FAKE_ARCH makes the device report another architecture: both
    products refuse with LUTGEMM_ERR_UNSUPPORTED and write nothing."""
    w = workloads.random_bcq(64, 512, 2, 128, m=1, seed=45)
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, None, w.g)
    x = torch.from_numpy(w.x).to(DEV)
    y = torch.full((1, 64), 3.0, dtype=torch.float16, device=DEV)
    monkeypatch.setenv("LUTGEMM_FAKE_ARCH", "gfx942")
    _say("fake arch")
    with pytest.raises(lg.LutGemmError) as e:
        pw(x, out=y)
    assert e.value.status == 6
    with pytest.raises(lg.LutGemmError) as e:
        pw.dequant(x, out=y)
    assert e.value.status == 6
    torch.cuda.synchronize()
    assert (y == 3.0).all()
    monkeypatch.delenv("LUTGEMM_FAKE_ARCH")
    _check(_gpu_y(pw, w.x), w)


def test_stream_read_probe_runs():
    """The streaming-read measurement kernel reads a buffer and writes nothing
    (its fold equals the magic value only by a 2^-32 chance per workgroup)."""
    n = (64 << 20) + 4096
    src = torch.ones(n, dtype=torch.uint8, device=DEV)
    sink = torch.zeros(1024, dtype=torch.int32, device=DEV)
    sh = torch.cuda.current_stream().cuda_stream
    lg.stream_read(src.data_ptr(), n, sink.data_ptr(), sink.numel(), True, sh)
    lg.stream_read(src.data_ptr(), n, sink.data_ptr(), sink.numel(), False, sh)
    torch.cuda.synchronize()
    assert (sink == 0).all()
    with pytest.raises(lg.LutGemmError):
        lg.stream_read(src.data_ptr() + 8, n - 16, sink.data_ptr(), sink.numel(), True, sh)


# the phase-traced build: same results as the regular one, stamps in order
@pytest.mark.parametrize("N,K,q,g,m,off,tile", [
    (32768, 4096, 3, 128, 1, False, None),   # x in LDS, early-issue ring (8 row tiles per CU)
    (4096, 12288, 3, 128, 1, True, None),    # split of the input dimension
    (4096, 4096, 2, 128, 1, False, None),    # nibble tables
    (2048, 3072, 3, 64, 4, True, "1,2,16,2,0,16,0,1"),   # paired tables
])
def test_phase_traced_build(monkeypatch, N, K, q, g, m, off, tile):
    import ctypes
    if not os.path.exists(lg.TRACE_LIB_PATH):
        pytest.skip("phase-traced library not built")
    if tile:
        monkeypatch.setenv("LUTGEMM_TILE", tile)
    T = ctypes.CDLL(lg.TRACE_LIB_PATH)
    T.lutgemm_trace_attach.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    T.lutgemm_run.argtypes = [ctypes.POINTER(lg.Shape), ctypes.c_int32] + [ctypes.c_void_p] * 6 + \
        [ctypes.c_size_t, ctypes.c_void_p]
    w = workloads.random_bcq(N, K, q, g, m=m, seed=N + K + m, with_offset=off, name=f"trace_{N}x{K}m{m}")
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, w.offset, w.g)
    x = torch.from_numpy(w.x).to(DEV)
    y_ref = pw(x)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plan = lg.query_plan(N, K, q, g, off, m, cus=cus,
                         workspace_bytes=None if cus == 256 else lg.workspace_size(N, K, q, g, off, m))
    _say(f"phase-traced build: {N}x{K} q={q} g={g} m={m} offset={off} plan={plan}")
    nwg = plan["workgroups"]
    stamps = torch.zeros(nwg * 8, dtype=torch.int64, device=DEV)
    nws = max(16, lg.workspace_size(N, K, q, g, off, m))
    wsp = torch.zeros(nws, dtype=torch.uint8, device=DEV)
    y = torch.empty((m, N), dtype=torch.float16, device=DEV)
    sh = torch.cuda.current_stream().cuda_stream
    assert T.lutgemm_trace_attach(stamps.data_ptr(), stamps.numel() * 8) == 0
    try:
        for _ in range(2):
            st = T.lutgemm_run(ctypes.byref(pw.shape), m, pw.d_bits.data_ptr(), pw.d_alpha.data_ptr(),
                               pw.d_offset.data_ptr() if pw.has_offset else None, x.data_ptr(),
                               y.data_ptr(), wsp.data_ptr(), nws, sh)
            assert st == 0
        torch.cuda.synchronize()
    finally:
        T.lutgemm_trace_attach(None, 0)
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    t = stamps.cpu().numpy().reshape(nwg, 8)
    assert (t[:, 0] > 0).all() and (t[:, 5] > 0).all() and (t[:, 6:] == 0).all()
    order = [0, 2, 3, 4, 5]
    for a, b in zip(order, order[1:]):
        assert (t[:, b] >= t[:, a]).all(), (a, b)
    assert ((t[:, 5] - t[:, 0]) < 100_000).all()    # under 1 ms at 100 MHz


# the nibble-table unit kernel (batch 1, few row tiles per compute unit):
# "0,1,16,1,NR,RI,1,0,0,1" forces it with RI row tiles per workgroup and ring depth NR
@pytest.mark.parametrize("N,K,q,g,off,ri,nr", [
    (11008, 4096, 4, 128, True, 3, 0),     # the int4 MLP shape: one plane-0 unit per row tile
    (3000, 4128, 3, 32, True, 2, 8),       # ragged rows and a ragged last input tile
    (3000, 4128, 3, 32, True, 5, 4),       # units 0..14 with 16 waves: one wave idle
    (777, 15360, 4, 64, True, 7, 4),       # the largest x staged in LDS, two units per wave
    (777, 15360, 4, 64, True, 7, 2),
    (64, 512, 1, 32, False, 1, 8),         # one input tile: fewer tiles than ring steps
    (1000, 8192, 8, 8192, True, 2, 0),     # row-wise groups (one group per row), q = 8
    (1000, 8192, 8, 8192, True, 7, 0),     # 56 units: four per wave
    (2000, 2048, 5, 256, False, 4, 0),     # two groups per input tile
    (500, 3072, 2, 1024, True, 6, 0),      # groups wider than an input tile
    (900, 7680, 6, 1536, True, 3, 2),      # groups of three input tiles, 18 units
    (512, 512, 3, 128, False, 1, 0),       # one row tile per workgroup, one input tile
    (6144, 12288, 3, 128, False, 2, 0),    # the one-of-eight row shard of the FFN-up matrix
])
def test_unit_kernel_all_outputs(monkeypatch, N, K, q, g, off, ri, nr):
    """The nibble-table unit kernel: 4-input tables built per phase of 8192
    inputs (15360 inputs: two phases), forced with RI row tiles per workgroup
    and ring depth NR (0: its default)."""
    w = workloads.random_bcq(N, K, q, g, m=1, seed=N + K + q + ri, with_offset=off,
                             x_dist="student_t" if q % 2 else "normal",
                             name=f"units_{N}x{K}q{q}g{g}ri{ri}nr{nr}")
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, w.offset, w.g)
    monkeypatch.setenv("LUTGEMM_TILE", f"0,1,16,1,{nr},{ri},1,0,0,1")
    _say(f"unit kernel RI={ri} NR={nr}: N={N} K={K} q={q} g={g} offset={off}")
    _check(_gpu_y(pw, w.x), w)
    monkeypatch.delenv("LUTGEMM_TILE")


def test_unit_kernel_declined_by_override(monkeypatch):
    """US = 0 in the override gives the dispatcher's choice without the unit
    kernel (split reduction here); both agree with the oracle."""
    w = workloads.random_bcq(6144, 12288, 3, 128, m=1, seed=46)
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, None, w.g)
    ref = oracle.gemv(w.bits, w.alpha, None, w.x, w.g)
    _say("unit kernel declined")
    y_units = _gpu_y(pw, w.x)
    monkeypatch.setenv("LUTGEMM_TILE", "0,0,0,0,0,0,-1,-1,-1,0")
    y_split = _gpu_y(pw, w.x)
    monkeypatch.delenv("LUTGEMM_TILE")
    _check(y_units, w, ref=ref)
    _check(y_split, w, ref=ref)

"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Acceptance per output (the tolerance the GEMV is specified to): |y_gpu - y_ref|
<= 1e-3 * sum_k |W_hat[j,k] x[k]| + 1e-4. Small problems are checked on every
output; the full-size workloads, run in the launch configuration the benchmark
times, are checked on sampled rows the oracle computes one by one.
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


def test_opt175b_ffn_up_sampled():
    w = workloads.generate("opt175b_ffn_up")
    _say("opt175b_ffn_up 49152x12288 q3 g128 m1")
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, None, w.g)
    y = _gpu_y(pw, w.x)
    assert np.isfinite(y).all()
    _check(y, w, rows=_sample_rows(w.N, 2048))


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


@pytest.mark.parametrize("m", [4, 16, 32])
def test_decode_batch_sampled(m):
    w = workloads.generate(f"decode_m{m}")
    _say(f"decode m={m} 12288x12288 q3 g128")
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, None, w.g)
    y = _gpu_y(pw, w.x)
    _check(y, w, rows=_sample_rows(w.N, 512, seed=m))


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
    """One workspace serves a large split call, then a smaller one, then the large again."""
    big = workloads.random_bcq(8192, 12288, 3, 128, m=1, seed=6)
    small = workloads.random_bcq(1024, 4096, 2, 64, m=3, seed=7)
    pb = lg.PackedBCQ.from_bcq(big.bits, big.alpha, None, big.g)
    ps = lg.PackedBCQ.from_bcq(small.bits, small.alpha, None, small.g)
    ps._ws = pb.workspace(1)[0]        # share
    _say("workspace reuse")
    for w, p in [(big, pb), (small, ps), (big, pb), (small, ps)]:
        y = _gpu_y(p, w.x)
        _check(y, w, rows=_sample_rows(w.N, 256))


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

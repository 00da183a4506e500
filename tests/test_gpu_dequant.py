"""Parity of the dequantizing comparison kernel (bcq_dequant_gemv) with the oracle.

It reads the same packed buffers as the LUT-GEMV and must reach the same
tolerance: |y - y_ref| <= 1e-3 * sum_k |W_hat[j,k] x[k]| + 1e-4 per output.
"""
import numpy as np
import pytest
import torch

import lut_gemv_amd as lg
import oracle
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _say(msg):
    print(f"[gpu-dequant] {msg}", flush=True)


def _check(w, pw, rows=None):
    if w.is_uniform:   # the BCQ form the rewrite produced (oracle's own rewrite)
        bits, alpha, off, _ = oracle.uniform_to_bcq(w.codes, w.scale, w.zero, w.q, w.g)
        w = workloads.Workload(w.name, w.N, w.K, w.q, w.g, w.m, w.x, bits, alpha, off)
    x = torch.from_numpy(w.x).to(DEV)
    y = pw.dequant(x)
    torch.cuda.synchronize()
    yg = y.cpu().numpy().astype(np.float64)
    if rows is None:
        rows = np.arange(w.N)
    ref, bound = oracle.gemv(w.bits, w.alpha, w.offset, w.x, w.g, rows=rows)
    ok, worst = oracle.parity_ok(yg[:, rows], ref, bound)
    _say(f"{w.name}: worst err/tol = {worst:.3f} over {ref.size} outputs")
    assert ok, f"{w.name}: worst err/tol {worst}"


def _packed(w):
    if w.is_uniform:
        return lg.PackedBCQ.from_uniform(w.codes, w.scale, w.zero, w.q, w.g)
    return lg.PackedBCQ.from_bcq(w.bits, w.alpha, w.offset, w.g)


def _rows(N, n, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, n)]))


@pytest.mark.parametrize("name", ["tiny", "opt175b_ffn_up", "llama7b_mlp_int4", "decode_m4",
                                  "decode_m16", "subbit_q1_g32", "subbit_q4_g8192"])
def test_workloads(name):
    w = workloads.generate(name)
    _say(name)
    rows = None if w.N * w.m <= 65536 else _rows(w.N, 1024)
    _check(w, _packed(w), rows)


@pytest.mark.parametrize("N,K,q,g,m,off", [(1, 512, 3, 128, 1, False), (17, 520, 3, 8, 1, True),
                                           (1000, 4104, 2, 24, 3, True), (300, 1536, 5, 64, 9, True),
                                           (77, 1024, 8, 32, 1, True)])
def test_edge_shapes(N, K, q, g, m, off):
    w = workloads.random_bcq(N, K, q, g, m=m, seed=N + K, with_offset=off)
    _say(f"edge N={N} K={K} q={q} g={g} m={m} off={off}")
    _check(w, _packed(w))


def test_empty():
    w = workloads.random_bcq(32, 512, 2, 128, m=1, seed=1)
    pw = _packed(w)
    assert pw.dequant(torch.zeros((0, 512), dtype=torch.float16, device=DEV)).shape == (0, 32)
    pk = lg.PackedBCQ(32, 0, 2, 8, torch.zeros(16, dtype=torch.uint8, device=DEV),
                      torch.zeros(16, dtype=torch.int16, device=DEV))
    y = torch.full((3, 32), 7.0, dtype=torch.float16, device=DEV)
    pk.dequant(torch.zeros((3, 0), dtype=torch.float16, device=DEV), out=y)
    torch.cuda.synchronize()
    assert (y == 0).all()

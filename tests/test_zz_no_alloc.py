"""lutgemm_run_noalloc (the entry point that allocates nothing) against
lutgemm_run, through the C ABI.

Two calls in a row on split launches, the second with a smaller input, each
checked against lutgemm_run's output and the fp64 oracle on every output with
the tolerance |y - y_ref| <= 1e-3 * sum_k |W_hat[j,k] x[k]| + 1e-4; a shape
whose best split would not fit the scratch (a smaller split is used); the
refusal of a forced split that would not fit. The scratch is shared by every
call on the GPU, so the calls here are ordered on one stream.
"""
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
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


def _both(w):
    """(y of lutgemm_run, y of lutgemm_run_noalloc) for workload w, on one stream."""
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, w.offset, w.g, device=DEV)
    x = torch.from_numpy(np.ascontiguousarray(w.x)).to(DEV)
    y_run = pw(x)
    y_na = torch.full((w.m, w.N), 7.0, dtype=torch.float16, device=DEV)
    sh = torch.cuda.current_stream().cuda_stream
    lg.lutgemm_run_noalloc(pw.shape, w.m, pw.d_bits.data_ptr(), pw.d_alpha.data_ptr(),
                           pw.d_offset.data_ptr() if pw.d_offset is not None else None,
                           x.data_ptr(), y_na.data_ptr(), sh)
    torch.cuda.synchronize()
    return y_run.cpu().numpy(), y_na.cpu().numpy()


def _check(w, y_run, y_na):
    ref, bound = oracle.gemv(w.bits, w.alpha, w.offset, w.x, w.g)
    ok_run, worst_run = oracle.parity_ok(y_run.astype(np.float64), ref, bound)
    ok_na, worst_na = oracle.parity_ok(y_na.astype(np.float64), ref, bound)
    # the no-alloc output against lutgemm_run's, with the same per-output tolerance
    ok_pair, worst_pair = oracle.parity_ok(y_na.astype(np.float64), y_run.astype(np.float64), bound)
    _say(f"{w.name}: worst err/tol run {worst_run:.3f}, no-alloc {worst_na:.3f}, "
         f"no-alloc vs run {worst_pair:.3f}")
    assert ok_run and ok_na and ok_pair


def test_noalloc_two_calls_second_smaller():
    """The scratch keeps the last call's contents: a large split call, then a
    smaller one (fewer rows, shorter input, another batch), both correct."""
    scratch = lg.noalloc_scratch_bytes()
    assert scratch == 4 << 20
    big = workloads.random_bcq(6144, 12288, 3, 128, m=2, seed=51, name="noalloc_big")
    small = workloads.random_bcq(1000, 4104, 2, 24, m=3, seed=52, with_offset=True,
                                 name="noalloc_small")
    for w in (big, small):
        need = lg.workspace_size(w.N, w.K, w.q, w.g, w.offset is not None, w.m)
        assert 0 < need <= scratch, (w.name, need)
        _say(f"{w.name}: N={w.N} K={w.K} q={w.q} g={w.g} m={w.m}, split workspace {need} B")
        y_run, y_na = _both(w)
        # with the same launch choice the two entry points round identically
        assert np.array_equal(y_run.view(np.uint16), y_na.view(np.uint16))
        _check(w, y_run, y_na)


def test_noalloc_split_limited_to_the_scratch():
    """A batch whose best split needs more than the scratch holds: the no-alloc
    call uses a split that fits (or none) and stays within tolerance."""
    w = workloads.random_bcq(12288, 16384, 3, 128, m=48, seed=53, name="noalloc_m48")
    need = lg.workspace_size(w.N, w.K, w.q, w.g, False, w.m)
    _say(f"{w.name}: lutgemm_run workspace {need} B, scratch {lg.noalloc_scratch_bytes()} B")
    assert need > lg.noalloc_scratch_bytes()
    y_run, y_na = _both(w)
    _check(w, y_run, y_na)


def test_noalloc_small_and_unsplit_shapes():
    """No split (no scratch used), K = 0 and an empty batch."""
    w = workloads.random_bcq(49152 // 8, 512, 3, 128, m=1, seed=54, name="noalloc_nosplit")
    y_run, y_na = _both(w)
    _check(w, y_run, y_na)
    pk = lg.PackedBCQ(32, 0, 2, 8, torch.zeros(16, dtype=torch.uint8, device=DEV),
                      torch.zeros(16, dtype=torch.int16, device=DEV))
    y = torch.full((3, 32), 7.0, dtype=torch.float16, device=DEV)
    x0 = torch.zeros((3, 16), dtype=torch.float16, device=DEV)
    sh = torch.cuda.current_stream().cuda_stream
    lg.lutgemm_run_noalloc(pk.shape, 3, pk.d_bits.data_ptr(), pk.d_alpha.data_ptr(), None,
                           x0.data_ptr(), y.data_ptr(), sh)
    lg.lutgemm_run_noalloc(pk.shape, 0, pk.d_bits.data_ptr(), pk.d_alpha.data_ptr(), None,
                           x0.data_ptr(), y.data_ptr(), sh)
    torch.cuda.synchronize()
    assert (y == 0).all()


def test_noalloc_refuses_a_forced_split_past_the_scratch(monkeypatch):
    w = workloads.random_bcq(4096, 32768, 3, 128, m=8, seed=55)
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, None, w.g, device=DEV)
    x = torch.from_numpy(w.x).to(DEV)
    y = torch.full((w.m, w.N), 7.0, dtype=torch.float16, device=DEV)
    monkeypatch.setenv("LUTGEMM_TILE", "1,64,16,1")   # 64 splits x 8 rows x 4096 x 4 B = 8 MiB
    sh = torch.cuda.current_stream().cuda_stream
    with pytest.raises(lg.LutGemmError) as e:
        lg.lutgemm_run_noalloc(pw.shape, w.m, pw.d_bits.data_ptr(), pw.d_alpha.data_ptr(), None,
                               x.data_ptr(), y.data_ptr(), sh)
    assert e.value.status == 4
    monkeypatch.delenv("LUTGEMM_TILE")
    torch.cuda.synchronize()
    assert (y == 7.0).all()

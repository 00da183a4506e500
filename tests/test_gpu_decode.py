"""The decode-step driver on the GPU: every product of a short layer stack is
checked against the oracle on the input it actually read, and the captured
token graph reproduces the eager token exactly on every replay."""
import sys

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from lut_gemv_amd.decode import DecodeStack  # noqa: E402

DEV = "cuda:0"


def _say(msg):
    print(f"[gpu-decode] {msg}", flush=True)
    sys.stdout.flush()


def _rows(N, n=96, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.r_[np.arange(16), np.arange(N - 16, N), rng.choice(N, n, replace=False)])


@pytest.fixture(scope="module")
def stack():
    _say("llama7b-shaped stack, 2 layers, q3 g128")
    st = DecodeStack("llama7b", layers=2, q=3, g=128, device=DEV, keep_logical=True)
    yield st
    del st
    torch.cuda.empty_cache()


def test_every_product_matches_oracle(stack):
    """Run the layers one at a time: each product against the oracle on sampled rows."""
    x_layer = stack.x
    for l, lw in enumerate(stack.weights):
        for p in stack.projs:
            src = (x_layer if p.src == "x" else stack.outs[p.src])[:, p.src_off:p.src_off + p.K]
            src = src.contiguous()
            y = lw[p.name](src)
            torch.cuda.synchronize()
            w = stack.logical[(p.N, p.K)]
            rows = _rows(p.N, seed=l)
            ref, bound = oracle.gemv(w.bits, w.alpha, None, src.cpu().numpy(), w.g, rows=rows)
            yg = y.cpu().numpy()[:, rows].astype(np.float64)
            ok, worst = oracle.parity_ok(yg, ref, bound)
            _say(f"layer {l} {p.name} {p.N}x{p.K}: worst err/tol {worst:.3f}")
            assert ok
            stack.outs[p.name].copy_(y)
        x_layer = stack.outs[stack.out_name]
    out = stack.outs[stack.out_name]
    assert torch.isfinite(out).all()
    rms = float(out.float().pow(2).mean().sqrt())
    _say(f"layer output rms {rms:.3f}")
    assert 0.05 < rms < 20.0


@pytest.mark.parametrize("kernel", ["lut", "dequant"])
def test_graph_replays_match_eager(stack, kernel):
    """Replays of the captured token equal the eager token bit for bit, with eager
    work and synchronisations between the replays."""
    eager = stack.token(kernel).clone()
    torch.cuda.synchronize()
    g = stack.capture(kernel)
    for r in range(3):
        stack.outs[stack.out_name].fill_(0)
        junk = torch.randn(1 << 16, device=DEV).sum()          # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = stack.outs[stack.out_name]
        assert torch.equal(got, eager), f"replay {r} differs"
        assert torch.isfinite(junk)
    _say(f"{kernel}: 3 replays equal the eager token")

"""Host-side checks of the decode-step driver (no GPU: buffers live on the CPU)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
from lut_gemv_amd import decode  # noqa: E402


def test_weight_bytes_closed_form():
    """Padding-free shapes: 12 d^2 weights per OPT layer at q/8 bytes plus 2q/g
    bytes of scales per weight."""
    d = 12288
    per_weight = 3 / 8 + 2 * 3 / 128
    assert decode.weight_bytes_per_step("opt175b", 3, 128) == int(96 * 12 * d * d * per_weight)
    d, f = 8192, 22016
    assert decode.weight_bytes_per_step("llama65b", 3, 128) == \
        int(80 * (4 * d * d + 3 * d * f) * per_weight)
    d, f = 4096, 11008                                  # 11008 rows pad to 16, inputs to 512
    assert decode.weight_bytes_per_step("llama7b", 3, 128) > int(32 * (4 * d * d + 3 * d * f) * per_weight)


def test_projection_chain_is_well_formed():
    for name, (layers, projs, out) in decode.MODELS.items():
        sizes = {"x": projs[0].K}
        for p in projs:
            assert p.src in sizes, (name, p)
            assert sizes[p.src] >= p.src_off + p.K, (name, p)   # reads K entries from src_off
            sizes[p.name] = p.N
        assert sizes[out] == projs[0].K                 # layer output feeds the next layer


def test_stack_layers_hold_their_own_copies():
    st = decode.DecodeStack("llama7b", layers=2, device="cpu")
    assert st.bytes_per_step() == decode.weight_bytes_per_step("llama7b", 3, 128, 2)
    assert [p.name for p in st.projs] == ["qkv", "out", "gate_up", "down"]
    a, b = st.weights[0]["down"], st.weights[1]["down"]
    assert a.d_bits.data_ptr() != b.d_bits.data_ptr()
    assert torch.equal(a.d_bits, b.d_bits) and torch.equal(a.d_alpha, b.d_alpha)
    nbytes = sum(w.d_bits.numel() + 2 * w.d_alpha.numel() for lw in st.weights for w in lw.values())
    assert nbytes == st.bytes_per_step()
    # scales keep one product's gain near one: sigma = 1/sqrt(q K)
    al = a.d_alpha.view(torch.float16).float().numpy()
    rms = float(np.sqrt((al[al != 0] ** 2).mean()))
    assert rms == pytest.approx(1 / np.sqrt(3 * 11008), rel=0.05)


def test_unknown_model_and_bad_layers():
    with pytest.raises(ValueError):
        decode.DecodeStack("gpt5", device="cpu")
    with pytest.raises(ValueError):
        decode.DecodeStack("llama7b", layers=0, device="cpu")


def test_packed_call_checks_arguments():
    """The binding rejects x or out of the wrong type, shape or device before any launch."""
    import lut_gemv_amd as lg
    import workloads
    w = workloads.random_bcq(32, 512, 2, 128, seed=1)
    pw = lg.PackedBCQ.from_bcq(w.bits, w.alpha, None, w.g, device="cpu")
    good = torch.zeros((2, 512), dtype=torch.float16)
    for bad in (torch.zeros((2, 512), dtype=torch.float32), torch.zeros((2, 256), dtype=torch.float16),
                torch.zeros(512, dtype=torch.float16)):
        with pytest.raises(ValueError):
            pw(bad)
    with pytest.raises(ValueError):
        pw(good, out=torch.empty((2, 31), dtype=torch.float16))
    with pytest.raises(ValueError):
        pw.dequant(good, out=torch.empty((2, 32), dtype=torch.float32))

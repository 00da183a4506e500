"""Pins of the fp64 oracle against facts fixed outside it.

Each test checks an oracle function against something it does not compute
itself: a worked example printed on (or derived by hand from) the pages, a
closed form, an exhaustive enumeration, integer arithmetic, or the definition
of uniform quantization. ``test_planted_mistakes`` plants plausible bugs in a
copy of the oracle and checks that these pins catch each of them.
"""

import numpy as np
import pytest

import oracle
from oracle import bcq as ob
from conftest import load_golden

# ---------------------------------------------------------------- helpers

def _encode_signs(sign_matrix):
    """+-1 matrix [..., K] -> sign bytes [..., K/8], written element by element.

    Encoding is done with explicit integer bit arithmetic (bit k%8 of byte k//8),
    independent of numpy's packbits/unpackbits used inside the oracle.
    """
    s = np.asarray(sign_matrix)
    K = s.shape[-1]
    out = np.zeros(s.shape[:-1] + (K // 8,), np.uint8)
    it = np.nditer(s[..., 0], flags=["multi_index"])
    for _ in it:
        lead = it.multi_index
        for k in range(K):
            if s[lead + (k,)] > 0:
                out[lead + (k // 8,)] |= np.uint8(1 << (k % 8))
    return out


def _int_bcq_problem(rng, N, K, q, g, m, with_offset):
    """A BCQ matrix whose weights are integers known independently of the oracle.

    Plane scales are alpha_i = 2^i * gamma[j, grp] with integer gamma, so each
    weight equals gamma * odd + delta where odd is the odd integer whose binary
    digits (shifted) are the sign bits. Returns the pieces and the integer W.
    """
    G = K // g
    odd = rng.integers(0, 1 << q, size=(N, K)) * 2 - ((1 << q) - 1)     # odd ints in [-(2^q-1), 2^q-1]
    digits = (odd + (1 << q) - 1) // 2                                    # in [0, 2^q)
    gamma = rng.integers(-3, 4, size=(N, G))
    delta = rng.integers(-5, 6, size=(N, G)) if with_offset else np.zeros((N, G), np.int64)
    W = np.repeat(gamma, g, axis=1) * odd + np.repeat(delta, g, axis=1)
    planes = np.stack([np.where((digits >> i) & 1, 1, -1) for i in range(q)])
    bits = _encode_signs(planes)
    alpha = np.stack([(gamma * (1 << i)) for i in range(q)]).astype(np.float16)
    offset = delta.astype(np.float16) if with_offset else None
    x = rng.integers(-8, 9, size=(m, K))
    return bits, alpha, offset, x.astype(np.float16), W, x


# ---------------------------------------------------------------- golden

def test_sign_order_golden():
    fx = load_golden("sign_order_example.json")
    for case in fx["cases"]:
        bits = np.array(case["bits"], np.uint8)
        alpha = np.array(case["alpha"], np.float16)
        off = np.array(case["offset"], np.float16) if "offset" in case else None
        x = np.array(case["x"], np.float16)[None, :]
        s = ob.signs(bits)
        assert np.array_equal(s.reshape(len(case["signs"]), -1), np.array(case["signs"]))
        y, bound = ob.gemv(bits, alpha, off, x, case["g"])
        assert y.shape == (1, 1)
        assert y[0, 0] == case["y"]
        assert ob.gemv_lut(bits, alpha, off, x, case["g"])[0, 0] == case["y"]


def test_lut_entries_golden():
    fx = load_golden("lut_entries_example.json")
    t = ob.lut_table(fx["x"])
    for p, v in fx["entries"].items():
        assert t[int(p)] == v


def test_uniform_rewrite_golden():
    fx = load_golden("uniform_rewrite_example.json")
    codes = np.array(fx["codes"], np.uint8)
    scale = np.array(fx["scale"], np.float16)
    zero = np.array(fx["zero"], np.uint8)
    bits, alpha, off, n_r = ob.uniform_to_bcq(codes, scale, zero, fx["q"], fx["g"])
    assert n_r == 0
    assert np.array_equal(alpha.astype(np.float64), np.array(fx["alpha"]))
    assert np.array_equal(off.astype(np.float64), np.array(fx["offset"]))
    assert np.array_equal(ob.signs(bits)[:, :, :4], np.array(fx["plane_signs"]))
    # pad K to 8 is not needed for the decode check above; rebuild with K=8
    w = ob.dequant_uniform(codes, scale, zero, fx["g"])
    assert np.array_equal(w, np.array(fx["weights"]))


def test_footprint_golden():
    fx = load_golden("footprint_example.json")
    for c in fx["cases"]:
        assert ob.footprint_bits(c["n"], c["q"], c["g"], c["offset"]) == c["bits"]
    # the page's point: the lower bit width costs more storage here
    a, b = fx["cases"]
    assert a["q"] < b["q"] and ob.footprint_bits(a["n"], a["q"], a["g"]) > ob.footprint_bits(b["n"], b["q"], b["g"])


def test_opt175b_size_consistency():
    fx = load_golden("opt175b_size.json")
    K, q = fx["K"], fx["q"]
    n = 10 ** 6 * K        # any multiple of K; the ratio is per weight
    ratio = 16 * n / ob.footprint_bits(n, q, K)
    assert round(ratio, 2) == fx["ratio"]
    assert round(fx["fp16_gb"] / ratio, 1) == fx["q3_gb"]
    # group size 128 would not reproduce the page's figure
    assert round(16 * n / ob.footprint_bits(n, q, 128), 2) != fx["ratio"]


# ---------------------------------------------------------------- tables

@pytest.mark.parametrize("seed", range(4))
def test_lut_closed_forms(seed):
    rng = np.random.default_rng(seed)
    x = rng.integers(-1000, 1001, size=8).astype(np.float64)   # exact in fp64
    t = ob.lut_table(x)
    total = x.sum()
    for p in range(256):
        chosen = sum(x[k] for k in range(8) if (p >> k) & 1)
        assert t[p] == 2 * chosen - total            # closed form
        assert t[p ^ 0xFF] == -t[p]                  # complement symmetry
    assert t[0xFF] == total and t[0] == -total
    for k in range(8):
        assert t[1 << k] == 2 * x[k] - total


# ---------------------------------------------------------------- brute force

def test_bruteforce_all_patterns_q2():
    """N=1, K=8, q=2: all 2^16 sign patterns (one per row) against integer sums."""
    x = np.array([3, -1, 4, 1, -5, 9, 2, -6], np.float16)
    xi = [3, -1, 4, 1, -5, 9, 2, -6]
    pats = [(a, b) for a in range(256) for b in range(256)]
    bits = np.array([[[a] for a, _ in pats], [[b] for _, b in pats]], np.uint8)   # [2][65536][1]
    alpha = np.ones((2, len(pats), 1), np.float16)
    alpha[1] = 2.0
    w = ob.reconstruct_rows(bits, alpha, None, 8, np.arange(len(pats)))
    y, _ = ob.gemv(bits, alpha, None, x[None], 8, block=4096)
    for r, (a, b) in enumerate(pats):
        expect = [(1 if (a >> k) & 1 else -1) + 2 * (1 if (b >> k) & 1 else -1) for k in range(8)]
        assert w[r].tolist() == expect
        assert y[0, r] == sum(e * v for e, v in zip(expect, xi))
    sub = np.arange(0, len(pats), 257)
    y_lut = ob.gemv_lut(bits[:, sub], alpha[:, sub], None, x[None], 8)
    assert np.array_equal(y_lut[0], y[0, sub])


@pytest.mark.parametrize("N,K,q,g,m,off", [
    (3, 16, 1, 8, 1, False),
    (4, 32, 2, 16, 2, True),
    (5, 64, 3, 32, 1, True),
    (2, 24, 4, 24, 3, False),
    (7, 40, 8, 8, 1, True),
])
def test_integer_weights_exact(N, K, q, g, m, off):
    rng = np.random.default_rng(N * 100 + K + q)
    bits, alpha, offset, x16, W, xi = _int_bcq_problem(rng, N, K, q, g, m, off)
    w = ob.reconstruct_rows(bits, alpha, offset, g, np.arange(N))
    assert np.array_equal(w, W.astype(np.float64))
    y, bound = ob.gemv(bits, alpha, offset, x16, g)
    assert np.array_equal(y, (xi @ W.T).astype(np.float64))
    assert np.array_equal(bound, (np.abs(xi) @ np.abs(W).T).astype(np.float64))
    assert np.array_equal(ob.gemv_lut(bits, alpha, offset, x16, g), y)


def test_gemv_rows_and_blocks():
    rng = np.random.default_rng(7)
    bits, alpha, offset, x16, W, xi = _int_bcq_problem(rng, 37, 64, 3, 16, 2, True)
    y_all, _ = ob.gemv(bits, alpha, offset, x16, 16, block=5)
    rows = np.array([36, 0, 17, 5])
    y_sel, _ = ob.gemv(bits, alpha, offset, x16, 16, rows=rows, block=3)
    assert np.array_equal(y_sel, y_all[:, rows])
    assert np.array_equal(y_all, (xi @ W.T).astype(np.float64))


def test_unit_vector_probes_and_zero():
    rng = np.random.default_rng(11)
    q, N, K, g = 3, 6, 32, 16
    bits = rng.integers(0, 256, size=(q, N, K // 8), dtype=np.uint8)
    alpha = (np.abs(rng.standard_normal((q, N, K // g))) * 0.02).astype(np.float16)
    w = ob.reconstruct_rows(bits, alpha, None, g, np.arange(N))
    for k in range(K):
        e = np.zeros((1, K), np.float16)
        e[0, k] = 1
        y, _ = ob.gemv(bits, alpha, None, e, g)
        # column k: sum_i alpha * sign, the sign read straight from the byte
        col = np.array([sum(float(alpha[i, j, k // g]) * (1 if (int(bits[i, j, k // 8]) >> (k % 8)) & 1 else -1)
                            for i in range(q)) for j in range(N)])
        assert np.array_equal(y[0], col)
        assert np.array_equal(w[:, k], col)
    y0, b0 = ob.gemv(bits, alpha, None, np.zeros((1, K), np.float16), g)
    assert not y0.any() and not b0.any()


def test_random_lut_vs_direct():
    rng = np.random.default_rng(5)
    for (N, K, q, g, m, off) in [(5, 64, 3, 32, 2, True), (3, 128, 2, 128, 1, False)]:
        bits = rng.integers(0, 256, size=(q, N, K // 8), dtype=np.uint8)
        alpha = (np.abs(rng.standard_normal((q, N, K // g))) * 0.02).astype(np.float16)
        offset = (rng.standard_normal((N, K // g)) * 0.02).astype(np.float16) if off else None
        x = rng.standard_normal((m, K)).astype(np.float16)
        y, bound = ob.gemv(bits, alpha, offset, x, g)
        y2 = ob.gemv_lut(bits, alpha, offset, x, g)
        assert np.allclose(y, y2, rtol=0, atol=1e-12 * (1 + bound.max()))


# ---------------------------------------------------------------- uniform -> BCQ

@pytest.mark.parametrize("q", range(1, 9))
def test_uniform_rewrite_exhaustive(q):
    """Every (code, zero-point) pair at unit scale: the BCQ form equals c - z exactly."""
    n = 1 << q
    codes = np.repeat(np.arange(n, dtype=np.uint8)[None, :], n, axis=0)      # [z][c]
    Kp = -(-n // 8) * 8
    codes_p = np.zeros((n, Kp), np.uint8)
    codes_p[:, :n] = codes
    g = Kp
    scale = np.ones((n, 1), np.float16)
    zero = np.arange(n, dtype=np.uint8)[:, None]
    bits, alpha, off, n_r = ob.uniform_to_bcq(codes_p, scale, zero, q, g)
    assert n_r == 0
    w = ob.reconstruct_rows(bits, alpha, off, g, np.arange(n))
    expect = codes_p.astype(np.int64) - np.arange(n)[:, None]
    assert np.array_equal(w, expect.astype(np.float64))


def _count_inexact_half(scale16, q, zero):
    """Groups whose rewritten values cannot all be fp16, counted from bit patterns.

    For q=4, z=8 the rewrite needs s/2 (alpha_0 and -offset) besides s, 2s, 4s.
    s/2 is an fp16 value unless s < 2^-13 and s is an odd multiple of 2^-24.
    """
    assert q == 4 and zero == 8
    u = scale16.view(np.uint16).astype(np.int64) & 0x7FFF
    exp_field = u >> 10
    small = exp_field == 0                       # subnormal: s = mant * 2^-24
    odd = (u & 1) == 1
    return int(np.count_nonzero(small & odd))


def test_uniform_rewrite_int4_scales():
    rng = np.random.default_rng(3)
    N, K, g = 64, 256, 128
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    scale = (np.abs(rng.standard_normal((N, K // g))) * 0.01).astype(np.float16)
    # force a few tiny odd subnormal scales, and a zero scale
    scale.view(np.uint16)[:4, 0] = [1, 3, 0x03FF, 2]
    scale[5, 1] = 0
    zero = np.full((N, K // g), 8, np.uint8)
    bits, alpha, off, n_r = ob.uniform_to_bcq(codes, scale, zero, 4, g)
    assert n_r == _count_inexact_half(scale, 4, 8)
    w_bcq = ob.reconstruct_rows(bits, alpha, off, g, np.arange(N))
    w_def = ob.dequant_uniform(codes, scale, zero, g)
    s_u = scale.view(np.uint16).astype(np.int64)
    exact_grp = ~(((s_u & 0x7C00) == 0) & ((s_u & 1) == 1))
    exact_el = np.repeat(exact_grp, g, axis=1)
    assert np.array_equal(w_bcq[exact_el], w_def[exact_el])
    # rounded groups: each of alpha_0 and offset is off by at most half a subnormal step
    assert np.all(np.abs(w_bcq - w_def)[~exact_el] <= 2.0 ** -24)


def test_uniform_rewrite_rejects():
    codes = np.zeros((1, 8), np.uint8)
    with pytest.raises(ValueError):
        ob.uniform_to_bcq(codes + 16, np.ones((1, 1), np.float16), np.zeros((1, 1), np.uint8), 4, 8)
    with pytest.raises(ValueError):
        ob.uniform_to_bcq(codes, np.ones((1, 1), np.float16), np.full((1, 1), 16, np.uint8), 4, 8)
    with pytest.raises(ValueError):
        ob.uniform_to_bcq(codes, np.full((1, 1), np.inf, np.float16), np.zeros((1, 1), np.uint8), 4, 8)
    with pytest.raises(ValueError):   # 4 * 60000 overflows fp16
        ob.uniform_to_bcq(codes, np.full((1, 1), 60000, np.float16), np.zeros((1, 1), np.uint8), 4, 8)


# ---------------------------------------------------------------- packed layout

def _unpack_by_loops(pb, pa, po, q, N, K, g):
    """Inverse of the packed layout, byte by byte from its definition (independent
    of the reshapes inside the oracle's packer). Returns the logical arrays over
    the padded extent."""
    RT = -(-N // 16)
    C = K // 8
    KT = -(-C // 64)
    G = K // g
    b = np.zeros((q, RT * 16, KT * 64), np.uint8)
    for rt in range(RT):
        for kt in range(KT):
            for i in range(q):
                base = ((kt * RT + rt) * q + i) * 1024
                for lane in range(64):
                    r4, c4 = lane // 16, lane % 16
                    for a in range(4):
                        for bb in range(4):
                            b[i, 16 * rt + 4 * r4 + a, 64 * kt + 4 * c4 + bb] = pb[base + lane * 16 + 4 * a + bb]
    a_out = np.zeros((q, RT * 16, G), np.uint16)
    o_out = np.zeros((RT * 16, G), np.uint16) if po.size else None
    for rt in range(RT):
        for grp in range(G):
            for i in range(q):
                for r in range(16):
                    a_out[i, 16 * rt + r, grp] = pa[((rt * G + grp) * q + i) * 16 + r]
            if o_out is not None:
                for r in range(16):
                    o_out[16 * rt + r, grp] = po[(rt * G + grp) * 16 + r]
    return b, a_out, o_out


@pytest.mark.parametrize("N,K,q,g,off", [(17, 520, 3, 8, True), (16, 512, 1, 512, False),
                                         (40, 1024, 4, 128, True), (1, 8, 2, 8, False)])
def test_pack_roundtrip(N, K, q, g, off):
    rng = np.random.default_rng(N + K)
    bits = rng.integers(0, 256, size=(q, N, K // 8), dtype=np.uint8)
    alpha = rng.standard_normal((q, N, K // g)).astype(np.float16)
    offset = rng.standard_normal((N, K // g)).astype(np.float16) if off else None
    pb, pa, po = ob.pack(bits, alpha, offset, g)
    nb, na, no = ob.packed_sizes(N, K, q, g, off)
    assert pb.size == nb and pa.size == na and po.size == no
    b_full, a_full, o_full = _unpack_by_loops(pb, pa, po, q, N, K, g)
    assert np.array_equal(b_full[:, :N, :K // 8], bits)
    assert np.array_equal(a_full[:, :N, :], alpha.view(np.uint16))
    # padding is zero
    assert not b_full[:, N:, :].any() and not b_full[:, :, K // 8:].any()
    assert not a_full[:, N:, :].any()
    if off:
        assert np.array_equal(o_full[:N], offset.view(np.uint16))
        assert not o_full[N:].any()


def test_pack_single_bit_positions():
    """Hand-placed bytes land where the layout definition says: block
    ((kt*RT + rt)*q + i)*1024, lane block 16*(16*r4 + c4), byte 4*a + b for
    row 16 rt + 4 r4 + a and chunk 64 kt + 4 c4 + b."""
    q, N, K, g = 2, 20, 1024, 256
    bits = np.zeros((q, N, K // 8), np.uint8)
    cases = {
        # (plane, row, chunk): row 17 -> rt 1, r4 0, a 1; chunk 70 -> kt 1, c4 1, b 2
        (1, 17, 70): ((1 * 2 + 1) * 2 + 1) * 1024 + 16 * (16 * 0 + 1) + 4 * 1 + 2,   # kt 1, rt 1
        (0, 0, 0): 0,
        # row 15 -> rt 0, r4 3, a 3; chunk 63 -> kt 0, c4 15, b 3
        (0, 15, 63): 16 * (16 * 3 + 15) + 4 * 3 + 3,
        # row 3 -> r4 0, a 3; chunk 127 -> kt 1, c4 15, b 3
        (1, 3, 127): ((1 * 2 + 0) * 2 + 1) * 1024 + 16 * 15 + 4 * 3 + 3,    # kt 1, rt 0
        # row 6 -> r4 1, a 2; chunk 9 -> kt 0, c4 2, b 1
        (0, 6, 9): 16 * (16 * 1 + 2) + 4 * 2 + 1,
    }
    for n, (i, j, c) in enumerate(cases):
        bits[i, j, c] = n + 1
    alpha = np.zeros((q, N, K // g), np.float16)
    alpha[1, 18, 3] = 1.0          # rt 1, grp 3, plane 1, row 2 -> ((1*4+3)*2+1)*16 + 2
    pb, pa, _ = ob.pack(bits, alpha, None, g)
    for n, (key, idx) in enumerate(cases.items()):
        assert pb[idx] == n + 1, key
    assert np.count_nonzero(pb) == len(cases)
    assert pa[((1 * 4 + 3) * 2 + 1) * 16 + 2] == np.float16(1.0).view(np.uint16)
    assert np.count_nonzero(pa) == 1


# ---------------------------------------------------------------- the checker itself

def test_parity_rule():
    ref = np.array([[1.0, -2.0, 0.0]])
    bound = np.array([[10.0, 10.0, 0.0]])
    ok, worst = ob.parity_ok(ref + np.array([[0.0100, -0.0100, 0.0001]]), ref, bound)
    assert ok and worst <= 1.0
    ok, _ = ob.parity_ok(ref + np.array([[0.0102, 0.0, 0.0]]), ref, bound)
    assert not ok
    ok, _ = ob.parity_ok(ref + np.array([[0.0, 0.0, 0.00011]]), ref, bound)
    assert not ok


# ---------------------------------------------------------------- planted mistakes

# ---------------------------------------------------------------- quantizer

def _balanced_bcq(rng, N, K, q, g, scale):
    """W = sum_i alpha_i b_i where, inside every group, each block of 2^q weights
    holds every sign combination once (in random order) and alpha_i =
    scale * 2^-i. Every pairwise product b_i b_k then averages to zero over the
    group, so the greedy step sees mean |residual| = alpha_i exactly."""
    assert g % (1 << q) == 0
    nc = 1 << q
    planes = np.empty((q, N, K), np.int8)
    for j in range(N):
        for blk in range(K // nc):
            perm = rng.permutation(nc)
            for t, c in enumerate(perm):
                for i in range(q):
                    planes[i, j, blk * nc + t] = 1 if (c >> i) & 1 else -1
    alpha = np.array([scale * 2.0 ** -i for i in range(q)])
    W = sum(alpha[i] * planes[i].astype(np.float64) for i in range(q))
    assert np.array_equal(W.astype(np.float16).astype(np.float64), W)
    return W.astype(np.float16), planes, alpha


@pytest.mark.parametrize("q,g,iters", [(1, 8, 0), (2, 16, 0), (3, 32, 0), (3, 32, 2), (4, 64, 3)])
def test_quantize_recovers_exact_bcq(q, g, iters):
    """A matrix that is exactly BCQ (with distinct combination values) comes back
    exactly: planes in order, bits LSB-first, scales [q][N][K/g], zero error."""
    rng = np.random.default_rng(20 + q)
    N, K = 3, 2 * g
    W, planes, alpha = _balanced_bcq(rng, N, K, q, g, 0.75)
    bits, a, err = ob.quantize_bcq(W, q, g, iters)
    assert err == 0.0
    assert np.array_equal(bits, _encode_signs(planes))
    for i in range(q):
        assert np.all(a[i].astype(np.float64) == alpha[i])


def test_quantize_q1_is_the_fp16_optimum():
    """For one plane, the result's error equals the best over every sign vector
    and, for each, both fp16 neighbours of its least-squares scale (exhaustive
    over 2^8 sign vectors per group)."""
    rng = np.random.default_rng(31)
    g = 8
    combos = np.array([[1.0 if (c >> k) & 1 else -1.0 for k in range(g)] for c in range(1 << g)])
    for trial in range(40):
        w = (rng.standard_normal(g) * rng.choice([1e-3, 0.1, 3.0])).astype(np.float16)
        if trial % 7 == 0:
            w[rng.integers(0, g)] = 0
        wd = w.astype(np.float64)
        best = np.inf
        for b in combos:
            a_ls = float(b @ wd) / g
            h = np.float16(a_ls)
            for cand in (h, np.nextafter(h, np.float16(np.inf)), np.nextafter(h, np.float16(-np.inf))):
                e = float(((wd - float(cand) * b) ** 2).sum())
                best = min(best, e)
        for iters in (0, 2):
            _, _, err = ob.quantize_bcq(w[None, :], 1, g, iters)
            assert err == pytest.approx(best, rel=1e-12, abs=1e-30)


def test_quantize_q2_lower_bound_and_refinement():
    """Two planes, groups of 8: no result beats the continuous optimum (found by
    trying all 2^16 plane pairs with least-squares scales), and the alternating
    rounds lower the total error against the greedy start."""
    rng = np.random.default_rng(32)
    g = 8
    c = np.array([[1.0 if (v >> k) & 1 else -1.0 for k in range(g)] for v in range(1 << g)])
    B0 = np.repeat(c, len(c), axis=0)
    B1 = np.tile(c, (len(c), 1))
    tot0 = tot3 = 0.0
    for _ in range(12):
        w = (rng.standard_normal(g) * 0.05).astype(np.float16)
        wd = w.astype(np.float64)
        # least squares per pair: [[g, d], [d, g]] a = [B0 w, B1 w]
        d = (B0 * B1).sum(axis=1)
        v0, v1 = B0 @ wd, B1 @ wd
        det = g * g - d * d
        ok = det > 0
        a0 = np.where(ok, (g * v0 - d * v1) / np.where(ok, det, 1), v0 / g)
        a1 = np.where(ok, (g * v1 - d * v0) / np.where(ok, det, 1), 0.0)
        e = ((wd[None, :] - a0[:, None] * B0 - a1[:, None] * B1) ** 2).sum(axis=1)
        floor = e.min()
        _, _, e0 = ob.quantize_bcq(w[None, :], 2, g, 0)
        _, _, e3 = ob.quantize_bcq(w[None, :], 2, g, 3)
        assert e0 >= floor * (1 - 1e-9) - 1e-18
        assert e3 >= floor * (1 - 1e-9) - 1e-18
        tot0 += e0
        tot3 += e3
    assert tot3 < tot0


def test_quantize_error_is_the_reconstruction_error():
    """The returned error is the squared distance between W and the returned
    planes and scales (decoded here with explicit bit arithmetic)."""
    rng = np.random.default_rng(33)
    N, K, q, g = 4, 64, 3, 16
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    bits, a, err = ob.quantize_bcq(w, q, g, 2)
    rec = np.zeros((N, K))
    for i in range(q):
        for j in range(N):
            for k in range(K):
                s = 1.0 if (int(bits[i, j, k // 8]) >> (k % 8)) & 1 else -1.0
                rec[j, k] += float(a[i, j, k // g]) * s
    assert err == pytest.approx(float(((w.astype(np.float64) - rec) ** 2).sum()), rel=1e-12)


def _run_pins():
    """The pins above, as a callable that raises AssertionError on any failure."""
    test_sign_order_golden()
    test_lut_entries_golden()
    test_uniform_rewrite_golden()
    test_footprint_golden()
    test_integer_weights_exact(5, 64, 3, 32, 1, True)
    test_integer_weights_exact(7, 40, 8, 8, 1, True)
    test_unit_vector_probes_and_zero()
    test_uniform_rewrite_exhaustive(4)
    test_pack_roundtrip(17, 520, 3, 8, True)
    test_pack_single_bit_positions()
    test_quantize_recovers_exact_bcq(3, 32, 0)
    test_quantize_recovers_exact_bcq(3, 32, 2)
    test_quantize_q1_is_the_fp16_optimum()
    test_quantize_q2_lower_bound_and_refinement()
    test_quantize_error_is_the_reconstruction_error()


def _mut_signs_msb_first(bits):
    b01 = np.unpackbits(np.asarray(bits, dtype=np.uint8), axis=-1, bitorder="big")
    return (b01.astype(np.int8) * 2 - 1).astype(np.int8)


def _mut_signs_flipped(bits):
    b01 = np.unpackbits(np.asarray(bits, dtype=np.uint8), axis=-1, bitorder="little")
    return (1 - b01.astype(np.int8) * 2).astype(np.int8)


_orig_reconstruct = ob.reconstruct_rows


def _mut_reconstruct_drop_offset(bits, alpha, offset, g, rows):
    return _orig_reconstruct(bits, alpha, None, g, rows)


def _mut_reconstruct_group_modulo(bits, alpha, offset, g, rows):
    # wrong group index: k % G instead of k // g
    q = bits.shape[0]
    b = ob.signs(bits[:, rows, :]).astype(np.float64)
    K = b.shape[-1]
    G = alpha.shape[-1]
    a = alpha[:, rows, :].astype(np.float64)
    a_full = np.tile(a, (1, 1, K // G))
    w = sum(a_full[i] * b[i] for i in range(q))
    if offset is not None:
        w = w + np.tile(offset[rows, :].astype(np.float64), (1, K // G))
    return w


def _mut_reconstruct_last_plane_dropped(bits, alpha, offset, g, rows):
    return _orig_reconstruct(bits[:-1], alpha[:-1], offset, g, rows) if bits.shape[0] > 1 else \
        _orig_reconstruct(bits, alpha * 0, offset, g, rows)


_orig_lut = ob.lut_table


def _mut_lut_wrong_sign(xc):
    return -_orig_lut(xc)


_orig_u2b = ob.uniform_to_bcq


def _mut_u2b_offset_sign(codes, scale, zero, q, g):
    bits, a, o, n = _orig_u2b(codes, scale, zero, q, g)
    return bits, a, (-o.astype(np.float64)).astype(np.float16), n


def _mut_u2b_alpha_scale(codes, scale, zero, q, g):
    bits, a, o, n = _orig_u2b(codes, scale, zero, q, g)
    return bits, (a.astype(np.float64) * 2).astype(np.float16), o, n


def _mut_footprint_no_scales(n, q, g, offset=False):
    return q * n


_orig_pack = ob.pack


def _mut_pack_rows_chunks_swapped(bits, alpha, offset, g):
    pb, pa, po = _orig_pack(bits, alpha, offset, g)
    q, N, C = bits.shape
    RT, KT = -(-N // 16), -(-C // 64)
    pb = pb.reshape(RT, KT, q, 4, 16, 4, 4).transpose(0, 1, 2, 3, 4, 6, 5).reshape(-1).copy()
    return pb, pa, po


_orig_quant = ob.quantize_bcq


def _mut_quant_planes_reversed(w, q, g, iters=0):
    bits, a, e = _orig_quant(w, q, g, iters)
    return bits[::-1].copy(), a[::-1].copy(), e


def _mut_quant_alpha_one_ulp(w, q, g, iters=0):
    bits, a, e = _orig_quant(w, q, g, iters)
    a2 = np.nextafter(a, np.float16(np.inf))
    rec = (np.stack([ob.signs(bits[i]) for i in range(q)]).astype(np.float64)
           * np.repeat(a2.astype(np.float64), g, axis=2)).sum(axis=0)
    return bits, a2, float(((np.asarray(w, np.float64) - rec) ** 2).sum())


def _mut_quant_bits_msb_first(w, q, g, iters=0):
    bits, a, e = _orig_quant(w, q, g, iters)
    return np.packbits(np.unpackbits(bits, axis=-1, bitorder="little"), axis=-1, bitorder="big"), a, e


def _mut_quant_error_first_group_only(w, q, g, iters=0):
    bits, a, e = _orig_quant(w, q, g, iters)
    _, _, e1 = _orig_quant(np.asarray(w)[:, :g], q, g, iters)
    return bits, a, e1


@pytest.mark.parametrize("name,mutant", [
    ("quantize_bcq", _mut_quant_planes_reversed),
    ("quantize_bcq", _mut_quant_alpha_one_ulp),
    ("quantize_bcq", _mut_quant_bits_msb_first),
    ("quantize_bcq", _mut_quant_error_first_group_only),
    ("signs", _mut_signs_msb_first),
    ("signs", _mut_signs_flipped),
    ("reconstruct_rows", _mut_reconstruct_drop_offset),
    ("reconstruct_rows", _mut_reconstruct_group_modulo),
    ("reconstruct_rows", _mut_reconstruct_last_plane_dropped),
    ("lut_table", _mut_lut_wrong_sign),
    ("uniform_to_bcq", _mut_u2b_offset_sign),
    ("uniform_to_bcq", _mut_u2b_alpha_scale),
    ("footprint_bits", _mut_footprint_no_scales),
    ("pack", _mut_pack_rows_chunks_swapped),
])
def test_planted_mistakes(monkeypatch, name, mutant):
    monkeypatch.setattr(ob, name, mutant)
    with pytest.raises(AssertionError):
        _run_pins()


def test_group_search_golden():
    """The oracle's (q, g) search against hand-worked cases (bits per weight)."""
    fx = load_golden("group_search_example.json")
    for c in fx["cases"]:
        got = ob.search_group_sizes(c["N"], c["K"], c["bpw"], c["offset"])
        want = {int(q): (g, bpw) for q, (g, bpw) in c["expect"].items()}
        assert sorted(got) == sorted(want)
        for q, (g, bpw) in want.items():
            assert got[q][0] == g
            assert got[q][1] == bpw * c["N"] * c["K"]

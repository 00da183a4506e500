"""fp64 reference for the binary-coding-quantization (BCQ) matrix-vector product.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the product
path may import this module.

What the method computes (LUT-GEMM, Park et al.; Elamur card "LUT-GEMM -- paper
by Park et al. (2022)", sections "Summary" and "Interesting ideas: Lookup tables
instead of multiplications"; pith.science page of the same title, original
abstract): a weight matrix stored as q binary (+-1) planes with scales,
multiplied directly with fp16 activations. The result the method reaches is, up
to rounding order, the plain product of the reconstructed weight matrix with x,
so :func:`gemv` is that definition written out in fp64 (reconstruct, then a
direct dot product). The lookup-table route is kept as a second, independent
function (:func:`gemv_lut`) whose agreement with :func:`gemv` checks the
method's algebra.

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):

* sign convention: a set bit is +1, a clear bit is -1; bits are taken least
  significant first along the input dimension (byte ``c`` holds inputs
  ``8c .. 8c+7``);
* group-wise scales: one fp16 scale per (plane, output row, group of ``g``
  consecutive inputs) (card section "Interesting ideas: Group size as a
  separate hyper-parameter");
* offset: an optional fp16 per (output row, group), added to the weight; it is
  what makes a uniform int-q matrix an exact BCQ matrix (card section
  "Interesting ideas: One format for many schemes");
* uniform -> BCQ rewrite: with ``c = sum_i 2^i beta_i`` (``beta_i`` the bits of
  the code) and ``b_i = 2 beta_i - 1``,
  ``s (c - z) = sum_i (s 2^(i-1)) b_i + s ((2^q - 1)/2 - z)``;
* the packed device layout (:func:`pack`) is this project's own format, not the
  pages'; the oracle re-implements its index function independently.

Pins (tests/test_oracle_*.py): brute-force enumeration on tiny shapes, the
closed forms of the table entries, hand-worked examples under tests/golden/,
special cases that reduce to integer arithmetic, the uniform-quantization
definition, and the pages' storage example (864 vs 640 bits). Every function
below has at least one such pin; none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "signs",
    "reconstruct_rows",
    "gemv",
    "lut_table",
    "gemv_lut",
    "dequant_uniform",
    "uniform_to_bcq",
    "pack",
    "packed_sizes",
    "footprint_bits",
    "parity_ok",
    "ROW_TILE",
    "CHUNK_TILE",
    "search_group_sizes",
    "quantize_bcq",
]

# Packed-layout tile sizes of this project's device format (see :func:`pack`).
ROW_TILE = 16      # output rows per row tile
CHUNK_TILE = 64    # 8-input chunks per input tile (512 inputs)


# --------------------------------------------------------------------------
# BCQ definition
# --------------------------------------------------------------------------

def signs(bits: np.ndarray) -> np.ndarray:
    """Sign planes b_i in {-1, +1} from the sign bytes.

    ``bits`` uint8 [..., K/8] -> int8 [..., K]: bit t (least significant first)
    of byte c is the sign of input 8c + t; 1 -> +1, 0 -> -1.
    (Card "Summary": weights are binary patterns with scales.)
    """
    b01 = np.unpackbits(np.asarray(bits, dtype=np.uint8), axis=-1, bitorder="little")
    return (b01.astype(np.int8) * 2 - 1).astype(np.int8)


def reconstruct_rows(bits, alpha, offset, g: int, rows) -> np.ndarray:
    """W_hat[j, k] = sum_i alpha[i, j, k//g] * b_i[j, k] (+ offset[j, k//g]), fp64.

    ``rows`` selects the output rows (an index array or slice). The sum over
    planes is exact in fp64 for fp16 scales (a handful of terms whose exponents
    span far fewer than 53 binades).
    """
    q = bits.shape[0]
    b = signs(bits[:, rows, :]).astype(np.float64)          # [q][r][K]
    K = b.shape[-1]
    if K == 0:
        return np.zeros(b.shape[1:], np.float64)
    a = alpha[:, rows, :].astype(np.float64)                 # [q][r][G]
    a_full = np.repeat(a, g, axis=-1)                        # [q][r][K]
    w = np.zeros(b.shape[1:], np.float64)
    for i in range(q):
        w += a_full[i] * b[i]
    if offset is not None:
        w += np.repeat(offset[rows, :].astype(np.float64), g, axis=-1)
    return w


def gemv(bits, alpha, offset, x, g: int, rows=None, block: int = 256):
    """Direct fp64 product y = W_hat x, plus the error scale sum_k |W_hat x|.

    Returns ``(y, bound)``, both fp64 [m][len(rows)] (all rows when ``rows`` is
    None). Rows are reconstructed in blocks so a large matrix is never
    materialised whole.
    """
    N = bits.shape[1]
    idx = np.arange(N) if rows is None else np.asarray(rows)
    xf = np.asarray(x, dtype=np.float64)
    if xf.ndim == 1:
        xf = xf[None, :]
    m = xf.shape[0]
    y = np.zeros((m, idx.size), np.float64)
    bound = np.zeros((m, idx.size), np.float64)
    for s in range(0, idx.size, block):
        sel = idx[s:s + block]
        w = reconstruct_rows(bits, alpha, offset, g, sel)      # [r][K]
        y[:, s:s + block] = xf @ w.T
        bound[:, s:s + block] = np.abs(xf) @ np.abs(w).T
    return y, bound


def parity_ok(y_test, y_ref, bound, rel: float = 1e-3, abs_: float = 1e-4):
    """The acceptance rule |y_test - y_ref| <= rel * bound + abs_, per output.

    Returns ``(ok, worst)`` where ``worst`` is the largest ratio
    |err| / (rel * bound + abs_) (<= 1 means within tolerance).
    """
    err = np.abs(np.asarray(y_test, np.float64) - y_ref)
    lim = rel * bound + abs_
    worst = float(np.max(err / lim)) if err.size else 0.0
    return bool(np.all(err <= lim)), worst


# --------------------------------------------------------------------------
# The lookup-table route (method's algebra, independent of the direct product)
# --------------------------------------------------------------------------

def lut_table(xc) -> np.ndarray:
    """All 256 signed sums of one 8-input chunk, fp64.

    Entry p is the sum over t < 8 of (+x_t if bit t of p is set, else -x_t):
    the partial result a weight byte p would select (card "Interesting ideas:
    Lookup tables instead of multiplications"). Written as the plain double
    loop over patterns and positions.
    """
    xc = [float(v) for v in np.asarray(xc, dtype=np.float64).reshape(8)]
    out = np.empty(256, np.float64)
    for p in range(256):
        s = 0.0
        for t in range(8):
            s += xc[t] if (p >> t) & 1 else -xc[t]
        out[p] = s
    return out


def gemv_lut(bits, alpha, offset, x, g: int) -> np.ndarray:
    """y via tables: for every chunk build the 256 sums once, then for every
    (plane, row, chunk) look the sum up by the weight byte and scale it by the
    group's alpha; the offset term adds offset * (sum of the group's inputs).

    fp64; meant for small shapes (tables are built with :func:`lut_table`).
    """
    q, N, C = bits.shape
    xf = np.asarray(x, dtype=np.float64)
    if xf.ndim == 1:
        xf = xf[None, :]
    m = xf.shape[0]
    y = np.zeros((m, N), np.float64)
    for r in range(m):
        tables = np.stack([lut_table(xf[r, 8 * c:8 * c + 8]) for c in range(C)]) \
            if C else np.zeros((0, 256))
        for i in range(q):
            for j in range(N):
                for c in range(C):
                    y[r, j] += float(alpha[i, j, (8 * c) // g]) * tables[c, bits[i, j, c]]
        if offset is not None:
            G = offset.shape[1]
            for j in range(N):
                for grp in range(G):
                    y[r, j] += float(offset[j, grp]) * float(np.sum(xf[r, grp * g:(grp + 1) * g]))
    return y


# --------------------------------------------------------------------------
# Uniform quantization and its BCQ rewrite
# --------------------------------------------------------------------------

def dequant_uniform(codes, scale, zero, g: int, rows=None) -> np.ndarray:
    """The uniform int-q matrix by definition: W[j, k] = s[j, k//g] (c[j, k] - z[j, k//g]), fp64."""
    sel = slice(None) if rows is None else rows
    c = np.asarray(codes[sel], dtype=np.float64)
    s = np.repeat(np.asarray(scale[sel], dtype=np.float64), g, axis=-1)
    z = np.repeat(np.asarray(zero[sel], dtype=np.float64), g, axis=-1)
    return s * (c - z)


def uniform_to_bcq(codes, scale, zero, q: int, g: int):
    """Rewrite a uniform int-q matrix as BCQ with q planes plus an offset.

    (Card "Interesting ideas: One format for many schemes"; "Summary": uniform
    quantization can be rewritten as BCQ.) Plane i carries bit i of the code;
    alpha_i = s * 2^(i-1); offset = s * ((2^q - 1)/2 - z). The fp64 values are
    rounded to fp16 to nearest-even; ``n_rounded`` counts the groups where any of
    them was not exactly representable. Returns
    ``(bits uint8 [q][N][K/8], alpha fp16 [q][N][K/g], offset fp16 [N][K/g], n_rounded)``.
    Raises ValueError on codes or zero-points >= 2^q, and on scales that are
    not finite or whose rewritten values overflow fp16.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    N, K = codes.shape
    if np.any(codes >= (1 << q)) or np.any(np.asarray(zero) >= (1 << q)):
        raise ValueError("code or zero-point out of range for q bits")
    s64 = np.asarray(scale, dtype=np.float16).astype(np.float64)   # [N][G]
    if not np.all(np.isfinite(s64)):
        raise ValueError("non-finite scale")
    z64 = np.asarray(zero, dtype=np.float64)
    # plane i <- bit i of the code
    planes = np.stack([((codes >> i) & 1).astype(np.uint8) for i in range(q)])  # [q][N][K]
    bits = np.packbits(planes, axis=-1, bitorder="little")                     # [q][N][K/8]
    a_exact = np.stack([s64 * (2.0 ** (i - 1)) for i in range(q)])              # [q][N][G]
    o_exact = s64 * ((2.0 ** q - 1.0) / 2.0 - z64)                              # [N][G]
    with np.errstate(over="ignore"):
        a16 = a_exact.astype(np.float16)
        o16 = o_exact.astype(np.float16)
    if not (np.all(np.isfinite(a16)) and np.all(np.isfinite(o16))):
        raise ValueError("rewritten scale overflows fp16")
    rounded = np.any(a16.astype(np.float64) != a_exact, axis=0) | (o16.astype(np.float64) != o_exact)
    return bits, a16, o16, int(np.count_nonzero(rounded))


# --------------------------------------------------------------------------
# Storage accounting and the device format
# --------------------------------------------------------------------------

def footprint_bits(n: int, q: int, g: int, offset: bool = False) -> int:
    """Storage in bits of n weights: q sign bits each, plus one fp16 scale per
    plane per group of g (and one fp16 offset per group when present). The
    scales are counted in, as the card's storage example ("Interesting ideas:
    Group size as a separate hyper-parameter") asks."""
    groups = -(-n // g)
    return q * n + 16 * q * groups + (16 * groups if offset else 0)


def quantize_bcq(w, q: int, g: int, iters: int = 0):
    """Binary-coding quantization of an fp16 matrix, step by step (the pages name
    the quantizer only by reference; this is the reading the design notes give):

    * greedy, per (row, group of g inputs): for plane i = 0..q-1, alpha_i is the
      mean absolute residual rounded to fp16, b_i is the sign of the residual
      (+1 for zero), and the residual loses alpha_i * b_i;
    * then `iters` rounds of: alpha by least squares for the current planes (the
      normal equations B^T B alpha = B^T w, Gaussian elimination in row order
      without pivoting, each entry rounded to fp16; a pivot <= 1e-9 g or an fp16
      overflow keeps the previous alpha), then every weight takes the sign
      combination whose value is nearest (ties: the lowest combination index, bit
      i of the index set meaning plane i is +1).

    Returns (bits uint8 [q][N][K/8] in the logical packing, alpha fp16
    [q][N][K/g], squared error). fp16 inputs make the sums exact in fp64, so the
    order of summation does not matter here.
    """
    w = np.asarray(w, dtype=np.float16)
    N, K = w.shape
    G = K // g
    B = np.zeros((q, N, K), np.int8)
    A = np.zeros((q, N, G), np.float16)
    err = 0.0
    combos = np.array([[1 if (c >> i) & 1 else -1 for i in range(q)] for c in range(1 << q)],
                      dtype=np.float64)            # [combination][plane]
    for j in range(N):
        for t in range(G):
            wg = w[j, t * g:(t + 1) * g].astype(np.float64)
            b = np.zeros((q, g))
            a16 = np.zeros(q, np.float16)
            r = wg.copy()
            for i in range(q):
                a16[i] = np.float16(np.abs(r).sum() / g)
                b[i] = np.where(r >= 0, 1.0, -1.0)
                r = r - float(a16[i]) * b[i]
            for _ in range(iters):
                M = [[float((b[i] * b[k]).sum()) for k in range(q)] for i in range(q)]
                v = [float((b[i] * wg).sum()) for i in range(q)]
                ok = True
                for c in range(q):
                    piv = M[c][c]
                    if not piv > 1e-9 * g:
                        ok = False
                        break
                    for rr in range(c + 1, q):
                        f = M[rr][c] / piv
                        for cc in range(c, q):
                            M[rr][cc] -= f * M[c][cc]
                        v[rr] -= f * v[c]
                if ok:
                    x = [0.0] * q
                    for c in range(q - 1, -1, -1):
                        acc = v[c]
                        for cc in range(c + 1, q):
                            acc -= M[c][cc] * x[cc]
                        x[c] = acc / M[c][c]
                    with np.errstate(over="ignore"):
                        na = np.array(x, dtype=np.float64).astype(np.float16)
                    if np.isfinite(na).all():
                        a16 = na
                vals = combos @ a16.astype(np.float64)          # value of each combination
                best = np.argmin(np.abs(wg[:, None] - vals[None, :]), axis=1)   # first minimum
                b = combos[best].T
            recon = (a16.astype(np.float64)[:, None] * b).sum(axis=0)
            err += float(((wg - recon) ** 2).sum())
            B[:, j, t * g:(t + 1) * g] = b.astype(np.int8)
            A[:, j, t] = a16
    bits = np.packbits((B > 0).astype(np.uint8), axis=2, bitorder="little")
    return bits, A, err


def search_group_sizes(N: int, K: int, max_bits_per_weight: float, has_offset: bool = False):
    """For each q = 1..8 the finest admissible group size (g a divisor of K and a
    multiple of 8) whose storage, by :func:`footprint_bits`, is within the target
    of bits per weight; {q: (g, bits)}, q absent when no g fits. Plain
    enumeration of every (q, g) pair (card section "Interesting ideas: Group size
    as a separate hyper-parameter": q and g are searched jointly for a target
    compression)."""
    n = N * K
    out = {}
    for q in range(1, 9):
        fits = [(g, footprint_bits(n, q, g, has_offset)) for g in range(8, K + 1, 8)
                if K % g == 0 and footprint_bits(n, q, g, has_offset) <= max_bits_per_weight * n]
        if fits:
            out[q] = min(fits)
    return out


def packed_sizes(N: int, K: int, q: int, g: int, has_offset: bool):
    """(bytes of packed bits, fp16 count of packed alpha, fp16 count of packed offset)."""
    Npad = -(-N // ROW_TILE) * ROW_TILE
    C = K // 8
    Cpad = -(-C // CHUNK_TILE) * CHUNK_TILE
    G = K // g if K else 0
    return q * Npad * Cpad, q * Npad * G, (Npad * G if has_offset else 0)


def pack(bits, alpha, offset, g: int):
    """This project's device layout, re-implemented from its definition.

    * rows are padded to a multiple of 16 (padding: sign bytes 0, scales 0);
      chunks (8 inputs) are padded to a multiple of 64 (padding bytes 0);
    * bits: per (input tile kt, row tile rt, plane i), in that order, a block
      of 1024 bytes made of 64 lane blocks of 16 bytes. Lane block L = 16*r4 +
      c4 covers rows 16 rt + 4 r4 + a and chunks 64 kt + 4 c4 + b (a, b in
      0..3); its byte 4 a + b is ``bits[i][16 rt + 4 r4 + a][64 kt + 4 c4 + b]``;
    * alpha : fp16 ``[rt][grp][i][r]`` = ``alpha[i][16 rt + r][grp]``;
    * offset: fp16 ``[rt][grp][r]`` = ``offset[16 rt + r][grp]``.

    Returns ``(bits uint8 1-D, alpha uint16 1-D, offset uint16 1-D)`` (the last
    one empty when there is no offset). Plain index loops over tiles.
    """
    q, N, C = bits.shape
    G = alpha.shape[2]
    RT = -(-N // ROW_TILE)
    KT = -(-C // CHUNK_TILE)
    out_b = np.zeros((KT, RT, q, 4, 16, 4, 4), np.uint8)    # [kt][rt][i][r4][c4][a][b]
    out_a = np.zeros((RT, G, q, ROW_TILE), np.uint16)
    out_o = np.zeros((RT, G, ROW_TILE), np.uint16)
    a16 = np.asarray(alpha, dtype=np.float16).view(np.uint16)
    for rt in range(RT):
        for kt in range(KT):
            for i in range(q):
                block = np.zeros((ROW_TILE, CHUNK_TILE), np.uint8)      # [row][chunk] of the tile
                r_hi = min(ROW_TILE, N - rt * ROW_TILE)
                c_hi = min(CHUNK_TILE, C - kt * CHUNK_TILE)
                block[:r_hi, :c_hi] = bits[i, rt * ROW_TILE:rt * ROW_TILE + r_hi,
                                           kt * CHUNK_TILE:kt * CHUNK_TILE + c_hi]
                # row 4 r4 + a, chunk 4 c4 + b  ->  [r4][c4][a][b]
                out_b[kt, rt, i] = block.reshape(4, 4, 16, 4).transpose(0, 2, 1, 3)
        r_hi = min(ROW_TILE, N - rt * ROW_TILE)
        rows = slice(rt * ROW_TILE, rt * ROW_TILE + r_hi)
        for grp in range(G):
            for i in range(q):
                out_a[rt, grp, i, :r_hi] = a16[i, rows, grp]
            if offset is not None:
                out_o[rt, grp, :r_hi] = np.asarray(offset, np.float16).view(np.uint16)[rows, grp]
    o_flat = out_o.reshape(-1) if offset is not None else np.zeros(0, np.uint16)
    return out_b.reshape(-1), out_a.reshape(-1), o_flat

"""Seeded synthetic inputs for the BCQ GEMV workloads.

This module only draws random numbers. It holds none of the method's arithmetic:
no sign decoding, no tables, no scaling, no packing. Both the product path
(bench, smoke) and the fp64 checker draw their inputs from here, so the two see
the same arrays.

Logical formats produced here (shared vocabulary of the whole project):

* ``x``      fp16 ``[m][K]`` activations, row-major.
* ``bits``   uint8 ``[q][N][K/8]``: byte ``c`` of row ``j`` in plane ``i`` carries the
  sign bits of weights ``(j, 8c .. 8c+7)``, least-significant bit first; a set bit
  stands for +1, a clear bit for -1.
* ``alpha``  fp16 ``[q][N][K/g]``: one scale per plane, output row and group of ``g``
  consecutive inputs.
* ``codes`` uint8 ``[N][K]``, ``scale`` fp16 ``[N][K/g]``, ``zero`` uint8 ``[N][K/g]``:
  a uniform int-q matrix whose value is ``scale * (code - zero)``.

The workload shapes stand in for the layers the LUT-GEMM pages measure on (an
OPT-175B FFN, a LLaMA-7B MLP, a 12288-wide attention projection, a 28672x8192
sweep); the pages' trained weights and datasets are not used: every value is
drawn from the distributions stated per workload below.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "generate",
    "random_bcq",
    "random_uniform",
]


@dataclass
class Workload:
    """One synthetic problem instance in the logical formats described above."""

    name: str
    N: int
    K: int
    q: int
    g: int
    m: int
    x: np.ndarray                        # fp16 [m][K]
    bits: Optional[np.ndarray] = None    # uint8 [q][N][K/8]   (BCQ workloads)
    alpha: Optional[np.ndarray] = None   # fp16 [q][N][K/g]    (BCQ workloads)
    offset: Optional[np.ndarray] = None  # fp16 [N][K/g]       (optional)
    codes: Optional[np.ndarray] = None   # uint8 [N][K]        (uniform workloads)
    scale: Optional[np.ndarray] = None   # fp16 [N][K/g]
    zero: Optional[np.ndarray] = None    # uint8 [N][K/g]
    meta: dict = field(default_factory=dict)

    @property
    def is_uniform(self) -> bool:
        return self.codes is not None


def _abs_normal_fp16(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    """|N(0, sigma)| drawn in float64, rounded to fp16 (round-to-nearest-even)."""
    return (np.abs(rng.standard_normal(shape)) * sigma).astype(np.float16)


def _normal_fp16(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape).astype(np.float16)


def _student_t_fp16(rng: np.random.Generator, shape, nu: float = 3.0,
                    scale: float = 0.5, clip: float = 60.0) -> np.ndarray:
    """Heavy-tailed activations: Student-t(nu) * scale, clipped to +-clip, fp16."""
    v = rng.standard_t(nu, size=shape) * scale
    return np.clip(v, -clip, clip).astype(np.float16)


def _random_bytes(rng: np.random.Generator, shape) -> np.ndarray:
    """iid uniform bytes: every sign bit is an independent fair +-1 draw."""
    return rng.integers(0, 256, size=shape, dtype=np.uint8)


def random_bcq(N: int, K: int, q: int, g: int, m: int = 1, seed: int = 0,
               sigma: float = 0.02, with_offset: bool = False,
               x_dist: str = "normal", name: str = "random_bcq") -> Workload:
    """A BCQ problem: x, then sign bytes, then |N(0, sigma)| scales (draw order)."""
    if K % 8 or (K and K % g):
        raise ValueError("K must be a multiple of 8 and of g")
    rng = np.random.default_rng(seed)
    if x_dist == "normal":
        x = _normal_fp16(rng, (m, K))
    elif x_dist == "student_t":
        x = _student_t_fp16(rng, (m, K))
    elif x_dist == "zeros":
        x = np.zeros((m, K), np.float16)
    else:
        raise ValueError(f"unknown x_dist {x_dist!r}")
    G = K // g if K else 0
    bits = _random_bytes(rng, (q, N, K // 8))
    alpha = _abs_normal_fp16(rng, (q, N, G), sigma)
    offset = None
    if with_offset:
        offset = (rng.standard_normal((N, G)) * sigma).astype(np.float16)
    return Workload(name=name, N=N, K=K, q=q, g=g, m=m, x=x, bits=bits,
                    alpha=alpha, offset=offset, meta={"seed": seed})


def random_uniform(N: int, K: int, q: int, g: int, m: int = 1, seed: int = 0,
                   sigma: float = 0.01, zero: Optional[int] = None,
                   name: str = "random_uniform") -> Workload:
    """A uniform int-q problem: x, then codes U[0, 2^q), then |N(0, sigma)| scales.

    ``zero`` fixes every zero-point; ``None`` draws them uniformly in [0, 2^q).
    """
    if K % 8 or (K and K % g):
        raise ValueError("K must be a multiple of 8 and of g")
    rng = np.random.default_rng(seed)
    x = _normal_fp16(rng, (m, K))
    G = K // g if K else 0
    codes = rng.integers(0, 1 << q, size=(N, K), dtype=np.uint8)
    scale = _abs_normal_fp16(rng, (N, G), sigma)
    if zero is None:
        zp = rng.integers(0, 1 << q, size=(N, G), dtype=np.uint8)
    else:
        zp = np.full((N, G), zero, dtype=np.uint8)
    return Workload(name=name, N=N, K=K, q=q, g=g, m=m, x=x, codes=codes,
                    scale=scale, zero=zp, meta={"seed": seed})


def _tiny():
    return random_bcq(512, 512, 3, 128, 1, seed=0, name="tiny")


def _opt175b_ffn_up():
    return random_bcq(49152, 12288, 3, 128, 1, seed=1, name="opt175b_ffn_up")


def _opt175b_ffn_up_shard8():
    # one GPU's rows of the FFN-up matrix split by rows over eight GPUs
    return random_bcq(6144, 12288, 3, 128, 1, seed=5, name="opt175b_ffn_up_shard8")


def _llama7b_mlp_int4():
    return random_uniform(11008, 4096, 4, 128, 1, seed=2, zero=8,
                          name="llama7b_mlp_int4")


def _decode(m: int):
    def make():
        rng_w = np.random.default_rng(3)
        N = K = 12288
        q, g = 3, 128
        bits = _random_bytes(rng_w, (q, N, K // 8))
        alpha = _abs_normal_fp16(rng_w, (q, N, K // g), 0.02)
        x = _normal_fp16(np.random.default_rng(30 + m), (m, K))
        return Workload(name=f"decode_m{m}", N=N, K=K, q=q, g=g, m=m, x=x,
                        bits=bits, alpha=alpha, meta={"seed": (3, 30 + m)})
    return make


_SUBBIT_G = (32, 64, 128, 8192)


def _subbit(q: int, g: int):
    def make():
        gi = _SUBBIT_G.index(g)
        N, K = 28672, 8192
        rng_w = np.random.default_rng(400 + 10 * q + gi)
        bits = _random_bytes(rng_w, (q, N, K // 8))
        alpha = _abs_normal_fp16(rng_w, (q, N, K // g), 0.02)
        x = _student_t_fp16(np.random.default_rng(40), (1, K))
        return Workload(name=f"subbit_q{q}_g{g}", N=N, K=K, q=q, g=g, m=1, x=x,
                        bits=bits, alpha=alpha,
                        meta={"seed": (400 + 10 * q + gi, 40)})
    return make


#: name -> (constructor, short description). The shapes and distributions are
#: the five workloads the GEMV is measured on.
WORKLOADS = {
    "tiny": (_tiny, "x[1x512] N(0,1); W 512x512 BCQ q=3 g=128; seed 0"),
    "opt175b_ffn_up": (_opt175b_ffn_up,
                       "x[1x12288] N(0,1); W 49152x12288 BCQ q=3 g=128; seed 1"),
    "opt175b_ffn_up_shard8": (_opt175b_ffn_up_shard8,
                              "x[1x12288] N(0,1); W 6144x12288 BCQ q=3 g=128 (one of eight "
                              "row shards of the FFN-up matrix); seed 5"),
    "llama7b_mlp_int4": (_llama7b_mlp_int4,
                         "x[1x4096]; W 11008x4096 uniform int4, zero 8, g=128 "
                         "-> BCQ q=4 + offset; seed 2"),
}
for _m in (2, 4, 8, 16, 32):
    WORKLOADS[f"decode_m{_m}"] = (
        _decode(_m), f"x[{_m}x12288]; W 12288x12288 BCQ q=3 g=128; seeds 3/{30 + _m}")
for _q in (1, 2, 4):
    for _g in _SUBBIT_G:
        WORKLOADS[f"subbit_q{_q}_g{_g}"] = (
            _subbit(_q, _g),
            f"x[1x8192] Student-t(3)*0.5 clip 60; W 28672x8192 BCQ q={_q} g={_g}")


def generate(name: str) -> Workload:
    """Build the named workload (deterministic: fixed seeds)."""
    try:
        ctor, _ = WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}")
    return ctor()

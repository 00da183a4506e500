"""Decode-step driver: the weight GEMVs of a decoder layer stack, one token at a time.

The pages quote the cost of token generation per token for whole models held
at 3 bits on one GPU (OPT-175B, LLaMA-7B, LLaMA-65B: Elamur card "LUT-GEMM --
paper by Park et al. (2022)", section "Key points"). In generation at batch 1
every linear layer of every decoder layer is one GEMV, so the per-token time of
the weight products is the sum of the per-GEMV times this library measures.
This driver makes that link concrete: it holds a synthetic, randomly
initialised layer stack of a named shape in device memory (every layer its own
packed BCQ weights), runs one token through all of its GEMVs in order, and
captures the token in a HIP graph so that replaying it measures the products
alone, without host launch overhead.

What is modelled and what is not:
  * every projection of a layer is one product with its own weights, chained
    so that each product reads the output of an earlier one (the data
    dependence of a real decode step);
  * attention over the key/value cache, normalisations, activation functions
    and residual additions are not part of the kernel and are left out: the
    output projection reads the first d entries of the fused QKV output in
    place of the attention output, and the down projection reads the up half
    of the fused gate/up output in place of the gated activation;
  * scales are drawn so that one product keeps the activations' root mean
    square roughly unchanged (|N(0, sigma)| with sigma = 1/sqrt(q K)), so a
    deep chain stays finite in fp16.

Weights: one seeded random BCQ matrix per distinct (N, K) is packed on the host
and copied into each layer's own device buffers (distinct addresses, so no
layer's weights are found in a cache from another's).
"""
from __future__ import annotations

import argparse
import json
import sys
import time
from dataclasses import dataclass
from typing import Dict, List, Optional, Tuple

import numpy as np

from . import PackedBCQ, packed_sizes

__all__ = ["MODELS", "Projection", "DecodeStack", "weight_bytes_per_step", "main"]


@dataclass(frozen=True)
class Projection:
    """One linear layer of a decoder layer: y [N] = W [N][K] x, x read from `src`
    (the layer input "x" or an earlier projection's output), entries
    src_off .. src_off + K - 1."""

    name: str
    N: int
    K: int
    src: str
    src_off: int = 0


def _opt(d: int) -> List[Projection]:
    return [Projection("qkv", 3 * d, d, "x"), Projection("out", d, d, "qkv"),
            Projection("fc1", 4 * d, d, "out"), Projection("fc2", d, 4 * d, "fc1")]


def _llama(d: int, f: int) -> List[Projection]:
    # gate and up read the same input, so they are one product of 2f rows (as
    # inference engines fuse them); down reads the up half
    return [Projection("qkv", 3 * d, d, "x"), Projection("out", d, d, "qkv"),
            Projection("gate_up", 2 * f, d, "out"), Projection("down", d, f, "gate_up", f)]


# name -> (decoder layers, projections of one layer, index of the layer output)
MODELS: Dict[str, Tuple[int, List[Projection], str]] = {
    "opt175b": (96, _opt(12288), "fc2"),
    "llama7b": (32, _llama(4096, 11008), "down"),
    "llama65b": (80, _llama(8192, 22016), "down"),
}


def weight_bytes_per_step(model: str, q: int = 3, g: int = 128,
                           layers: Optional[int] = None) -> int:
    """Packed bytes (sign planes + fp16 scales) of every projection of every layer:
    what one decode step reads from memory, at the least (whatever the batch)."""
    full_layers, projs, _ = MODELS[model]
    tot = 0
    for p in projs:
        nb, na, _ = packed_sizes(p.N, p.K, q, g, False)
        tot += nb + 2 * na
    return tot * (full_layers if layers is None else int(layers))


class DecodeStack:
    """A synthetic layer stack in device memory and its per-token GEMV chain."""

    def __init__(self, model: str, layers: Optional[int] = None, q: int = 3, g: int = 128,
                 m: int = 1, seed: int = 0, device: str = "cuda:0", keep_logical: bool = False,
                 log=None):
        import torch
        import workloads

        if model not in MODELS:
            raise ValueError(f"unknown model {model!r}; choose from {sorted(MODELS)}")
        full_layers, projs, out_name = MODELS[model]
        self.model, self.q, self.g, self.m = model, int(q), int(g), int(m)
        self.layers = full_layers if layers is None else int(layers)
        if self.layers < 1:
            raise ValueError("layers must be >= 1")
        self.projs, self.out_name, self.device = projs, out_name, device
        self.logical = {}
        protos = {}
        for k, p in enumerate(projs):
            if (p.N, p.K) in protos:
                continue
            sigma = 1.0 / np.sqrt(self.q * p.K)
            w = workloads.random_bcq(p.N, p.K, self.q, self.g, self.m, seed=seed + 7919 * k,
                                     sigma=sigma, name=f"{model}_{p.name}")
            protos[(p.N, p.K)] = PackedBCQ.from_bcq(w.bits, w.alpha, None, self.g, device=device)
            if log:
                log(f"packed {p.name} {p.N}x{p.K}")
            if keep_logical:
                self.logical[(p.N, p.K)] = w
        # every layer gets its own copy of the packed buffers
        self.weights: List[Dict[str, PackedBCQ]] = []
        for _ in range(self.layers):
            lw = {}
            for p in projs:
                src = protos[(p.N, p.K)]
                lw[p.name] = PackedBCQ(p.N, p.K, self.q, self.g, src.d_bits.clone(),
                                       src.d_alpha.clone(), None)
            self.weights.append(lw)
        del protos
        # activations: the token input and one output buffer per projection
        rng = np.random.default_rng(seed)
        d_model = projs[0].K
        x0 = rng.standard_normal((self.m, d_model)).astype(np.float16)
        self.x = torch.from_numpy(x0).to(device)
        self.outs = {p.name: torch.empty((self.m, p.N), dtype=torch.float16, device=device)
                     for p in projs}
        self.graph = None
        self.graph_kernel = None

    # ------------------------------------------------------------ sizes
    def bytes_per_step(self) -> int:
        """Packed weight bytes every decode step reads (bits + scales, all layers)."""
        return weight_bytes_per_step(self.model, self.q, self.g, self.layers)

    # ------------------------------------------------------------ one token
    def _src(self, p: Projection, x_layer):
        t = x_layer if p.src == "x" else self.outs[p.src]
        return t[:, p.src_off:p.src_off + p.K] if t.shape[1] != p.K else t

    def token(self, kernel: str = "lut"):
        """Run every product of every layer once, in order, on the current stream.
        The layer output is the next layer's input; returns the last output (a
        buffer the next token overwrites)."""
        x_layer = self.x
        for l, lw in enumerate(self.weights):
            for p in self.projs:
                src = self._src(p, x_layer)
                if src.shape[1] != p.K or not src.is_contiguous():
                    src = src.contiguous()
                w = lw[p.name]
                if kernel == "lut":
                    w(src, out=self.outs[p.name])
                elif kernel == "dequant":
                    w.dequant(src, out=self.outs[p.name])
                else:
                    raise ValueError(f"unknown kernel {kernel!r}")
            # the next layer reads this output in place: its first product runs
            # before this buffer is written again
            x_layer = self.outs[self.out_name]
        return self.outs[self.out_name]

    def capture(self, kernel: str = "lut"):
        """Capture one token into a HIP graph. An eager token runs first on the
        capture stream, so the split-K workspaces (one per stream) are set up
        outside the capture and the graph reuses them."""
        import torch
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            self.token(kernel)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cs):
            self.token(kernel)
        torch.cuda.synchronize()
        self.graph, self.graph_kernel = g, kernel
        return g

    def time_tokens(self, kernel: str = "lut", tokens: int = 20, warmup: int = 5) -> dict:
        """Time of one decode step (one token for each of the m sequences),
        replaying the captured step graph `tokens` times."""
        import torch
        if self.graph is None or self.graph_kernel != kernel:
            self.capture(kernel)
        for _ in range(warmup):
            self.graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(tokens):
            self.graph.replay()
        e1.record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / tokens
        ms = e0.elapsed_time(e1) / tokens
        return {"kernel": kernel, "ms_per_step": ms, "wall_ms_per_step": wall,
                "tokens_per_s": self.m / (ms * 1e-3),
                "GBps": self.bytes_per_step() / (ms * 1e-3) / 1e9}


    def time_projection(self, name: str, kernel: str = "lut", reps: int = 10,
                        warmup: int = 3) -> dict:
        """Per-GEMV time of one projection: a graph running that projection of
        every layer back to back (distinct weights, so nothing is served from a
        cache), replayed `reps` times."""
        import torch
        p = next(pp for pp in self.projs if pp.name == name)
        self.token(kernel)                       # fills every source buffer
        torch.cuda.synchronize()
        src = self._src(p, self.outs[self.out_name]).contiguous()

        def run():
            for lw in self.weights:
                w = lw[name]
                if kernel == "lut":
                    w(src, out=self.outs[name])
                else:
                    w.dequant(src, out=self.outs[name])

        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            run()                                # workspaces of the capture stream
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cs):
            run()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * self.layers)
        nb, na, _ = packed_sizes(p.N, p.K, self.q, self.g, False)
        return {"projection": name, "N": p.N, "K": p.K, "kernel": kernel, "us": us,
                "GBps": (nb + 2 * na) / (us * 1e-6) / 1e9}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--model", default="opt175b", choices=sorted(MODELS))
    ap.add_argument("--layers", type=int, default=None, help="decoder layers (default: the model's)")
    ap.add_argument("--q", type=int, default=3)
    ap.add_argument("--g", type=int, default=128)
    ap.add_argument("--m", type=int, default=1,
                    help="sequences decoded together (batch rows of every product)")
    ap.add_argument("--tokens", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--kernel", default="both", choices=["lut", "dequant", "both"])
    ap.add_argument("--breakdown", action="store_true",
                    help="also time each projection on its own (us per GEMV)")
    a = ap.parse_args(argv)

    import torch
    if not torch.cuda.is_available():
        print("decode driver: no GPU visible", file=sys.stderr)
        return 2
    t0 = time.perf_counter()
    st = DecodeStack(a.model, a.layers, a.q, a.g, a.m,
                     log=lambda msg: print(f"[decode] {msg}", flush=True))
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t0
    print(f"[decode] {a.model}: {st.layers} layers, {st.bytes_per_step() / 1e9:.2f} GB packed "
          f"weights, set up in {setup_s:.1f} s", flush=True)
    res = {}
    kernels = ["lut", "dequant"] if a.kernel == "both" else [a.kernel]
    for k in kernels:
        r = st.time_tokens(k, a.tokens, a.warmup)
        y = st.outs[st.out_name]
        r["finite"] = bool(torch.isfinite(y).all().item())
        res[k] = r
        print(f"[decode] {k}: {r['ms_per_step']:.3f} ms per step of {st.m} token(s) "
              f"({r['tokens_per_s']:.0f} tokens/s, {r['GBps']:.0f} GB/s of weights)", flush=True)
    if a.breakdown:
        for k in kernels:
            rows = []
            for p in st.projs:
                r = st.time_projection(p.name, k, reps=max(2, a.tokens // 2))
                rows.append(r)
                print(f"[decode] {k} {p.name:5s} {p.N}x{p.K}: {r['us']:.2f} us "
                      f"({r['GBps']:.0f} GB/s)", flush=True)
            res[k]["breakdown"] = rows
    line = {"model": a.model, "layers": st.layers, "q": a.q, "g": a.g, "m": a.m,
            "weight_bytes_per_step": st.bytes_per_step(), "gemvs_per_step":
            st.layers * len(st.projs), "tokens": a.tokens, "results": res}
    if "lut" in res and "dequant" in res:
        line["dequant_over_lut"] = res["dequant"]["ms_per_step"] / res["lut"]["ms_per_step"]
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""Python binding of ``liblutgemm.so``, the MI355X (gfx950) BCQ LUT-GEMV library.

Argument marshalling only: every step of the product runs in the HIP kernels
behind the C ABI declared in ``include/lutgemm.h``. PyTorch supplies device
memory and streams. There is no CPU fallback: if the library is not built, or
the device is not gfx950, calls raise.

Names follow the C ABI: :func:`bcq_pack`, :func:`bcq_pack_uniform`,
:func:`lutgemm_run`, plus the size queries. :class:`PackedBCQ` bundles a
packed weight held in device memory with a reusable workspace.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

__all__ = [
    "LIB_PATH", "LutGemmError", "Shape", "lib", "abi_version", "status_string",
    "check_shape", "packed_sizes", "workspace_size", "workspace_init",
    "bcq_pack", "bcq_pack_uniform", "lutgemm_run", "bcq_dequant_gemv", "footprint_bits",
    "search_group_sizes", "bcq_quantize", "stream_read", "lutgemm_run_noalloc",
    "noalloc_scratch_bytes", "query_plan", "TABLES", "trace_attach", "use_traced_library",
    "PackedBCQ", "STATUS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblutgemm.so")
TRACE_LIB_PATH = os.path.join(_HERE, "liblutgemm_trace.so")

STATUS = {
    0: "LUTGEMM_OK", 1: "LUTGEMM_ERR_NULL", 2: "LUTGEMM_ERR_SHAPE", 3: "LUTGEMM_ERR_VALUE",
    4: "LUTGEMM_ERR_BUFFER", 5: "LUTGEMM_ERR_ALIGN", 6: "LUTGEMM_ERR_UNSUPPORTED",
    7: "LUTGEMM_ERR_HIP", 8: "LUTGEMM_ERR_INTERNAL",
}


class LutGemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.name = STATUS.get(status, f"status {status}")
        super().__init__(f"{where}: {self.name} ({status_string(status)})")


TABLES = {0: "single", 1: "paired", 2: "half", 3: "nibble", 4: "split", 5: "paired_mfma",
          6: "sign_mfma"}


class _Plan(ctypes.Structure):
    _fields_ = [("tables", ctypes.c_int32), ("waves", ctypes.c_int32),
                ("rows_per_wave", ctypes.c_int32), ("batch_rows", ctypes.c_int32),
                ("row_tiles", ctypes.c_int32), ("split", ctypes.c_int32),
                ("x_in_lds", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("items", ctypes.c_int64), ("workgroups", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_uint64)]


class Shape(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("K", ctypes.c_int32), ("q", ctypes.c_int32),
                ("g", ctypes.c_int32), ("has_offset", ctypes.c_int32)]

    def __repr__(self):
        return (f"Shape(N={self.N}, K={self.K}, q={self.q}, g={self.g}, "
                f"has_offset={self.has_offset})")


_LIB = None
_P = ctypes.c_void_p
_SZ = ctypes.c_size_t
_SZP = ctypes.POINTER(ctypes.c_size_t)
_SHP = ctypes.POINTER(Shape)


def lib() -> ctypes.CDLL:
    """Load the library once. Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    # torch first: its HIP runtime carries the same soname, so the library binds
    # to the runtime torch already loaded and torch's streams are valid here.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m lut_gemv_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    L.lutgemm_abi_version.restype = ctypes.c_int
    L.lutgemm_abi_version.argtypes = []
    L.lutgemm_status_string.restype = ctypes.c_char_p
    L.lutgemm_status_string.argtypes = [ctypes.c_int]
    L.lutgemm_check_shape.restype = ctypes.c_int
    L.lutgemm_check_shape.argtypes = [_SHP]
    L.lutgemm_packed_sizes.restype = ctypes.c_int
    L.lutgemm_packed_sizes.argtypes = [_SHP, _SZP, _SZP, _SZP]
    L.lutgemm_workspace_size.restype = ctypes.c_int
    L.lutgemm_workspace_size.argtypes = [_SHP, ctypes.c_int32, _SZP]
    L.lutgemm_workspace_init.restype = ctypes.c_int
    L.lutgemm_workspace_init.argtypes = [_P, _SZ, _P]
    L.bcq_pack.restype = ctypes.c_int
    L.bcq_pack.argtypes = [_SHP, _P, _P, _P, _P, _SZ, _P, _SZ, _P, _SZ]
    L.bcq_pack_uniform.restype = ctypes.c_int
    L.bcq_pack_uniform.argtypes = [_SHP, _P, _P, _P, _P, _SZ, _P, _SZ, _P, _SZ, _SZP]
    L.lutgemm_run.restype = ctypes.c_int
    L.lutgemm_run.argtypes = [_SHP, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _SZ, _P]
    L.bcq_footprint_bits.restype = ctypes.c_int
    L.bcq_footprint_bits.argtypes = [_SHP, ctypes.POINTER(ctypes.c_uint64)]
    L.bcq_search_group_sizes.restype = ctypes.c_int
    L.bcq_search_group_sizes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_double, ctypes.POINTER(ctypes.c_int32),
                                         ctypes.POINTER(ctypes.c_uint64)]
    L.bcq_quantize.restype = ctypes.c_int
    L.bcq_quantize.argtypes = [_SHP, _P, ctypes.c_int32, _P, _SZ, _P, _SZ,
                               ctypes.POINTER(ctypes.c_double)]
    L.bcq_dequant_gemv.restype = ctypes.c_int
    L.bcq_dequant_gemv.argtypes = [_SHP, ctypes.c_int32, _P, _P, _P, _P, _P, _P]
    L.lutgemm_run_noalloc.restype = ctypes.c_int
    L.lutgemm_run_noalloc.argtypes = [_SHP, ctypes.c_int32, _P, _P, _P, _P, _P, _P]
    L.lutgemm_noalloc_scratch_bytes.restype = ctypes.c_size_t
    L.lutgemm_noalloc_scratch_bytes.argtypes = []
    L.lutgemm_stream_read.restype = ctypes.c_int
    L.lutgemm_stream_read.argtypes = [_P, _SZ, _P, _SZ, ctypes.c_int, _P]
    L.lutgemm_trace_attach.restype = ctypes.c_int
    L.lutgemm_trace_attach.argtypes = [_P, _SZ]
    L.lutgemm_query_plan.restype = ctypes.c_int
    L.lutgemm_query_plan.argtypes = [_SHP, ctypes.c_int32, ctypes.c_int32, _SZ,
                                     ctypes.POINTER(_Plan)]
    _LIB = L
    return L


def _check(status: int, where: str):
    if status != 0:
        raise LutGemmError(status, where)


def abi_version() -> int:
    return lib().lutgemm_abi_version()


def status_string(status: int) -> str:
    return lib().lutgemm_status_string(status).decode()


def _shape(N, K, q, g, has_offset) -> Shape:
    return Shape(int(N), int(K), int(q), int(g), int(bool(has_offset)))


def check_shape(N, K, q, g, has_offset=False) -> int:
    """Status code of the shape check (0 when valid)."""
    s = _shape(N, K, q, g, has_offset)
    return lib().lutgemm_check_shape(ctypes.byref(s))


def packed_sizes(N, K, q, g, has_offset=False):
    """(bytes of packed bits, fp16 count of packed alpha, fp16 count of packed offset)."""
    s = _shape(N, K, q, g, has_offset)
    b, a, o = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().lutgemm_packed_sizes(ctypes.byref(s), ctypes.byref(b), ctypes.byref(a),
                                      ctypes.byref(o)), "lutgemm_packed_sizes")
    return b.value, a.value, o.value


def workspace_size(N, K, q, g, has_offset, m) -> int:
    s = _shape(N, K, q, g, has_offset)
    out = ctypes.c_size_t()
    _check(lib().lutgemm_workspace_size(ctypes.byref(s), int(m), ctypes.byref(out)),
           "lutgemm_workspace_size")
    return out.value


def workspace_init(d_workspace: int, nbytes: int, stream: Optional[int] = None):
    """Zero-fill a device workspace on ``stream`` (required before its first use)."""
    _check(lib().lutgemm_workspace_init(d_workspace, int(nbytes), stream), "lutgemm_workspace_init")


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _u16(a):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("fp16 arrays must be float16 or their uint16 bit patterns")
    return a


def bcq_pack(bits: np.ndarray, alpha: np.ndarray, offset: Optional[np.ndarray], g: int):
    """Pack a BCQ matrix (logical format) into the device format, on the host.

    ``bits`` uint8 [q][N][K/8], ``alpha`` fp16 [q][N][K/g], ``offset`` fp16
    [N][K/g] or None. Returns ``(packed_bits uint8, packed_alpha uint16,
    packed_offset uint16 or None)``.
    """
    bits = _c(bits, np.uint8)
    alpha = _u16(alpha)
    offset = _u16(offset)
    q, N, C = bits.shape
    K = 8 * C
    s = _shape(N, K, q, g, offset is not None)
    nb, na, no = packed_sizes(N, K, q, g, offset is not None)
    ob = np.empty(nb, np.uint8)
    oa = np.empty(na, np.uint16)
    oo = np.empty(no, np.uint16) if offset is not None else None
    _check(lib().bcq_pack(ctypes.byref(s), _ptr(bits), _ptr(alpha), _ptr(offset), _ptr(ob), nb,
                          _ptr(oa), na, _ptr(oo), no), "bcq_pack")
    return ob, oa, oo


def bcq_pack_uniform(codes: np.ndarray, scale: np.ndarray, zero: np.ndarray, q: int, g: int):
    """Rewrite a uniform int-q matrix as BCQ + offset and pack it, on the host.

    Returns ``(packed_bits, packed_alpha, packed_offset, n_rounded)``.
    """
    codes = _c(codes, np.uint8)
    scale = _u16(scale)
    zero = _c(zero, np.uint8)
    N, K = codes.shape
    s = _shape(N, K, q, g, True)
    nb, na, no = packed_sizes(N, K, q, g, True)
    ob = np.empty(nb, np.uint8)
    oa = np.empty(na, np.uint16)
    oo = np.empty(no, np.uint16)
    n_r = ctypes.c_size_t()
    _check(lib().bcq_pack_uniform(ctypes.byref(s), _ptr(codes), _ptr(scale), _ptr(zero),
                                  _ptr(ob), nb, _ptr(oa), na, _ptr(oo), no, ctypes.byref(n_r)),
           "bcq_pack_uniform")
    return ob, oa, oo, n_r.value


def lutgemm_run(shape: Shape, m: int, d_bits: int, d_alpha: int, d_offset: Optional[int],
                d_x: int, d_y: int, d_workspace: Optional[int], workspace_bytes: int,
                stream: Optional[int]):
    """Raw entry point: device addresses as integers, ``stream`` a hipStream_t handle."""
    _check(lib().lutgemm_run(ctypes.byref(shape), int(m), d_bits, d_alpha, d_offset, d_x, d_y,
                             d_workspace, int(workspace_bytes), stream), "lutgemm_run")


def lutgemm_run_noalloc(shape: Shape, m: int, d_bits: int, d_alpha: int, d_offset: Optional[int],
                        d_x: int, d_y: int, stream: Optional[int]):
    """Raw entry point that allocates nothing (its split partials live in the
    library's per-GPU scratch); calls that overlap in time on one GPU race."""
    _check(lib().lutgemm_run_noalloc(ctypes.byref(shape), int(m), d_bits, d_alpha, d_offset, d_x,
                                     d_y, stream), "lutgemm_run_noalloc")


def noalloc_scratch_bytes() -> int:
    """Bytes of the per-GPU scratch array of :func:`lutgemm_run_noalloc`."""
    return lib().lutgemm_noalloc_scratch_bytes()


def query_plan(N: int, K: int, q: int, g: int, has_offset: bool, m: int, cus: int = 256,
               workspace_bytes: Optional[int] = None) -> dict:
    """The launch chosen for this shape and batch on `cus` compute units with its
    split limited to `workspace_bytes` (None: unlimited); host only."""
    pl = _Plan()
    ws = (1 << 64) - 1 if workspace_bytes is None else int(workspace_bytes)
    _check(lib().lutgemm_query_plan(ctypes.byref(_shape(N, K, q, g, has_offset)), int(m), int(cus),
                                    ws, ctypes.byref(pl)), "lutgemm_query_plan")
    d = {f: int(getattr(pl, f)) for f, _ in _Plan._fields_ if f != "reserved"}
    d["tables"] = TABLES[d["tables"]]
    return d


def use_traced_library() -> None:
    """Make this process load the phase-traced build (liblutgemm_trace.so)
    instead of the regular one; call before anything else of this module."""
    global LIB_PATH
    if _LIB is not None and LIB_PATH != TRACE_LIB_PATH:
        raise RuntimeError("the regular library is already loaded in this process")
    LIB_PATH = TRACE_LIB_PATH


def trace_attach(d_buffer: Optional[int], nbytes: int) -> None:
    """Phase stamps of later launches into a device buffer of uint64
    [workgroup][8] (lutgemm_trace_attach); the traced library only."""
    _check(lib().lutgemm_trace_attach(d_buffer, int(nbytes)), "lutgemm_trace_attach")


def footprint_bits(N: int, K: int, q: int, g: int, has_offset: bool = False) -> int:
    """Storage in bits of an N x K BCQ matrix, scales (and offsets) included."""
    out = ctypes.c_uint64()
    _check(lib().bcq_footprint_bits(ctypes.byref(_shape(N, K, q, g, has_offset)), ctypes.byref(out)),
           "bcq_footprint_bits")
    return out.value


def search_group_sizes(N: int, K: int, max_bits_per_weight: float, has_offset: bool = False):
    """{q: (g, bits)} for q = 1..8: the finest group size meeting the storage target
    (q absent when none does)."""
    gs = (ctypes.c_int32 * 8)()
    bs = (ctypes.c_uint64 * 8)()
    _check(lib().bcq_search_group_sizes(int(N), int(K), int(bool(has_offset)),
                                        float(max_bits_per_weight), gs, bs),
           "bcq_search_group_sizes")
    return {q + 1: (gs[q], bs[q]) for q in range(8) if gs[q]}


def bcq_quantize(w, q: int, g: int, iters: int = 0):
    """fp16 W [N][K] -> (bits uint8 [q][N][K/8], alpha fp16 [q][N][K/g], squared error)."""
    w = np.ascontiguousarray(w, dtype=np.float16)
    N, K = w.shape
    bits = np.zeros((q, N, K // 8), np.uint8)
    alpha = np.zeros((q, N, K // g if K else 0), np.uint16)
    err = ctypes.c_double()
    _check(lib().bcq_quantize(ctypes.byref(_shape(N, K, q, g, False)), w.ctypes.data, int(iters),
                              bits.ctypes.data, bits.nbytes, alpha.ctypes.data, alpha.size,
                              ctypes.byref(err)), "bcq_quantize")
    return bits, alpha.view(np.float16), err.value


def bcq_dequant_gemv(shape: Shape, m: int, d_bits: int, d_alpha: int, d_offset: Optional[int],
                     d_x: int, d_y: int, stream: Optional[int]):
    """Raw entry point of the dequantizing comparison kernel (same packed format)."""
    _check(lib().bcq_dequant_gemv(ctypes.byref(shape), int(m), d_bits, d_alpha, d_offset, d_x,
                                  d_y, stream), "bcq_dequant_gemv")


def stream_read(d_src: int, nbytes: int, d_sink: int, sink_count: int, nontemporal: bool,
                stream: Optional[int]):
    """Measurement aid: read ``nbytes`` of device memory once (lutgemm_stream_read)."""
    _check(lib().lutgemm_stream_read(d_src, int(nbytes), d_sink, int(sink_count),
                                     int(bool(nontemporal)), stream), "lutgemm_stream_read")


class PackedBCQ:
    """A packed BCQ weight in device memory, ready for :meth:`__call__`.

    Device buffers are torch tensors (memory only); the product itself is one
    :func:`lutgemm_run` call on the current torch stream.
    """

    def __init__(self, N: int, K: int, q: int, g: int, d_bits, d_alpha, d_offset=None):
        self.N, self.K, self.q, self.g = int(N), int(K), int(q), int(g)
        self.has_offset = d_offset is not None
        self.shape = _shape(N, K, q, g, self.has_offset)
        self.d_bits, self.d_alpha, self.d_offset = d_bits, d_alpha, d_offset
        self._ws = {}   # stream handle -> workspace tensor

    @classmethod
    def _upload(cls, N, K, q, g, pb, pa, po, device):
        import torch
        d_bits = torch.from_numpy(pb).to(device)
        d_alpha = torch.from_numpy(pa.view(np.int16)).to(device)
        d_off = torch.from_numpy(po.view(np.int16)).to(device) if po is not None else None
        return cls(N, K, q, g, d_bits, d_alpha, d_off)

    @classmethod
    def from_bcq(cls, bits, alpha, offset, g, device="cuda"):
        q, N, C = np.asarray(bits).shape
        pb, pa, po = bcq_pack(bits, alpha, offset, g)
        return cls._upload(N, 8 * C, q, g, pb, pa, po, device)

    @classmethod
    def from_uniform(cls, codes, scale, zero, q, g, device="cuda"):
        N, K = np.asarray(codes).shape
        pb, pa, po, n_r = bcq_pack_uniform(codes, scale, zero, q, g)
        obj = cls._upload(N, K, q, g, pb, pa, po, device)
        obj.n_rounded = n_r
        return obj

    def workspace(self, m: int, stream=None):
        """A zero-filled device workspace large enough for batch m on ``stream``
        (default: the current stream), or ``(None, 0)`` when none is needed.

        Calls that overlap in time must not share a workspace, so one is kept per
        stream and reused by every later call on that stream (each completed call
        leaves its counters zero). It is allocated while that stream is current,
        so when a larger one replaces it the allocator reuses the old memory only
        in that stream's order."""
        import torch
        need = workspace_size(self.N, self.K, self.q, self.g, self.has_offset, m)
        if need == 0:
            return None, 0
        dev = self.d_bits.device
        if stream is None:
            stream = torch.cuda.current_stream(dev)
        key = stream.cuda_stream
        ws = self._ws.get(key)
        if ws is None or ws.numel() < need:
            with torch.cuda.stream(stream):
                ws = torch.empty(need, dtype=torch.uint8, device=dev)
            workspace_init(ws.data_ptr(), need, key)
            self._ws[key] = ws
        return ws, ws.numel()

    def _check_io(self, x, out):
        import torch
        if x.dtype != torch.float16 or x.dim() != 2 or x.shape[1] != self.K:
            raise ValueError(f"x must be fp16 [m][{self.K}]")
        if x.device != self.d_bits.device:
            raise ValueError(f"x is on {x.device}, the weights on {self.d_bits.device}")
        if out is not None and (out.dtype != torch.float16 or tuple(out.shape) != (x.shape[0], self.N)
                                or out.device != x.device or not out.is_contiguous()):
            raise ValueError(f"out must be a contiguous fp16 [{x.shape[0]}][{self.N}] tensor on {x.device}")

    def __call__(self, x, out=None):
        """y = W_hat x for fp16 x [m][K] on the device; returns fp16 y [m][N]."""
        import torch
        self._check_io(x, out)
        x = x.contiguous()
        m = x.shape[0]
        if out is None:
            out = torch.empty((m, self.N), dtype=torch.float16, device=x.device)
        strm = torch.cuda.current_stream(x.device)
        ws, ws_bytes = self.workspace(m, strm)
        stream = strm.cuda_stream
        lutgemm_run(self.shape, m, self.d_bits.data_ptr(), self.d_alpha.data_ptr(),
                    self.d_offset.data_ptr() if self.d_offset is not None else None,
                    x.data_ptr(), out.data_ptr(),
                    ws.data_ptr() if ws is not None else None, ws_bytes, stream)
        return out

    def dequant(self, x, out=None):
        """The same product by the dequantizing comparison kernel (bcq_dequant_gemv)."""
        import torch
        self._check_io(x, out)
        x = x.contiguous()
        m = x.shape[0]
        if out is None:
            out = torch.empty((m, self.N), dtype=torch.float16, device=x.device)
        stream = torch.cuda.current_stream(x.device).cuda_stream
        bcq_dequant_gemv(self.shape, m, self.d_bits.data_ptr(), self.d_alpha.data_ptr(),
                         self.d_offset.data_ptr() if self.d_offset is not None else None,
                         x.data_ptr(), out.data_ptr(), stream)
        return out

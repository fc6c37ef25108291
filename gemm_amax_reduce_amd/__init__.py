"""Python binding of the MI355X NVFP4 linear-layer library (``libnvfp4.so``).

Argument marshalling only: every step of quantize / dequantize / GEMM runs in
the gfx950 kernels behind the C ABI of ``include/nvfp4.h``.  torch supplies
device memory and the current HIP stream.  There is no CPU fallback: if the
library is not built, or no GPU is visible, the calls raise.

Names follow the C ABI: ``nvfp4_quantize``, ``nvfp4_rht_quantize``,
``nvfp4_dequantize``, ``nvfp4_gemm``.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["NVFP4Tensor", "NVFP4Error", "nvfp4_quantize", "nvfp4_rht_quantize", "nvfp4_quantize_dual", "nvfp4_amax",
           "nvfp4_quantize_amax", "MXFP4Tensor", "mxfp4_quantize", "mxfp4_gemm", "MXFP8Tensor", "mxfp8_quantize",
           "mxfp8_gemm",
           "nvfp4_dequantize", "nvfp4_gemm", "nvfp4_gemm_ws", "nvfp4_gemm_noalloc", "gemm_workspace", "lib", "LIB_PATH", "F32", "BF16", "RNE", "SR"]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvfp4.so")

F32, BF16 = 0, 1
RNE, SR = 0, 1


class NVFP4Error(RuntimeError):
    pass


class _CTensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("meta", ctypes.c_void_p),
                ("outer", ctypes.c_int64), ("k", ctypes.c_int64)]


class _MXTensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("outer", ctypes.c_int64),
                ("k", ctypes.c_int64)]


_lib = None

# every symbol the header declares
EXPORTS = ("nvfp4_quantize", "nvfp4_rht_quantize", "nvfp4_amax", "nvfp4_quantize_amax", "nvfp4_quantize_dual",
           "mxfp4_quantize", "mxfp4_gemm", "nvfp4_dequantize", "nvfp4_gemm", "nvfp4_gemm_ws",
           "nvfp4_gemm_workspace_bytes", "nvfp4_gemm_noalloc", "mxfp8_quantize", "mxfp8_gemm", "nvfp4_probe_mfma",
           "nvfp4_probe_philox", "nvfp4_status_string")


def lib() -> ctypes.CDLL:
    """Load ``libnvfp4.so`` (build it with ``gemm_amax_reduce_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise NVFP4Error(f"{LIB_PATH} is missing: run gemm_amax_reduce_amd/build.py "
                             "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        i64, u64, vp, ci = ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int
        pt = ctypes.POINTER(_CTensor)
        L.nvfp4_quantize.argtypes = [vp, ci, i64, i64, ci, ci, u64, u64, pt, vp]
        L.nvfp4_quantize.restype = ci
        L.nvfp4_rht_quantize.argtypes = [vp, ci, i64, i64, ci, ci, u64, u64, ctypes.c_uint16, pt, vp]
        L.nvfp4_rht_quantize.restype = ci
        mt = ctypes.POINTER(_MXTensor)
        L.mxfp4_quantize.argtypes = [vp, ci, i64, i64, ci, mt, vp]
        L.mxfp4_quantize.restype = ci
        L.mxfp4_gemm.argtypes = [mt, mt, vp, ci, i64, vp]
        L.mxfp4_gemm.restype = ci
        L.mxfp8_quantize.argtypes = [vp, ci, i64, i64, ci, mt, vp]
        L.mxfp8_quantize.restype = ci
        L.mxfp8_gemm.argtypes = [mt, mt, vp, ci, i64, vp]
        L.mxfp8_gemm.restype = ci
        L.nvfp4_amax.argtypes = [vp, ci, i64, i64, ci, ci, ctypes.c_uint16, vp, vp]
        L.nvfp4_amax.restype = ci
        L.nvfp4_quantize_amax.argtypes = [vp, ci, i64, i64, ci, ci, u64, u64, ci, ctypes.c_uint16, vp, pt, vp]
        L.nvfp4_quantize_amax.restype = ci
        L.nvfp4_quantize_dual.argtypes = [vp, ci, i64, i64, ci, u64, u64, pt, ci, ctypes.c_uint16, ci, u64, u64,
                                          pt, vp]
        L.nvfp4_quantize_dual.restype = ci
        L.nvfp4_dequantize.argtypes = [pt, vp, ci, vp]
        L.nvfp4_dequantize.restype = ci
        L.nvfp4_gemm.argtypes = [pt, pt, vp, ci, i64, vp]
        L.nvfp4_gemm.restype = ci
        L.nvfp4_gemm_ws.argtypes = [pt, pt, vp, ci, i64, vp, i64, vp]
        L.nvfp4_gemm_ws.restype = ci
        L.nvfp4_gemm_workspace_bytes.argtypes = []
        L.nvfp4_gemm_noalloc.argtypes = [pt, pt, vp, ci, i64, vp]
        L.nvfp4_gemm_noalloc.restype = ci
        L.nvfp4_gemm_workspace_bytes.restype = i64
        L.nvfp4_probe_mfma.argtypes = [i64, vp, vp]
        L.nvfp4_probe_mfma.restype = ci
        L.nvfp4_probe_philox.argtypes = [i64, vp, vp]
        L.nvfp4_probe_philox.restype = ci
        L.nvfp4_status_string.argtypes = [ci]
        L.nvfp4_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(rc: int, what: str):
    if rc != 0:
        msg = lib().nvfp4_status_string(rc).decode()
        raise NVFP4Error(f"{what} failed: {msg} ({rc})")


def _stream_handle(stream, device) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return int(s.cuda_stream)


def _require_device(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise NVFP4Error(f"{name} must be a GPU tensor (no CPU path exists)")


def _require_buffer(t: torch.Tensor, name: str, dtype: torch.dtype, numel: int, device: torch.device):
    """A caller-supplied device buffer the kernels write or read whole: the
    C ABI cannot see its size, so it is checked here."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != device:
        raise NVFP4Error(f"{name} must be a GPU tensor on {device}")
    if t.dtype != dtype:
        raise NVFP4Error(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous() or t.numel() < numel:
        raise NVFP4Error(f"{name} must be contiguous with at least {numel} elements")


def _out_code(dtype) -> int:
    if dtype == torch.float32:
        return F32
    if dtype == torch.bfloat16:
        return BF16
    raise NVFP4Error(f"unsupported output dtype {dtype} (float32 or bfloat16)")


def _require_matrix_out(out: torch.Tensor, rows: int, cols: int, dtype, device: torch.device) -> int:
    """Check a caller-supplied [rows][cols] output view (row stride >= cols)
    and return its leading dimension."""
    if not isinstance(out, torch.Tensor) or not out.is_cuda or out.device != device:
        raise NVFP4Error(f"out must be a GPU tensor on {device}")
    if out.dtype != dtype:
        raise NVFP4Error(f"out has dtype {out.dtype}, expected {dtype}")
    if out.dim() != 2 or tuple(out.shape) != (rows, cols):
        raise NVFP4Error(f"out must have shape ({rows}, {cols}), got {tuple(out.shape)}")
    if cols > 1 and out.stride(1) != 1:
        raise NVFP4Error("out must be row-major (unit column stride)")
    if rows > 1 and out.stride(0) < cols:
        raise NVFP4Error("out rows overlap (row stride < columns)")
    return out.stride(0) if rows > 1 else max(cols, 1)


class NVFP4Tensor:
    """Device buffers of one NVFP4 tensor in its quantized [outer][k] layout:
    ``codes`` u8 [outer, k/2], ``scales`` u8 [outer, k/16], ``meta`` f32 [2]
    = (amax, g)."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor, meta: torch.Tensor, outer: int, k: int):
        self.codes, self.scales, self.meta = codes, scales, meta
        self.outer, self.k = int(outer), int(k)

    @classmethod
    def empty(cls, outer: int, k: int, device=None) -> "NVFP4Tensor":
        device = device if device is not None else torch.device("cuda", torch.cuda.current_device())
        codes = torch.empty((outer, k // 2), dtype=torch.uint8, device=device)
        scales = torch.empty((outer, k // 16), dtype=torch.uint8, device=device)
        meta = torch.empty(2, dtype=torch.float32, device=device)
        return cls(codes, scales, meta, outer, k)

    @property
    def device(self) -> torch.device:
        return self.codes.device

    def _c(self) -> _CTensor:
        if self.outer < 0 or self.k < 0 or self.k % 16:
            raise NVFP4Error(f"invalid NVFP4 shape ({self.outer}, {self.k})")
        dev = self.codes.device
        _require_buffer(self.codes, "codes", torch.uint8, self.outer * (self.k // 2), dev)
        _require_buffer(self.scales, "scales", torch.uint8, self.outer * (self.k // 16), dev)
        _require_buffer(self.meta, "meta", torch.float32, 2, dev)
        return _CTensor(self.codes.data_ptr(), self.scales.data_ptr(), self.meta.data_ptr(), self.outer, self.k)

    @property
    def shape(self):
        return (self.outer, self.k)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise NVFP4Error(f"unsupported input dtype {t.dtype} (f32 or bf16)")


def _rounding_code(r) -> int:
    if isinstance(r, str):
        r = {"rne": RNE, "sr": SR}[r.lower()]
    return int(r)


def _same_device(q, x: torch.Tensor):
    if q.device != x.device:
        raise NVFP4Error(f"output on {q.device}, input on {x.device}")


def _quantize(x, axis, rounding, seed, offset, rht, sign_mask, out, stream):
    _require_device(x, "x")
    if x.dim() != 2 or not x.is_contiguous():
        raise NVFP4Error("x must be a contiguous 2-D tensor")
    rows, cols = x.shape
    outer, k = (rows, cols) if axis == 1 else (cols, rows)
    if out is None:
        out = NVFP4Tensor.empty(outer, k, device=x.device)
    _same_device(out, x)
    ct = out._c()
    with torch.cuda.device(x.device):
        if rht:
            rc = lib().nvfp4_rht_quantize(x.data_ptr(), _dtype_code(x), rows, cols, axis, _rounding_code(rounding),
                                          seed, offset, sign_mask & 0xFFFF, ctypes.byref(ct),
                                          _stream_handle(stream, x.device))
        else:
            rc = lib().nvfp4_quantize(x.data_ptr(), _dtype_code(x), rows, cols, axis, _rounding_code(rounding),
                                      seed, offset, ctypes.byref(ct), _stream_handle(stream, x.device))
    _check(rc, "nvfp4_rht_quantize" if rht else "nvfp4_quantize")
    return out


def nvfp4_quantize(x: torch.Tensor, axis: int = 1, rounding="rne", seed: int = 0, offset: int = 0,
                   out: NVFP4Tensor | None = None, stream=None) -> NVFP4Tensor:
    """Quantize a 2-D f32/bf16 GPU tensor to NVFP4 (see include/nvfp4.h)."""
    return _quantize(x, axis, rounding, seed, offset, False, 0, out, stream)


def nvfp4_rht_quantize(x: torch.Tensor, sign_mask: int, axis: int = 1, rounding="rne", seed: int = 0,
                       offset: int = 0, out: NVFP4Tensor | None = None, stream=None) -> NVFP4Tensor:
    """Quantize after the 16-point random Hadamard transform along k."""
    return _quantize(x, axis, rounding, seed, offset, True, sign_mask, out, stream)


def nvfp4_amax(x: torch.Tensor, axis: int = 1, rht: bool = False, sign_mask: int = 0,
               out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The tensor amax of x on `axis` (after the RHT if rht), as f32 [1] on x's device."""
    _require_device(x, "x")
    if x.dim() != 2 or not x.is_contiguous():
        raise NVFP4Error("x must be a contiguous 2-D tensor")
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=x.device)
    _require_buffer(out, "out", torch.float32, 1, x.device)
    rows, cols = x.shape
    with torch.cuda.device(x.device):
        _check(lib().nvfp4_amax(x.data_ptr(), _dtype_code(x), rows, cols, axis, int(bool(rht)), sign_mask & 0xFFFF,
                                out.data_ptr(), _stream_handle(stream, x.device)), "nvfp4_amax")
    return out


def nvfp4_quantize_amax(x: torch.Tensor, amax: torch.Tensor, axis: int = 1, rounding="rne", seed: int = 0,
                        offset: int = 0, rht: bool = False, sign_mask: int = 0,
                        out: NVFP4Tensor | None = None, stream=None) -> NVFP4Tensor:
    """Quantize with the tensor amax supplied (device f32, element 0)."""
    _require_device(x, "x")
    _require_device(amax, "amax")
    if x.dim() != 2 or not x.is_contiguous():
        raise NVFP4Error("x must be a contiguous 2-D tensor")
    _require_buffer(amax, "amax", torch.float32, 1, x.device)
    rows, cols = x.shape
    outer, k = (rows, cols) if axis == 1 else (cols, rows)
    if out is None:
        out = NVFP4Tensor.empty(outer, k, device=x.device)
    _same_device(out, x)
    ct = out._c()
    with torch.cuda.device(x.device):
        _check(lib().nvfp4_quantize_amax(x.data_ptr(), _dtype_code(x), rows, cols, axis, _rounding_code(rounding),
                                         seed, offset, int(bool(rht)), sign_mask & 0xFFFF, amax.data_ptr(),
                                         ctypes.byref(ct), _stream_handle(stream, x.device)), "nvfp4_quantize_amax")
    return out


def nvfp4_quantize_dual(x: torch.Tensor, rounding1="rne", seed1: int = 0, offset1: int = 0,
                        rht0: bool = False, sign_mask0: int = 0, rounding0="rne", seed0: int = 0,
                        offset0: int = 0, out1: NVFP4Tensor | None = None, out0: NVFP4Tensor | None = None,
                        stream=None) -> tuple[NVFP4Tensor, NVFP4Tensor]:
    """Both layouts of x with one amax read: (axis-1 tensor, axis-0 tensor),
    bit-identical to the two single quantizations (see include/nvfp4.h)."""
    _require_device(x, "x")
    if x.dim() != 2 or not x.is_contiguous():
        raise NVFP4Error("x must be a contiguous 2-D tensor")
    rows, cols = x.shape
    if out1 is None:
        out1 = NVFP4Tensor.empty(rows, cols, device=x.device)
    if out0 is None:
        out0 = NVFP4Tensor.empty(cols, rows, device=x.device)
    _same_device(out1, x)
    _same_device(out0, x)
    c1, c0 = out1._c(), out0._c()
    with torch.cuda.device(x.device):
        rc = lib().nvfp4_quantize_dual(x.data_ptr(), _dtype_code(x), rows, cols, _rounding_code(rounding1), seed1,
                                       offset1, ctypes.byref(c1), int(bool(rht0)), sign_mask0 & 0xFFFF,
                                       _rounding_code(rounding0), seed0, offset0, ctypes.byref(c0),
                                       _stream_handle(stream, x.device))
    _check(rc, "nvfp4_quantize_dual")
    return out1, out0


def nvfp4_dequantize(q: NVFP4Tensor, dtype=torch.float32, out: torch.Tensor | None = None,
                     stream=None) -> torch.Tensor:
    """Decode to f32/bf16 in the quantized [outer][k] layout."""
    code = _out_code(dtype)
    dev = q.device
    if out is None:
        out = torch.empty((q.outer, q.k), dtype=dtype, device=dev)
    _require_buffer(out, "out", dtype, q.outer * q.k, dev)
    ct = q._c()
    with torch.cuda.device(dev):
        _check(lib().nvfp4_dequantize(ctypes.byref(ct), out.data_ptr(), code, _stream_handle(stream, dev)),
               "nvfp4_dequantize")
    return out


def nvfp4_gemm(a: NVFP4Tensor, b: NVFP4Tensor, out_dtype=torch.float32, out: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
    """C = A . B^T for A [M, K] and B [N, K] NVFP4 tensors, f32 accumulation."""
    code = _out_code(out_dtype)
    dev = a.device
    if b.device != dev:
        raise NVFP4Error(f"operands on {a.device} and {b.device}")
    if out is None:
        out = torch.empty((a.outer, b.outer), dtype=out_dtype, device=dev)
    ldc = _require_matrix_out(out, a.outer, b.outer, out_dtype, dev)
    ca, cb = a._c(), b._c()
    with torch.cuda.device(dev):
        _check(lib().nvfp4_gemm(ctypes.byref(ca), ctypes.byref(cb), out.data_ptr(), code, ldc,
                                _stream_handle(stream, dev)), "nvfp4_gemm")
    return out


_workspaces: dict = {}


def gemm_workspace(device=None, stream=None) -> torch.Tensor:
    """The split-tail GEMM workspace for one (device, stream): allocated
    zero-filled on first use and kept (the kernel leaves it zero-filled).
    Calls on one stream run in order, so a workspace per stream is never
    used by two calls at once."""
    device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    s = stream if stream is not None else torch.cuda.current_stream(device)
    key = (device, int(s.cuda_stream))
    ws = _workspaces.get(key)
    if ws is None:
        ws = torch.zeros(int(lib().nvfp4_gemm_workspace_bytes()), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def nvfp4_gemm_ws(a: NVFP4Tensor, b: NVFP4Tensor, out_dtype=torch.float32, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """C = A . B^T with a workspace (same result contract as nvfp4_gemm):
    the tiles of a partly filled last round split into K ranges where that
    is faster; `workspace` defaults to the one of (device, stream)."""
    code = _out_code(out_dtype)
    dev = a.device
    if b.device != dev:
        raise NVFP4Error(f"operands on {a.device} and {b.device}")
    if out is None:
        out = torch.empty((a.outer, b.outer), dtype=out_dtype, device=dev)
    ldc = _require_matrix_out(out, a.outer, b.outer, out_dtype, dev)
    ws = workspace if workspace is not None else gemm_workspace(dev, stream)
    _require_buffer(ws, "workspace", torch.uint8, int(lib().nvfp4_gemm_workspace_bytes()), dev)
    ca, cb = a._c(), b._c()
    with torch.cuda.device(dev):
        _check(lib().nvfp4_gemm_ws(ctypes.byref(ca), ctypes.byref(cb), out.data_ptr(), code, ldc, ws.data_ptr(),
                                   ws.numel(), _stream_handle(stream, dev)), "nvfp4_gemm_ws")
    return out


def nvfp4_gemm_noalloc(a: NVFP4Tensor, b: NVFP4Tensor, out: torch.Tensor, out_dtype=torch.float32,
                       stream=None) -> torch.Tensor:
    """nvfp4_gemm_ws with the library's own per-GPU workspace: allocates
    nothing (the caller supplies `out`).  Calls overlapping in time on one
    GPU race."""
    code = _out_code(out_dtype)
    dev = a.device
    if b.device != dev:
        raise NVFP4Error(f"operands on {a.device} and {b.device}")
    ldc = _require_matrix_out(out, a.outer, b.outer, out_dtype, dev)
    ca, cb = a._c(), b._c()
    with torch.cuda.device(dev):
        _check(lib().nvfp4_gemm_noalloc(ctypes.byref(ca), ctypes.byref(cb), out.data_ptr(), code, ldc,
                                        _stream_handle(stream, dev)), "nvfp4_gemm_noalloc")
    return out


def nvfp4_probe_mfma(iters: int, stream=None) -> float:
    """Run the MFMA ceiling probe (include/nvfp4.h) once on the current device
    and return its rate in TFLOP/s, timed with events on the probe's stream.
    A measurement helper for the benchmark, not part of the method."""
    dev = torch.device("cuda", torch.cuda.current_device())
    out = torch.empty(1024 * 256, dtype=torch.float32, device=dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        _check(lib().nvfp4_probe_mfma(min(iters, 8), out.data_ptr(), _stream_handle(s, dev)), "nvfp4_probe_mfma")
        e0.record(s)
        _check(lib().nvfp4_probe_mfma(iters, out.data_ptr(), _stream_handle(s, dev)), "nvfp4_probe_mfma")
        e1.record(s)
    e1.synchronize()
    return 1024 * 4 * iters * 32 * 32768 / (e0.elapsed_time(e1) * 1e-3) / 1e12


def nvfp4_probe_philox(calls: int, stream=None) -> float:
    """Run the Philox probe (include/nvfp4.h) once for `calls` counters on the
    current device and return its time in ms (events on the probe's stream).
    A measurement helper for the benchmark, not part of the method."""
    dev = torch.device("cuda", torch.cuda.current_device())
    out = torch.empty(4096 * 256, dtype=torch.int32, device=dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        _check(lib().nvfp4_probe_philox(min(calls, 1 << 20), out.data_ptr(), _stream_handle(s, dev)),
               "nvfp4_probe_philox")
        e0.record(s)
        _check(lib().nvfp4_probe_philox(calls, out.data_ptr(), _stream_handle(s, dev)), "nvfp4_probe_philox")
        e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1)


class MXFP4Tensor:
    """Device buffers of one MXFP4 tensor in its quantized [outer][k] layout:
    ``codes`` u8 [outer, k/2], ``scales`` u8 [outer, k/32] (E8M0)."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor, outer: int, k: int):
        self.codes, self.scales, self.outer, self.k = codes, scales, int(outer), int(k)

    @classmethod
    def empty(cls, outer: int, k: int, device=None) -> "MXFP4Tensor":
        device = device if device is not None else torch.device("cuda", torch.cuda.current_device())
        return cls(torch.empty((outer, k // 2), dtype=torch.uint8, device=device),
                   torch.empty((outer, k // 32), dtype=torch.uint8, device=device), outer, k)

    @property
    def device(self) -> torch.device:
        return self.codes.device

    def _c(self) -> _MXTensor:
        if self.outer < 0 or self.k < 0 or self.k % 32:
            raise NVFP4Error(f"invalid MXFP4 shape ({self.outer}, {self.k})")
        dev = self.codes.device
        _require_buffer(self.codes, "codes", torch.uint8, self.outer * (self.k // 2), dev)
        _require_buffer(self.scales, "scales", torch.uint8, self.outer * (self.k // 32), dev)
        return _MXTensor(self.codes.data_ptr(), self.scales.data_ptr(), self.outer, self.k)


def mxfp4_quantize(x: torch.Tensor, axis: int = 1, out: MXFP4Tensor | None = None, stream=None) -> MXFP4Tensor:
    """Quantize a 2-D f32/bf16 GPU tensor to MXFP4 (see include/nvfp4.h)."""
    _require_device(x, "x")
    if x.dim() != 2 or not x.is_contiguous():
        raise NVFP4Error("x must be a contiguous 2-D tensor")
    rows, cols = x.shape
    outer, k = (rows, cols) if axis == 1 else (cols, rows)
    if out is None:
        out = MXFP4Tensor.empty(outer, k, device=x.device)
    _same_device(out, x)
    ct = out._c()
    with torch.cuda.device(x.device):
        _check(lib().mxfp4_quantize(x.data_ptr(), _dtype_code(x), rows, cols, axis, ctypes.byref(ct),
                                    _stream_handle(stream, x.device)), "mxfp4_quantize")
    return out


def mxfp4_gemm(a: MXFP4Tensor, b: MXFP4Tensor, out_dtype=torch.float32, out: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
    """C = A . B^T for MXFP4 A [M, K] and B [N, K] (K % 256 == 0), f32 accumulation."""
    code = _out_code(out_dtype)
    dev = a.device
    if b.device != dev:
        raise NVFP4Error(f"operands on {a.device} and {b.device}")
    if out is None:
        out = torch.empty((a.outer, b.outer), dtype=out_dtype, device=dev)
    ldc = _require_matrix_out(out, a.outer, b.outer, out_dtype, dev)
    ca, cb = a._c(), b._c()
    with torch.cuda.device(dev):
        _check(lib().mxfp4_gemm(ctypes.byref(ca), ctypes.byref(cb), out.data_ptr(), code, ldc,
                                _stream_handle(stream, dev)), "mxfp4_gemm")
    return out



class MXFP8Tensor:
    """Device buffers of one MXFP8 tensor in its quantized [outer][k] layout:
    ``codes`` u8 [outer, k] (E4M3), ``scales`` u8 [outer, k/32] (E8M0).  The
    C struct has the same fields as the MXFP4 one."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor, outer: int, k: int):
        self.codes, self.scales, self.outer, self.k = codes, scales, int(outer), int(k)

    @classmethod
    def empty(cls, outer: int, k: int, device=None) -> "MXFP8Tensor":
        device = device if device is not None else torch.device("cuda", torch.cuda.current_device())
        return cls(torch.empty((outer, k), dtype=torch.uint8, device=device),
                   torch.empty((outer, k // 32), dtype=torch.uint8, device=device), outer, k)

    @property
    def device(self) -> torch.device:
        return self.codes.device

    def _c(self) -> _MXTensor:
        if self.outer < 0 or self.k < 0 or self.k % 32:
            raise NVFP4Error(f"invalid MXFP8 shape ({self.outer}, {self.k})")
        dev = self.codes.device
        _require_buffer(self.codes, "codes", torch.uint8, self.outer * self.k, dev)
        _require_buffer(self.scales, "scales", torch.uint8, self.outer * (self.k // 32), dev)
        return _MXTensor(self.codes.data_ptr(), self.scales.data_ptr(), self.outer, self.k)


def mxfp8_quantize(x: torch.Tensor, axis: int = 1, out: MXFP8Tensor | None = None, stream=None) -> MXFP8Tensor:
    """Quantize a 2-D f32/bf16 GPU tensor to MXFP8 (see include/nvfp4.h)."""
    _require_device(x, "x")
    if x.dim() != 2 or not x.is_contiguous():
        raise NVFP4Error("x must be a contiguous 2-D tensor")
    rows, cols = x.shape
    outer, k = (rows, cols) if axis == 1 else (cols, rows)
    if out is None:
        out = MXFP8Tensor.empty(outer, k, device=x.device)
    _same_device(out, x)
    ct = out._c()
    with torch.cuda.device(x.device):
        _check(lib().mxfp8_quantize(x.data_ptr(), _dtype_code(x), rows, cols, axis, ctypes.byref(ct),
                                    _stream_handle(stream, x.device)), "mxfp8_quantize")
    return out


def mxfp8_gemm(a: MXFP8Tensor, b: MXFP8Tensor, out_dtype=torch.float32, out: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
    """C = A . B^T for MXFP8 A [M, K] and B [N, K] (K % 128 == 0), f32 accumulation."""
    code = _out_code(out_dtype)
    dev = a.device
    if b.device != dev:
        raise NVFP4Error(f"operands on {a.device} and {b.device}")
    if out is None:
        out = torch.empty((a.outer, b.outer), dtype=out_dtype, device=dev)
    ldc = _require_matrix_out(out, a.outer, b.outer, out_dtype, dev)
    ca, cb = a._c(), b._c()
    with torch.cuda.device(dev):
        _check(lib().mxfp8_gemm(ctypes.byref(ca), ctypes.byref(cb), out.data_ptr(), code, ldc,
                                _stream_handle(stream, dev)), "mxfp8_gemm")
    return out

"""CPU oracle for the NVFP4 linear-layer path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never does, and
this package imports nothing from the product.

The quantizer, dequantizer and exact decode live in plain C
(``nvfp4_oracle.c``, loaded with ctypes); the GEMM oracle is the plain
definition written with a library matmul in float64:

    C[m, n] = g_A * g_B * sum_k (q_A S_A)[m, k] * (q_B S_B)[n, k]

where q*S is the exactly decoded element (an NVFP4 element times its E4M3
block scale), g is the per-tensor FP32 decode scale, and the pages' source is
the NVFP4 format description ([P4] aisight.pl "Koniec marnowania mocy ...",
section "Architektura NVFP4 kontra ograniczenia mikroskalowania": 16-element
blocks, E4M3 block scale, an FP32 tensor-level scale) together with the
accelerated GEMM the format feeds ([P1] hyper.ai "NVIDIA revolutioniert
KI-Praetrainingsgeschwindigkeit mit 4-Bit-Genauigkeit", body).

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against worked examples, closed forms, library routines and brute force.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
# NVFP4_ORACLE_SANITIZE=1 selects a build instrumented with AddressSanitizer
# and UndefinedBehaviorSanitizer (the process must preload gcc's libasan);
# tests/test_oracle_sanitized.py runs the oracle pins that way.
SANITIZE = os.environ.get("NVFP4_ORACLE_SANITIZE") == "1"
_LIB_PATH = os.path.join(_HERE, "liboracle_san.so" if SANITIZE else "liboracle.so")
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]

F32, BF16 = 0, 1
RNE, SR = 0, 1


def build(force: bool = True, sanitize: bool = SANITIZE) -> str:
    """Compile the oracle's C code with gcc (OpenMP, no FP contraction) into
    ``liboracle.so``, or with ``sanitize`` into ``liboracle_san.so`` with
    AddressSanitizer and UndefinedBehaviorSanitizer (any finding aborts)."""
    path = os.path.join(_HERE, "liboracle_san.so" if sanitize else "liboracle.so")
    if not force and os.path.exists(path):
        return path
    tmp = path + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2" if not sanitize else "-O1", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-Wextra",
           *(SANITIZE_FLAGS if sanitize else []), "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, path)
    return path


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        c_i64, c_u64, c_u32, vp = ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p
        L.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
        L.oracle_e2m1_value.restype = ctypes.c_float
        L.oracle_e2m1_rne.argtypes = [ctypes.c_float]
        L.oracle_e2m1_rne.restype = ctypes.c_uint8
        L.oracle_e2m1_sr.argtypes = [ctypes.c_float, c_u32]
        L.oracle_e2m1_sr.restype = ctypes.c_uint8
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_value.restype = ctypes.c_float
        L.oracle_e4m3_rne_sat.argtypes = [ctypes.c_float]
        L.oracle_e4m3_rne_sat.restype = ctypes.c_uint8
        L.oracle_philox4x32_10.argtypes = [vp, vp, vp]
        L.oracle_philox4x32_10.restype = None
        L.oracle_sr_bits.argtypes = [c_u64, c_u64, c_u64]
        L.oracle_sr_bits.restype = c_u32
        L.oracle_rht16.argtypes = [vp, c_u32, vp]
        L.oracle_rht16.restype = None
        L.oracle_quantize.argtypes = [vp, ctypes.c_int, c_i64, c_i64, ctypes.c_int,
                                      ctypes.c_int, c_u64, c_u64, ctypes.c_int, c_u32,
                                      vp, c_i64, vp, vp, vp]
        L.oracle_quantize.restype = ctypes.c_int
        L.oracle_dequantize.argtypes = [vp, vp, vp, c_i64, c_i64, ctypes.c_int, vp]
        L.oracle_dequantize.restype = ctypes.c_int
        L.oracle_decode_qs.argtypes = [vp, vp, c_i64, vp, c_i64, vp]
        L.oracle_decode_qs.restype = ctypes.c_int
        L.oracle_mx_scale_exp.argtypes = [c_u32]
        L.oracle_mx_scale_exp.restype = ctypes.c_int
        L.oracle_mxfp4_quantize.argtypes = [vp, ctypes.c_int, c_i64, c_i64, ctypes.c_int, vp, vp]
        L.oracle_mxfp4_quantize.restype = ctypes.c_int
        L.oracle_mxfp4_decode.argtypes = [vp, vp, c_i64, vp, c_i64, vp]
        L.oracle_mxfp4_decode.restype = ctypes.c_int
        L.oracle_mx8_scale_exp.argtypes = [c_u32]
        L.oracle_mx8_scale_exp.restype = ctypes.c_int
        L.oracle_mxfp8_quantize.argtypes = [vp, ctypes.c_int, c_i64, c_i64, ctypes.c_int, vp, vp]
        L.oracle_mxfp8_quantize.restype = ctypes.c_int
        L.oracle_mxfp8_decode.argtypes = [vp, vp, c_i64, vp, c_i64, vp]
        L.oracle_mxfp8_decode.restype = ctypes.c_int
        L.oracle_mxfp8_trunc_bound.argtypes = [vp, vp, vp, vp, c_i64, vp, c_i64, vp, c_i64, vp]
        L.oracle_mxfp8_trunc_bound.restype = ctypes.c_int
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def num_threads() -> int:
    return int(lib().oracle_num_threads())


# --------------------------------------------------------------------------
# scalar primitives
# --------------------------------------------------------------------------

def e2m1_value(code: int) -> float:
    return float(lib().oracle_e2m1_value(code))


def e2m1_rne(v: float) -> int:
    return int(lib().oracle_e2m1_rne(v))


def e2m1_sr(v: float, r16: int) -> int:
    return int(lib().oracle_e2m1_sr(v, r16))


def e4m3_value(b: int) -> float:
    return float(lib().oracle_e4m3_value(b))


def e4m3_rne_sat(t: float) -> int:
    return int(lib().oracle_e4m3_rne_sat(t))


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32).reshape(4))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32).reshape(2))
    out = np.zeros(4, dtype=np.uint32)
    lib().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sr_bits(seed: int, offset: int, i: int) -> int:
    return int(lib().oracle_sr_bits(seed, offset, i))


def rht16(x, sign_mask: int) -> np.ndarray:
    xv = np.ascontiguousarray(np.asarray(x, dtype=np.float32).reshape(16))
    y = np.zeros(16, dtype=np.float32)
    lib().oracle_rht16(_ptr(xv), sign_mask & 0xFFFF, _ptr(y))
    return y


# --------------------------------------------------------------------------
# tensors
# --------------------------------------------------------------------------

class Quantized:
    """Oracle result: codes [outer][K/2] u8, scales [outer][K/16] u8, meta f32[2]."""

    def __init__(self, codes, scales, meta, outer, k):
        self.codes, self.scales, self.meta = codes, scales, meta
        self.outer, self.k = outer, k

    @property
    def amax(self) -> float:
        return float(self.meta[0])

    @property
    def g(self) -> float:
        return float(self.meta[1])


def _as_raw(x):
    """Accept a numpy f32 array, a numpy uint16 array of bf16 bits, or a torch
    CPU tensor (float32 / bfloat16).  Returns (array, dtype code)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            t = x.detach().cpu().contiguous()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16), BF16
            if t.dtype == torch.float32:
                return t.numpy(), F32
            raise TypeError(f"unsupported dtype {t.dtype}")
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(x)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError(f"unsupported dtype {a.dtype}")


def quantize(x, axis: int = 1, rounding: int = RNE, seed: int = 0, offset: int = 0,
             rht: bool = False, sign_mask: int = 0, amax=None, outer0: int = 0) -> Quantized:
    """amax: None (computed, step 2) or a supplied tensor amax (float32).
    outer0: global index of x's first output row when x is a slice of a
    larger tensor (shifts the SR element index only)."""
    a, dt = _as_raw(x)
    a = np.ascontiguousarray(a)
    rows, cols = a.shape
    outer, K = (rows, cols) if axis else (cols, rows)
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    codes = np.zeros((outer, K // 2), dtype=np.uint8)
    scales = np.zeros((outer, K // 16), dtype=np.uint8)
    meta = np.zeros(2, dtype=np.float32)
    amax_in = None if amax is None else np.array([amax], dtype=np.float32)
    rc = lib().oracle_quantize(_ptr(a), dt, rows, cols, axis, rounding, seed, offset,
                               1 if rht else 0, sign_mask & 0xFFFF,
                               None if amax_in is None else _ptr(amax_in), int(outer0),
                               _ptr(codes), _ptr(scales), _ptr(meta))
    if rc != 0:
        raise ValueError(f"oracle_quantize failed: {rc}")
    return Quantized(codes, scales, meta, outer, K)


def dequantize(q: Quantized, y_dtype: int = F32) -> np.ndarray:
    out = np.zeros((q.outer, q.k), dtype=np.float32 if y_dtype == F32 else np.uint16)
    rc = lib().oracle_dequantize(_ptr(q.codes), _ptr(q.scales), _ptr(q.meta),
                                 q.outer, q.k, y_dtype, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_dequantize failed: {rc}")
    return out


def decode_qs(q: Quantized, rows=None) -> np.ndarray:
    """Exact q*S (without g) for the selected outer rows, float64 [n][K]."""
    if rows is None:
        rows = np.arange(q.outer, dtype=np.int64)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = np.zeros((rows.size, q.k), dtype=np.float64)
    rc = lib().oracle_decode_qs(_ptr(q.codes), _ptr(q.scales), q.k, _ptr(rows),
                                rows.size, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_decode_qs failed: {rc}")
    return out


def gemm(qa: Quantized, qb: Quantized, rows=None, cols=None):
    """GEMM oracle C = A B^T on the NVFP4 operands, float64.

    Returns (C, bound) restricted to the selected rows of A (outer index m)
    and rows of B (outer index n).  bound = g_A g_B sum_k |(qS)_A (qS)_B|, the
    scale the tolerance 1e-5 * bound is taken against.
    """
    if qa.k != qb.k:
        raise ValueError("K mismatch")
    da = decode_qs(qa, rows)
    db = decode_qs(qb, cols)
    gg = float(np.float64(qa.meta[1]) * np.float64(qb.meta[1]))
    c = (da @ db.T) * gg
    bound = (np.abs(da) @ np.abs(db).T) * abs(gg)
    return c, bound


def check_gemm_f32(c_gpu: np.ndarray, c_ref: np.ndarray, bound: np.ndarray,
                   rtol: float = 1e-5):
    """Tolerance rule for f32 output: |C - Cref| <= rtol * bound elementwise
    (bound == 0 requires C == 0 exactly).  Returns (ok, worst ratio)."""
    c = np.asarray(c_gpu, dtype=np.float64)
    err = np.abs(c - c_ref)
    lim = rtol * bound
    ok = bool(np.all(err <= lim))
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    return ok, float(np.max(ratio)) if ratio.size else 0.0


def _bf16_rne_of_f64(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (nearest even) via f32; returns float64.

    Used only with values whose f32 rounding cannot change the bf16 result
    interval test (the interval ends are rounded the same way)."""
    import torch
    t = torch.from_numpy(np.asarray(x, dtype=np.float64)).to(torch.bfloat16)
    return t.to(torch.float64).numpy()


def check_gemm_bf16(c_gpu_bf16_as_f64: np.ndarray, c_ref: np.ndarray, bound: np.ndarray,
                    rtol: float = 1e-5):
    """Tolerance rule for bf16 output: bf16(Cref - rtol*bound) <= C <=
    bf16(Cref + rtol*bound) (rounding is monotone)."""
    lo = _bf16_rne_of_f64(c_ref - rtol * bound)
    hi = _bf16_rne_of_f64(c_ref + rtol * bound)
    c = np.asarray(c_gpu_bf16_as_f64, dtype=np.float64)
    ok = bool(np.all((c >= lo) & (c <= hi)))
    return ok, int(np.sum(~((c >= lo) & (c <= hi))))


# --------------------------------------------------------------- MXFP4 ----

class MXQuantized:
    """An MXFP4 tensor in its quantized [outer][k] layout: codes u8
    [outer, k/2] (element 2j in the low nibble), scales u8 [outer, k/32]
    (E8M0: 2^(code - 127))."""

    def __init__(self, codes, scales, outer, k):
        self.codes, self.scales, self.outer, self.k = codes, scales, outer, k


def mx_scale_exp(amax: float) -> int:
    """Exponent e of the MXFP4 block scale for a block maximum amax >= 0."""
    bits = int(np.array([amax], dtype=np.float32).view(np.uint32)[0])
    return lib().oracle_mx_scale_exp(bits)


def mxfp4_quantize(x, axis: int = 1) -> MXQuantized:
    a, dt = _as_raw(x)
    a = np.ascontiguousarray(a)
    rows, cols = a.shape
    outer, K = (rows, cols) if axis else (cols, rows)
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    codes = np.zeros((outer, K // 2), dtype=np.uint8)
    scales = np.zeros((outer, K // 32), dtype=np.uint8)
    rc = lib().oracle_mxfp4_quantize(_ptr(a), dt, rows, cols, axis, _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError(f"oracle_mxfp4_quantize failed: {rc}")
    return MXQuantized(codes, scales, outer, K)


def mxfp4_decode(q: MXQuantized, rows=None) -> np.ndarray:
    """Exact values q * 2^e of the selected outer rows, float64 [n][K]."""
    if rows is None:
        rows = np.arange(q.outer, dtype=np.int64)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = np.zeros((rows.size, q.k), dtype=np.float64)
    rc = lib().oracle_mxfp4_decode(_ptr(q.codes), _ptr(q.scales), q.k, _ptr(rows), rows.size, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_mxfp4_decode failed: {rc}")
    return out


def mxfp4_gemm(qa: MXQuantized, qb: MXQuantized, rows=None, cols=None):
    """C = A B^T of the decoded MXFP4 operands in float64 (every product is
    exact), with bound = sum_k |a b| for the tolerance."""
    if qa.k != qb.k:
        raise ValueError("K mismatch")
    da = mxfp4_decode(qa, rows)
    db = mxfp4_decode(qb, cols)
    return da @ db.T, np.abs(da) @ np.abs(db).T



# --------------------------------------------------------------- MXFP8 ----

class MX8Quantized:
    """An MXFP8 tensor in its quantized [outer][k] layout: codes u8
    [outer, k] (OCP E4M3FN), scales u8 [outer, k/32] (E8M0: 2^(code - 127))."""

    def __init__(self, codes, scales, outer, k):
        self.codes, self.scales, self.outer, self.k = codes, scales, outer, k


def mx8_scale_exp(amax: float) -> int:
    """Exponent e of the MXFP8 block scale for a block maximum amax >= 0."""
    bits = int(np.array([amax], dtype=np.float32).view(np.uint32)[0])
    return lib().oracle_mx8_scale_exp(bits)


def mxfp8_quantize(x, axis: int = 1) -> MX8Quantized:
    a, dt = _as_raw(x)
    a = np.ascontiguousarray(a)
    rows, cols = a.shape
    outer, K = (rows, cols) if axis else (cols, rows)
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    codes = np.zeros((outer, K), dtype=np.uint8)
    scales = np.zeros((outer, K // 32), dtype=np.uint8)
    rc = lib().oracle_mxfp8_quantize(_ptr(a), dt, rows, cols, axis, _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError(f"oracle_mxfp8_quantize failed: {rc}")
    return MX8Quantized(codes, scales, outer, K)


def mxfp8_decode(q: MX8Quantized, rows=None) -> np.ndarray:
    """Exact values e4m3(code) * 2^e of the selected outer rows, float64 [n][K]."""
    if rows is None:
        rows = np.arange(q.outer, dtype=np.int64)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = np.zeros((rows.size, q.k), dtype=np.float64)
    rc = lib().oracle_mxfp8_decode(_ptr(q.codes), _ptr(q.scales), q.k, _ptr(rows), rows.size, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_mxfp8_decode failed: {rc}")
    return out


def mxfp8_gemm(qa: MX8Quantized, qb: MX8Quantized, rows=None, cols=None):
    """GEMM oracle C = A B^T of the decoded MXFP8 operands, float64 (every
    product is exact in float64).  Returns (C, bound) as gemm() does."""
    if qa.k != qb.k:
        raise ValueError("K mismatch")
    da = mxfp8_decode(qa, rows)
    db = mxfp8_decode(qb, cols)
    return da @ db.T, np.abs(da) @ np.abs(db).T


def mxfp8_trunc_bound(qa: MX8Quantized, qb: MX8Quantized, rows=None, cols=None) -> np.ndarray:
    """Per-element bound of what the FP8 block-scaled MFMA loses to its product
    truncation (the C function states the measured reading); the MXFP8 GEMM
    tolerance is this plus rtol * sum|ab|."""
    if qa.k != qb.k:
        raise ValueError("K mismatch")
    ra = np.ascontiguousarray(np.arange(qa.outer) if rows is None else np.asarray(rows), dtype=np.int64)
    rb = np.ascontiguousarray(np.arange(qb.outer) if cols is None else np.asarray(cols), dtype=np.int64)
    out = np.zeros((ra.size, rb.size), dtype=np.float64)
    rc = lib().oracle_mxfp8_trunc_bound(_ptr(qa.codes), _ptr(qa.scales), _ptr(qb.codes), _ptr(qb.scales), qa.k,
                                        _ptr(ra), ra.size, _ptr(rb), rb.size, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_mxfp8_trunc_bound failed: {rc}")
    return out


def check_gemm_mx8_f32(c_gpu: np.ndarray, c_ref: np.ndarray, bound: np.ndarray, trunc: np.ndarray,
                       rtol: float = 1e-5):
    """MXFP8 tolerance rule for f32 output: |C - Cref| <= trunc + rtol * bound
    elementwise.  Returns (ok, worst |err| / (trunc + rtol * bound), worst
    |err| / bound)."""
    c = np.asarray(c_gpu, dtype=np.float64)
    err = np.abs(c - c_ref)
    lim = trunc + rtol * bound
    ok = bool(np.all(err <= lim))
    with np.errstate(divide="ignore", invalid="ignore"):
        r1 = np.where(lim > 0, err / np.where(lim > 0, lim, 1.0), np.where(err > 0, np.inf, 0.0))
        r2 = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    return ok, float(np.max(r1)) if r1.size else 0.0, float(np.max(r2)) if r2.size else 0.0

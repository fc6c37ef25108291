"""The C-ABI library loads, exports every symbol include/nvfp4.h declares, and
reports argument errors synchronously, before anything is launched (so these
run without a GPU)."""
import ctypes
import os
import re

import pytest

import gemm_amax_reduce_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:nvfp4|mxfp4|mxfp8)_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(nv.LIB_PATH):
        pytest.fail("libnvfp4.so not built (run __graft_entry__.build())")
    return nv.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert set(names) == set(nv.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4, -5):
        assert L.nvfp4_status_string(code)
    assert L.nvfp4_status_string(12345) == b"unknown status"


FAKE = 0x10000  # a 16-byte-aligned non-null address; never dereferenced

# Every call below passes at least one invalid argument, so validation must
# return before any launch.  The fake device addresses would fault a real
# GPU if a validation bug let a launch through, so these tests only run
# where no GPU is visible.
_no_gpu = pytest.mark.skipif(__import__("torch").cuda.is_available(),
                             reason="fake-pointer argument tests run only without a GPU")


def _t(outer, k, codes=FAKE, scales=FAKE, meta=FAKE):
    return nv._CTensor(codes, scales, meta, outer, k)


@_no_gpu
def test_quantize_argument_errors(L):
    q = _t(16, 32)
    by = ctypes.byref
    assert L.nvfp4_quantize(FAKE, 1, 16, 32, 1, 0, 0, 0, None, None) == -1      # out NULL
    assert L.nvfp4_quantize(FAKE, 2, 16, 32, 1, 0, 0, 0, by(q), None) == -3     # dtype
    assert L.nvfp4_quantize(FAKE, 1, 16, 32, 1, 7, 0, 0, by(q), None) == -3     # rounding
    assert L.nvfp4_quantize(FAKE, 1, 16, 32, 2, 0, 0, 0, by(q), None) == -3     # axis
    assert L.nvfp4_quantize(FAKE, 1, -1, 32, 1, 0, 0, 0, by(q), None) == -2     # negative
    q24 = _t(16, 24)
    assert L.nvfp4_quantize(FAKE, 1, 16, 24, 1, 0, 0, 0, by(q24), None) == -2   # K % 16
    assert L.nvfp4_quantize(FAKE, 1, 16, 48, 1, 0, 0, 0, by(q), None) == -2     # out shape
    assert L.nvfp4_quantize(FAKE, 1, 16, 32, 0, 0, 0, 0, by(q), None) == -2     # axis-0 view is 32x16
    assert L.nvfp4_quantize(None, 1, 16, 32, 1, 0, 0, 0, by(q), None) == -1     # x NULL
    assert L.nvfp4_quantize(FAKE + 2, 1, 16, 32, 1, 0, 0, 0, by(q), None) == -5 # x misaligned
    qn = _t(16, 32, meta=0)
    assert L.nvfp4_quantize(FAKE, 1, 16, 32, 1, 0, 0, 0, by(qn), None) == -1    # meta NULL
    qa = _t(16, 32, codes=FAKE + 4)
    assert L.nvfp4_quantize(FAKE, 1, 16, 32, 1, 0, 0, 0, by(qa), None) == -5    # codes misaligned
    assert L.nvfp4_rht_quantize(FAKE, 1, 16, 24, 1, 0, 0, 0, 0xFFFF, by(q24), None) == -2


@_no_gpu
def test_dequantize_argument_errors(L):
    by = ctypes.byref
    assert L.nvfp4_dequantize(None, FAKE, 0, None) == -1
    assert L.nvfp4_dequantize(by(_t(16, 24)), FAKE, 0, None) == -2
    assert L.nvfp4_dequantize(by(_t(16, 32)), FAKE, 5, None) == -3
    assert L.nvfp4_dequantize(by(_t(16, 32)), None, 0, None) == -1
    assert L.nvfp4_dequantize(by(_t(16, 32)), FAKE + 8, 0, None) == -5


@_no_gpu
def test_gemm_argument_errors(L):
    by = ctypes.byref
    a, b = _t(8, 32), _t(4, 32)
    assert L.nvfp4_gemm(None, by(b), FAKE, 0, 4, None) == -1
    assert L.nvfp4_gemm(by(a), by(_t(4, 48)), FAKE, 0, 4, None) == -2     # K mismatch
    assert L.nvfp4_gemm(by(a), by(b), FAKE, 3, 4, None) == -3             # dtype
    assert L.nvfp4_gemm(by(a), by(b), FAKE, 0, 3, None) == -2             # ldc < N
    assert L.nvfp4_gemm(by(a), by(b), None, 0, 4, None) == -1             # C NULL
    assert L.nvfp4_gemm(by(a), by(b), FAKE + 2, 0, 4, None) == -5         # C misaligned (f32)
    assert L.nvfp4_gemm(by(_t(-1, 32)), by(b), FAKE, 0, 4, None) == -2
    # K % 64 == 0: scale rows move by DMA in whole dwords, so scales must be
    # 4-byte aligned; other K read them byte by byte (any alignment)
    a64, b64 = _t(8, 64, scales=FAKE + 1), _t(4, 64)
    assert L.nvfp4_gemm(by(a64), by(b64), FAKE, 0, 4, None) == -5
    assert L.nvfp4_gemm(by(_t(8, 64)), by(_t(4, 64, scales=FAKE + 2)), FAKE, 0, 4, None) == -5
    assert L.nvfp4_gemm(by(_t(8, 48, scales=FAKE + 1)), by(_t(4, 48)), None, 0, 4, None) == -1  # not an ALIGN error


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(nv.NVFP4Error, match="GPU"):
        nv.nvfp4_quantize(torch.zeros(16, 32))


@_no_gpu
def test_gemm_ws_argument_errors(L):
    by = ctypes.byref
    a, b = _t(64, 64), _t(32, 64)
    need = L.nvfp4_gemm_workspace_bytes()
    assert need == (64 << 10) + 256 * (256 << 10)
    call = L.nvfp4_gemm_ws
    assert call(None, by(b), FAKE, 0, 32, FAKE, need, None) == -1           # a NULL
    assert call(by(a), by(b), FAKE, 0, 32, None, need, None) == -1          # workspace NULL
    assert call(by(a), by(b), FAKE, 0, 32, FAKE, need - 1, None) == -2      # workspace too small
    assert call(by(a), by(b), FAKE, 0, 32, FAKE + 16, need, None) == -5     # workspace misaligned
    assert call(by(a), by(b), FAKE, 7, 32, FAKE, need, None) == -3          # dtype
    assert call(by(a), by(b), FAKE, 0, 31, FAKE, need, None) == -2          # ldc < N
    assert call(by(a), by(_t(32, 48)), FAKE, 0, 32, FAKE, need, None) == -2 # K mismatch


@_no_gpu
def test_quantize_dual_argument_errors(L):
    by = ctypes.byref
    q1, q0 = _t(16, 32), _t(32, 16, meta=FAKE + 64)
    call = L.nvfp4_quantize_dual
    assert call(FAKE, 1, 16, 32, 0, 0, 0, None, 0, 0, 0, 0, 0, by(q0), None) == -1       # out1 NULL
    assert call(FAKE, 1, 16, 32, 0, 0, 0, by(q1), 0, 0, 0, 0, 0, None, None) == -1       # out0 NULL
    assert call(FAKE, 9, 16, 32, 0, 0, 0, by(q1), 0, 0, 0, 0, 0, by(q0), None) == -3     # dtype
    assert call(FAKE, 1, 16, 32, 5, 0, 0, by(q1), 0, 0, 0, 0, 0, by(q0), None) == -3     # rounding1
    assert call(FAKE, 1, 16, 32, 0, 0, 0, by(q1), 0, 0, 5, 0, 0, by(q0), None) == -3     # rounding0
    assert call(FAKE, 1, 16, 32, 0, 0, 0, by(q1), 2, 0, 0, 0, 0, by(q0), None) == -3     # rht0
    q1b, q0b = _t(24, 32), _t(32, 24, meta=FAKE + 64)
    assert call(FAKE, 1, 24, 32, 0, 0, 0, by(q1b), 0, 0, 0, 0, 0, by(q0b), None) == -2   # rows % 16
    assert call(FAKE, 1, 16, 32, 0, 0, 0, by(q0), 0, 0, 0, 0, 0, by(q1), None) == -2     # swapped outputs
    qsame = _t(32, 16)
    assert call(FAKE, 1, 16, 32, 0, 0, 0, by(q1), 0, 0, 0, 0, 0, by(qsame), None) == -2  # shared meta
    # overlapping meta pairs: out0's {amax, g} one float after out1's, and before it
    for m0 in (FAKE + 4, FAKE - 4):
        qover = _t(32, 16, meta=m0)
        assert call(FAKE, 1, 16, 32, 0, 0, 0, by(q1), 0, 0, 0, 0, 0, by(qover), None) == -2
    assert call(None, 1, 16, 32, 0, 0, 0, by(q1), 0, 0, 0, 0, 0, by(q0), None) == -1     # x NULL
    assert call(FAKE + 2, 1, 16, 32, 0, 0, 0, by(q1), 0, 0, 0, 0, 0, by(q0), None) == -5 # x misaligned


@_no_gpu
def test_amax_and_quantize_amax_argument_errors(L):
    by = ctypes.byref
    assert L.nvfp4_amax(FAKE, 1, 16, 32, 1, 0, 0, None, None) == -1           # amax NULL
    assert L.nvfp4_amax(FAKE, 4, 16, 32, 1, 0, 0, FAKE, None) == -3           # dtype
    assert L.nvfp4_amax(FAKE, 1, 16, 32, 3, 0, 0, FAKE, None) == -3           # axis
    assert L.nvfp4_amax(FAKE, 1, 16, 32, 1, 2, 0, FAKE, None) == -3           # rht
    assert L.nvfp4_amax(FAKE, 1, 16, 24, 1, 0, 0, FAKE, None) == -2           # K % 16 (axis 1: cols)
    assert L.nvfp4_amax(FAKE, 1, 24, 32, 0, 0, 0, FAKE, None) == -2           # K % 16 (axis 0: rows)
    assert L.nvfp4_amax(None, 1, 16, 32, 1, 0, 0, FAKE, None) == -1           # x NULL
    assert L.nvfp4_amax(FAKE, 1, 16, 32, 1, 0, 0, FAKE + 2, None) == -5       # amax misaligned
    q = _t(16, 32)
    call = L.nvfp4_quantize_amax
    assert call(FAKE, 1, 16, 32, 1, 0, 0, 0, 0, 0, None, by(q), None) == -1   # amax NULL
    assert call(FAKE, 1, 16, 32, 1, 0, 0, 0, 0, 0, FAKE, None, None) == -1    # out NULL
    assert call(FAKE, 1, 16, 32, 1, 3, 0, 0, 0, 0, FAKE, by(q), None) == -3   # rounding
    assert call(FAKE, 1, 16, 32, 1, 0, 0, 0, 5, 0, FAKE, by(q), None) == -3   # rht
    assert call(FAKE, 1, 16, 32, 0, 0, 0, 0, 0, 0, FAKE, by(q), None) == -2   # axis-0 view is 32x16
    assert call(FAKE, 1, 16, 32, 1, 0, 0, 0, 0, 0, FAKE + 1, by(q), None) == -5


def _mx(outer, k, codes=FAKE, scales=FAKE):
    return nv._MXTensor(codes, scales, outer, k)


@_no_gpu
def test_mxfp4_argument_errors(L):
    by = ctypes.byref
    q = _mx(16, 64)
    assert L.mxfp4_quantize(FAKE, 1, 16, 64, 1, None, None) == -1          # out NULL
    assert L.mxfp4_quantize(FAKE, 7, 16, 64, 1, by(q), None) == -3         # dtype
    assert L.mxfp4_quantize(FAKE, 1, 16, 64, 2, by(q), None) == -3         # axis
    q48 = _mx(16, 48)
    assert L.mxfp4_quantize(FAKE, 1, 16, 48, 1, by(q48), None) == -2       # K % 32
    assert L.mxfp4_quantize(FAKE, 1, 16, 64, 0, by(q), None) == -2         # axis-0 view is 64x16
    assert L.mxfp4_quantize(FAKE + 8, 1, 16, 64, 1, by(q), None) == -5     # x misaligned
    assert L.mxfp4_quantize(FAKE, 1, 16, 64, 1, by(_mx(16, 64, codes=FAKE + 8)), None) == -5
    a, b = _mx(8, 256), _mx(4, 256)
    assert L.mxfp4_gemm(None, by(b), FAKE, 0, 4, None) == -1
    assert L.mxfp4_gemm(by(a), by(_mx(4, 512)), FAKE, 0, 4, None) == -2    # K mismatch
    assert L.mxfp4_gemm(by(_mx(8, 96)), by(_mx(4, 96)), FAKE, 0, 4, None) == -2   # K % 256
    assert L.mxfp4_gemm(by(a), by(b), FAKE, 2, 4, None) == -3              # dtype
    assert L.mxfp4_gemm(by(a), by(b), FAKE, 0, 3, None) == -2              # ldc < N
    assert L.mxfp4_gemm(by(a), by(b), None, 0, 4, None) == -1              # c NULL
    assert L.mxfp4_gemm(by(_mx(8, 256, codes=FAKE + 8)), by(b), FAKE, 0, 4, None) == -5   # codes: 16 B
    assert L.mxfp4_gemm(by(a), by(_mx(4, 256, scales=FAKE + 2)), FAKE, 0, 4, None) == -5  # scales: 4 B


@_no_gpu
def test_size_limits_are_shape_errors(L):
    """Sizes beyond the documented launch-geometry limits are refused before
    anything is launched (NVFP4_ERR_SHAPE)."""
    by = ctypes.byref
    rows = 4194240 + 16                                  # axis 0: rows <= 4 194 240
    q0 = _t(16, rows)
    assert L.nvfp4_quantize(FAKE, 1, rows, 16, 0, 0, 0, 0, by(q0), None) == -2
    assert L.nvfp4_rht_quantize(FAKE, 1, rows, 16, 0, 0, 0, 0, 0, by(q0), None) == -2
    assert L.nvfp4_amax(FAKE, 1, rows, 16, 0, 0, 0, FAKE, None) == -2
    assert L.nvfp4_quantize_amax(FAKE, 1, rows, 16, 0, 0, 0, 0, 0, 0, FAKE, by(q0), None) == -2
    q1 = _t(rows, 16)
    assert L.nvfp4_quantize_dual(FAKE, 1, rows, 16, 0, 0, 0, by(q1), 0, 0, 0, 0, 0,
                                 by(_t(16, rows, meta=FAKE + 64)), None) == -2
    mrows = 16776960 + 32                                # MXFP4 axis 0: rows <= 16 776 960
    assert L.mxfp4_quantize(FAKE, 1, mrows, 64, 0, by(_mx(64, mrows)), None) == -2
    k = 1 << 25                                          # GEMM: K <= 2^25 - 16
    assert L.nvfp4_gemm(by(_t(4, k)), by(_t(4, k)), FAKE, 0, 4, None) == -2
    assert L.mxfp4_gemm(by(_mx(4, k)), by(_mx(4, k)), FAKE, 0, 4, None) == -2
    big = 1 << 40                                        # more tiles than a grid holds
    assert L.nvfp4_gemm(by(_t(big, 16)), by(_t(big, 16)), FAKE, 0, big, None) == -2
    # element counts above 2^60 (rows * cols, outer * k, M * ldc)
    r = c = 1 << 31
    assert L.nvfp4_quantize(FAKE, 1, r, c, 1, 0, 0, 0, by(_t(r, c)), None) == -2
    assert L.nvfp4_amax(FAKE, 1, r, c, 1, 0, 0, FAKE, None) == -2
    assert L.nvfp4_quantize_amax(FAKE, 1, r, c, 1, 0, 0, 0, 0, 0, FAKE, by(_t(r, c)), None) == -2
    assert L.nvfp4_quantize_dual(FAKE, 1, r, c, 0, 0, 0, by(_t(r, c)), 0, 0, 0, 0, 0,
                                 by(_t(c, r, meta=FAKE + 64)), None) == -2
    assert L.mxfp4_quantize(FAKE, 1, r, c, 1, by(_mx(r, c)), None) == -2
    assert L.nvfp4_dequantize(by(_t(r, c)), FAKE, 0, None) == -2
    assert L.nvfp4_gemm(by(_t(1 << 20, 16)), by(_t(4, 16)), FAKE, 0, 1 << 41, None) == -2
    assert L.mxfp4_gemm(by(_mx(1 << 20, 256)), by(_mx(4, 256)), FAKE, 0, 1 << 41, None) == -2


@_no_gpu
def test_probe_argument_errors(L):
    assert L.nvfp4_probe_mfma(10, None, None) == -1
    assert L.nvfp4_probe_mfma(-1, FAKE, None) == -2
    assert L.nvfp4_probe_mfma(10, FAKE + 2, None) == -5
    assert L.nvfp4_probe_philox(10, None, None) == -1
    assert L.nvfp4_probe_philox(-1, FAKE, None) == -2
    assert L.nvfp4_probe_philox(10, FAKE + 2, None) == -5


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs on one GPU only: --gpus above 1 exits with a message
    before touching a device."""
    import json
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]

"""GPU parity of the quantizer and dequantizer against the CPU oracle.

Bit-exact on codes, scales and meta for every rounding mode, transform,
axis and input dtype, at small ragged sizes, at edge cases and on the full
workload tensors.  The GPU path is called through the C ABI (the ctypes
binding of libnvfp4.so).
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

MASK = workloads.rht_sign_mask()


@functools.lru_cache(maxsize=None)
def _nv():
    import gemm_amax_reduce_amd as nv
    nv.lib()
    return nv


def _gpu_quant(x, axis, rounding, seed=0, offset=0, rht=False, mask=MASK):
    nv = _nv()
    xd = x.cuda()
    if rht:
        q = nv.nvfp4_rht_quantize(xd, mask, axis=axis, rounding=rounding, seed=seed, offset=offset)
    else:
        q = nv.nvfp4_quantize(xd, axis=axis, rounding=rounding, seed=seed, offset=offset)
    torch.cuda.synchronize()
    return q


def _assert_same(q, ref, label=""):
    codes = q.codes.cpu().numpy()
    scales = q.scales.cpu().numpy()
    meta = q.meta.cpu().numpy()
    np.testing.assert_array_equal(meta.view(np.uint32), ref.meta.view(np.uint32), err_msg=f"meta {label}")
    np.testing.assert_array_equal(scales, ref.scales, err_msg=f"scales {label}")
    if not np.array_equal(codes, ref.codes):
        bad = np.argwhere(codes != ref.codes)
        o, j = bad[0]
        raise AssertionError(f"codes differ {label}: {len(bad)} bytes, first at outer={o} byte={j}: "
                             f"gpu={codes[o, j]:02x} oracle={ref.codes[o, j]:02x}")


def _check(x, axis, rounding, seed=0, offset=0, rht=False, label=""):
    print(f"[quantize] {label} shape={tuple(x.shape)} dtype={x.dtype} axis={axis} rounding={rounding} rht={rht}",
          flush=True)
    r = oracle.SR if rounding == "sr" else oracle.RNE
    ref = oracle.quantize(x, axis=axis, rounding=r, seed=seed, offset=offset, rht=rht, sign_mask=MASK)
    q = _gpu_quant(x, axis, rounding, seed, offset, rht)
    _assert_same(q, ref, label)
    return q, ref


VARIANTS = [("rne", False), ("sr", False), ("rne", True), ("sr", True)]


@pytest.mark.parametrize("rounding,rht", VARIANTS)
@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_small_ragged(rounding, rht, axis, dtype):
    # several workgroups' worth of blocks plus ragged tails in both dims
    rows, cols = (208, 176) if axis == 1 else (176, 203)
    x = workloads.with_outliers(workloads.normal(rows, cols, 101), 102, p=0.01)
    x = workloads.to_bf16(x) if dtype == "bf16" else torch.from_numpy(x)
    _check(x, axis, rounding, seed=0x1234, offset=5, rht=rht, label=f"small {dtype}")


@pytest.mark.parametrize("axis", [0, 1])
def test_tiny_config(axis):
    g = workloads.TINY
    op = g.a if axis == 1 else g.b
    _check(op.generate(), op.axis, "rne", label="tiny")


def test_edge_values():
    # zeros, negative zeros, subnormals, huge values, exact grid points,
    # midpoints, and a zero block inside a nonzero tensor
    rng = np.random.default_rng(5)
    x = np.zeros((64, 64), dtype=np.float32)
    x[0] = -0.0
    x[1] = np.float32(1e-40) * rng.standard_normal(64).astype(np.float32)
    x[2] = rng.standard_normal(64).astype(np.float32) * 1e30
    x[3] = np.tile(np.array([6, 3.2, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -5, -3.5, -0.25, 4, 2, 1, 0.5],
                            dtype=np.float32), 4)
    x[4:] = rng.standard_normal((60, 64)).astype(np.float32) * np.exp2(rng.integers(-30, 30, (60, 1))).astype(np.float32)
    x[10, 16:32] = 0.0
    for axis in (0, 1):
        for rounding in ("rne", "sr"):
            for rht in (False, True):
                _check(torch.from_numpy(x), axis, rounding, seed=3, rht=rht, label="edges")


def test_zero_tensor_and_empty():
    _check(torch.zeros((32, 48), dtype=torch.bfloat16), 1, "rne", label="zeros")
    nv = _nv()
    for shape, axis in (((0, 32), 1), ((32, 0), 1), ((0, 7), 0), ((16, 0), 0)):
        print(f"[quantize] empty {shape} axis={axis}", flush=True)
        x = torch.zeros(shape, dtype=torch.float32, device="cuda")
        q = nv.nvfp4_quantize(x, axis=axis)
        torch.cuda.synchronize()
        assert q.meta.cpu().tolist() == [0.0, 0.0]


def test_nonfinite_meta():
    x = torch.ones((32, 64))
    x[3, 7] = float("inf")
    q = _gpu_quant(x, 1, "rne")
    assert np.isinf(q.meta[0].item())
    x[5, 9] = float("nan")
    q = _gpu_quant(x, 1, "rne")
    assert np.isnan(q.meta[0].item())


def test_argument_errors_are_synchronous():
    nv = _nv()
    x = torch.zeros((16, 24), device="cuda")
    with pytest.raises(nv.NVFP4Error, match="shape"):
        nv.nvfp4_quantize(x)  # K = 24 is not a multiple of 16
    with pytest.raises(nv.NVFP4Error, match="misaligned"):
        nv.nvfp4_quantize(torch.zeros(16 * 33, device="cuda")[1:1 + 16 * 32].view(16, 32))


def test_deterministic():
    x = workloads.to_bf16(workloads.normal(256, 512, 77))
    a = _gpu_quant(x, 1, "sr", seed=9, rht=True)
    b = _gpu_quant(x, 1, "sr", seed=9, rht=True)
    assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)


# -------------------------------------------------------------- dequantize --

@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_dequantize_bit_exact(out):
    nv = _nv()
    x = workloads.to_bf16(workloads.mixed_rows(96, 320, 55))
    ref = oracle.quantize(x, axis=1)
    q = nv.NVFP4Tensor(torch.from_numpy(ref.codes).cuda(), torch.from_numpy(ref.scales).cuda(),
                       torch.from_numpy(ref.meta).cuda(), ref.outer, ref.k)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    y = nv.nvfp4_dequantize(q, dt)
    torch.cuda.synchronize()
    exp = oracle.dequantize(ref, oracle.F32 if out == "f32" else oracle.BF16)
    got = y.cpu().view(torch.int32 if out == "f32" else torch.int16).numpy()
    np.testing.assert_array_equal(got.view(exp.dtype), exp)


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1, 16), (3, 48), (4096, 5120)], ids=["1x16", "3x48", "4096x5120"])
def test_dequantize_sizes(out, shape):
    """One block, an odd number of blocks, and a layer-sized operand (grid
    far above one round of the CUs), bit-exact against the oracle."""
    nv = _nv()
    rows, cols = shape
    x = workloads.to_bf16(workloads.normal(rows, cols, 57 + rows))
    ref = oracle.quantize(x, axis=1)
    q = nv.NVFP4Tensor(torch.from_numpy(ref.codes).cuda(), torch.from_numpy(ref.scales).cuda(),
                       torch.from_numpy(ref.meta).cuda(), ref.outer, ref.k)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    y = nv.nvfp4_dequantize(q, dt)
    torch.cuda.synchronize()
    exp = oracle.dequantize(ref, oracle.F32 if out == "f32" else oracle.BF16)
    got = y.cpu().view(torch.int32 if out == "f32" else torch.int16).numpy()
    np.testing.assert_array_equal(got.view(exp.dtype), exp)


# ------------------------------------------------------ full workloads ----

FULL = [
    ("fprop X", lambda: workloads.FPROP.a),
    ("fprop W", lambda: workloads.FPROP.b),
    ("dgrad dY", lambda: workloads.DGRAD.a),
    ("dgrad W", lambda: workloads.DGRAD.b),
    ("wgrad X", lambda: workloads.WGRAD.a),
    ("wgrad dY", lambda: workloads.WGRAD.b),
]


@functools.lru_cache(maxsize=4)
def _gen(op):
    return op.generate()


@pytest.mark.parametrize("name,opf", FULL, ids=[f[0] for f in FULL])
def test_full_workload_operand(name, opf):
    op = opf()
    x = _gen(op)
    _check(x, op.axis, op.rounding, seed=workloads.SR_SEED, offset=op.sr_offset, rht=op.rht, label=name)


@pytest.mark.parametrize("rounding,rht", VARIANTS)
def test_full_sweep_tensor(rounding, rht):
    x = _gen(workloads.SWEEP)
    _check(x, 1, rounding, seed=workloads.SR_SEED, rht=rht, label="sweep")

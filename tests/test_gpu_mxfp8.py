"""GPU parity of the MXFP8 path against the CPU oracle, through the C ABI:
the quantizer bit-exact on codes and scales (axis 1 and 0, bf16 and f32,
ragged shapes, subnormal and tied elements, zero blocks), and the GEMM on the
block-scaled FP8 MFMA within its tolerance: per element, the instruction's
truncation bound (oracle.mxfp8_trunc_bound: products truncated to 13 bits
below their group's exponent sum, groups of 8 K positions, as measured on
MI355X) plus 1e-5 * sum|a*b| for the binary32 accumulation.  bf16 outputs
by the rounding interval of that tolerance."""
import functools

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu
RTOL = 1e-5


@functools.lru_cache(maxsize=None)
def _nv():
    import gemm_amax_reduce_amd as nv
    nv.lib()
    return nv


def _x(rows, cols, seed, dtype):
    x = workloads.mixed_rows(rows, cols, seed)
    x[: rows // 4] *= np.float32(1e-3)       # blocks of very different scale
    return torch.from_numpy(x) if dtype == "f32" else workloads.to_bf16(x)


@pytest.mark.parametrize("rows,cols,axis", [(32, 32, 1), (48, 96, 1), (272, 160, 1), (96, 64, 0), (320, 48, 0),
                                            (512, 130, 0), (160, 7, 0)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_matches_oracle(rows, cols, axis, dtype):
    print(f"[mxfp8 quantize] {rows}x{cols} axis={axis} {dtype}", flush=True)
    nv = _nv()
    x = _x(rows, cols, 5, dtype)
    q = nv.mxfp8_quantize(x.cuda(), axis=axis)
    torch.cuda.synchronize()
    ref = oracle.mxfp8_quantize(x, axis=axis)
    np.testing.assert_array_equal(q.scales.cpu().numpy(), ref.scales)
    np.testing.assert_array_equal(q.codes.cpu().numpy(), ref.codes)


def test_quantize_edge_values():
    """Subnormal E4M3 outputs, ties between neighbouring codes, -0.0, tiny
    negatives, an all-zero block, a block at 448 exactly, and maxima near
    the f32 range ends (scales clamped at 2^-127 and large exponents)."""
    nv = _nv()
    x = np.zeros((8, 128), dtype=np.float32)
    x[0, :32] = np.float32(1.0 / 512) * np.arange(-16, 16)        # multiples of the subnormal step
    x[0, 31] = 448.0
    x[1, :32] = (np.arange(32) + 0.5).astype(np.float32) * np.float32(2.0 ** -9)   # ties
    x[1, 0] = 448.0
    x[2, :32] = -1e-30
    x[2, 3] = -0.0
    x[3, 32:64] = 448.0
    x[4, :32] = np.float32(3e-39)                                  # subnormal f32 maxima
    x[5, :32] = np.float32(1e38) * np.linspace(-1, 1, 32, dtype=np.float32)
    x[6] = np.float32(1e-20) * np.arange(128, dtype=np.float32)
    q = nv.mxfp8_quantize(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    ref = oracle.mxfp8_quantize(x)
    np.testing.assert_array_equal(q.scales.cpu().numpy(), ref.scales)
    np.testing.assert_array_equal(q.codes.cpu().numpy(), ref.codes)


def _check(c, ra, rb, out, rows=None, cols=None, label=""):
    cref, bound = oracle.mxfp8_gemm(ra, rb, rows, cols)
    trunc = oracle.mxfp8_trunc_bound(ra, rb, rows, cols)
    if rows is not None:
        c = c[torch.as_tensor(rows)]
    if cols is not None:
        c = c[:, torch.as_tensor(cols)]
    got = c.double().numpy()
    ok, worst_tol, worst_sum = oracle.check_gemm_mx8_f32(got, cref, bound, trunc, RTOL) if out == "f32" else \
        (None, None, None)
    if out == "f32":
        print(f"[mxfp8 gemm] {label}: worst |err|/tolerance = {worst_tol:.3e}, worst |err|/sum|ab| = "
              f"{worst_sum:.3e}", flush=True)
        assert ok, f"{label}: worst |err|/tolerance = {worst_tol:.3e}"
    else:
        # the bf16 interval of the same tolerance: rtol * b_eff = trunc + rtol * bound
        ok, nbad = oracle.check_gemm_bf16(got, cref, bound + trunc / RTOL, RTOL)
        assert ok, f"{label}: {nbad} bf16 outputs outside the tolerance interval"


def _gemm_case(m, n, k, out, seed=1):
    nv = _nv()
    xa, xb = _x(m, k, seed, "bf16"), _x(n, k, seed + 1, "bf16")
    qa, qb = nv.mxfp8_quantize(xa.cuda()), nv.mxfp8_quantize(xb.cuda())
    dt = torch.float32 if out == "f32" else torch.bfloat16
    c = nv.mxfp8_gemm(qa, qb, dt)
    torch.cuda.synchronize()
    _check(c.cpu(), oracle.mxfp8_quantize(xa), oracle.mxfp8_quantize(xb), out, label=f"{m}x{n}x{k} {out}")


@pytest.mark.parametrize("m,n,k", [(256, 256, 128), (200, 136, 256), (257, 129, 128), (1, 1, 128),
                                   (384, 640, 1024), (64, 300, 768), (64, 40000, 128), (96, 80, 20480)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemm_matches_oracle(m, n, k, out):
    print(f"[mxfp8 gemm] {m}x{n}x{k} {out}", flush=True)
    _gemm_case(m, n, k, out)


def test_gemm_truncation_follows_the_k_groups():
    """256 and 0.046875 in one aligned run of 8 K positions lose the
    0.015625 below 2^(8-13); eight positions apart they add exactly.  Checks
    the operand layout keeps memory K order within the instruction's groups."""
    nv = _nv()
    for pos, want in ((1, 256.03125), (7, 256.03125), (8, 256.046875), (31, 256.046875), (32, 256.046875)):
        a = np.zeros((1, 128), np.uint8)
        a[0, 0], a[0, pos] = 0x78, 0x14                     # 256, 0.046875
        b = np.full((1, 128), 0x38, np.uint8)               # 1.0
        s = np.full((1, 4), 127, np.uint8)
        qa = nv.MXFP8Tensor(torch.from_numpy(a).cuda(), torch.from_numpy(s).cuda(), 1, 128)
        qb = nv.MXFP8Tensor(torch.from_numpy(b).cuda(), torch.from_numpy(s.copy()).cuda(), 1, 128)
        c = nv.mxfp8_gemm(qa, qb)
        torch.cuda.synchronize()
        assert float(c[0, 0]) == want, (pos, float(c[0, 0]))


def test_gemm_k_rules():
    nv = _nv()
    a, b = nv.MXFP8Tensor.empty(8, 0), nv.MXFP8Tensor.empty(4, 0)
    c = torch.full((8, 4), 5.0, device="cuda")
    nv.mxfp8_gemm(a, b, out=c)
    torch.cuda.synchronize()
    assert torch.all(c == 0)
    with pytest.raises(nv.NVFP4Error, match="shape"):
        nv.mxfp8_gemm(nv.MXFP8Tensor.empty(8, 96), nv.MXFP8Tensor.empty(4, 96))


@pytest.mark.parametrize("name", ["fprop", "dgrad", "wgrad"])
def test_full_workload_step(name):
    """The MXFP8 step at the full layer shapes, as the benchmark runs it:
    both operands quantized on the GPU (bit-exact against the oracle on the
    whole tensors, along the layer's axes), then the GEMM checked on 64+
    sampled rows and columns."""
    nv = _nv()
    g = workloads.GEMMS[name]
    m, n, k = g.mnk
    print(f"[mxfp8] full {name} {g.mnk}", flush=True)
    qs = []
    for op in (g.a, g.b):
        x = op.generate()
        ref = oracle.mxfp8_quantize(x, axis=op.axis)
        q = nv.mxfp8_quantize(x.cuda(), axis=op.axis)
        torch.cuda.synchronize()
        assert torch.equal(q.scales.cpu(), torch.from_numpy(ref.scales)), f"{name} scales"
        assert torch.equal(q.codes.cpu(), torch.from_numpy(ref.codes)), f"{name} codes"
        qs.append((q, ref))
    (qa, ra), (qb, rb) = qs
    dt = torch.float32 if g.out == "f32" else torch.bfloat16
    c = nv.mxfp8_gemm(qa, qb, dt)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, m - 1], rng.choice(m, 64, replace=False)]))
    cols = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 64, replace=False)]))
    cc = c.cpu()
    _check(cc, ra, rb, g.out, rows=rows, label=f"{name} rows")
    _check(cc, ra, rb, g.out, cols=cols, label=f"{name} cols")

"""GPU parity of the MXFP4 path against the CPU oracle: the quantizer
bit-exact on codes and scales (axis 1 and 0, bf16 and f32, ragged shapes),
the block-scaled FP4 MFMA GEMM within 1e-5 * sum|a*b| (bf16 outputs by the
rounding interval), including tile tails and both tile widths.  Called
through the C ABI."""
import functools

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


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
                                            (512, 130, 0)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_matches_oracle(rows, cols, axis, dtype):
    print(f"[mxfp4 quantize] {rows}x{cols} axis={axis} {dtype}", flush=True)
    nv = _nv()
    x = _x(rows, cols, 5, dtype)
    q = nv.mxfp4_quantize(x.cuda(), axis=axis)
    torch.cuda.synchronize()
    ref = oracle.mxfp4_quantize(x, axis=axis)
    np.testing.assert_array_equal(q.scales.cpu().numpy(), ref.scales)
    np.testing.assert_array_equal(q.codes.cpu().numpy(), ref.codes)


def _gemm_case(m, n, k, out, seed=1):
    nv = _nv()
    xa, xb = _x(m, k, seed, "bf16"), _x(n, k, seed + 1, "bf16")
    qa, qb = nv.mxfp4_quantize(xa.cuda()), nv.mxfp4_quantize(xb.cuda())
    dt = torch.float32 if out == "f32" else torch.bfloat16
    c = nv.mxfp4_gemm(qa, qb, dt)
    torch.cuda.synchronize()
    ra, rb = oracle.mxfp4_quantize(xa), oracle.mxfp4_quantize(xb)
    cref, bound = oracle.mxfp4_gemm(ra, rb)
    if out == "f32":
        ok, worst = oracle.check_gemm_f32(c.cpu().numpy(), cref, bound, 1e-5)
        print(f"[mxfp4 gemm] {m}x{n}x{k}: worst |err|/bound = {worst:.3e}", flush=True)
        assert ok, f"{m}x{n}x{k}: worst |err|/bound = {worst:.3e}"
    else:
        ok, nbad = oracle.check_gemm_bf16(c.double().cpu().numpy(), cref, bound, 1e-5)
        assert ok, f"{m}x{n}x{k}: {nbad} bf16 outputs outside the tolerance interval"


@pytest.mark.parametrize("m,n,k", [(256, 256, 256), (200, 136, 512), (257, 129, 256), (1, 1, 256),
                                   (384, 640, 1024), (64, 300, 768), (64, 40000, 256)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemm_matches_oracle(m, n, k, out):
    print(f"[mxfp4 gemm] {m}x{n}x{k} {out}", flush=True)
    _gemm_case(m, n, k, out)


def test_gemm_k_rules():
    nv = _nv()
    a, b = nv.MXFP4Tensor.empty(8, 0), nv.MXFP4Tensor.empty(4, 0)
    c = torch.full((8, 4), 5.0, device="cuda")
    nv.mxfp4_gemm(a, b, out=c)
    torch.cuda.synchronize()
    assert torch.all(c == 0)
    with pytest.raises(nv.NVFP4Error, match="shape"):
        nv.mxfp4_gemm(nv.MXFP4Tensor.empty(8, 96), nv.MXFP4Tensor.empty(4, 96))


@pytest.mark.parametrize("name", ["fprop", "dgrad", "wgrad"])
def test_full_workload_step(name):
    """The MXFP4 step at the full layer shapes, as the benchmark runs it:
    both operands quantized on the GPU (bit-exact against the oracle on the
    whole tensors, along the layer's axes), then the GEMM checked on 128+
    sampled rows and columns (every tile position of the sampled lines)."""
    nv = _nv()
    g = workloads.GEMMS[name]
    m, n, k = g.mnk
    print(f"[mxfp4] full {name} {g.mnk}", flush=True)
    qs = []
    for op in (g.a, g.b):
        x = op.generate()
        ref = oracle.mxfp4_quantize(x, axis=op.axis)
        q = nv.mxfp4_quantize(x.cuda(), axis=op.axis)
        torch.cuda.synchronize()
        assert torch.equal(q.scales.cpu(), torch.from_numpy(ref.scales)), f"{name} scales"
        assert torch.equal(q.codes.cpu(), torch.from_numpy(ref.codes)), f"{name} codes"
        qs.append((q, ref))
    (qa, ra), (qb, rb) = qs
    dt = torch.float32 if g.out == "f32" else torch.bfloat16
    c = nv.mxfp4_gemm(qa, qb, dt)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, m - 1], rng.choice(m, 128, replace=False)]))
    cols = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 128, replace=False)]))
    cref, bound = oracle.mxfp4_gemm(ra, rb, rows, cols)
    got = c[torch.as_tensor(rows, device="cuda")][:, torch.as_tensor(cols, device="cuda")].double().cpu().numpy()
    if g.out == "f32":
        ok, worst = oracle.check_gemm_f32(got, cref, bound, 1e-5)
        print(f"[mxfp4 gemm] {name}: worst |err|/bound = {worst:.3e}", flush=True)
        assert ok, f"{name}: worst |err|/bound = {worst:.3e}"
    else:
        ok, nbad = oracle.check_gemm_bf16(got, cref, bound, 1e-5)
        assert ok, f"{name}: {nbad} bf16 outputs outside the tolerance interval"

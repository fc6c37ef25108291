"""GPU parity of the block-scaled NVFP4 GEMM against the float64 oracle.

Operands are quantized by the oracle and uploaded, so the GEMM is checked on
its own; the end-to-end test then feeds it the GPU quantizer's output (which
is bit-identical to the oracle's).  Tolerance (every element):
|C - Cref| <= 1e-5 * gA gB sum_k |(qA SA)(qB SB)|; bf16 outputs must lie in
[bf16(Cref - tol), bf16(Cref + tol)].
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

RTOL = 1e-5
MASK = workloads.rht_sign_mask()


@functools.lru_cache(maxsize=None)
def _nv():
    import gemm_amax_reduce_amd as nv
    nv.lib()
    return nv


def _upload(ref):
    nv = _nv()
    return nv.NVFP4Tensor(torch.from_numpy(ref.codes).cuda(), torch.from_numpy(ref.scales).cuda(),
                          torch.from_numpy(ref.meta).cuda(), ref.outer, ref.k)


def _gemm(qa, qb, out="f32", ldc_pad=0):
    nv = _nv()
    dt = torch.float32 if out == "f32" else torch.bfloat16
    if ldc_pad:
        buf = torch.full((qa.outer, qb.outer + ldc_pad), 7.0, dtype=dt, device="cuda")
        c = nv.nvfp4_gemm(qa, qb, dt, out=buf[:, :qb.outer])
        torch.cuda.synchronize()
        assert torch.all(buf[:, qb.outer:] == 7.0), "wrote outside ldc window"
    else:
        c = nv.nvfp4_gemm(qa, qb, dt)
        torch.cuda.synchronize()
    return c.cpu()


def _check(c_gpu, ref_a, ref_b, out, rows=None, cols=None, label=""):
    cref, bound = oracle.gemm(ref_a, ref_b, rows, cols)
    if rows is not None:
        c_gpu = c_gpu[torch.as_tensor(rows)]
    if cols is not None:
        c_gpu = c_gpu[:, torch.as_tensor(cols)]
    if out == "f32":
        ok, worst = oracle.check_gemm_f32(c_gpu.double().numpy(), cref, bound, RTOL)
        print(f"[gemm] {label}: worst |err|/bound = {worst:.3e}", flush=True)
        assert ok, f"{label}: worst |err|/bound = {worst:.3e} > {RTOL}"
        return worst
    ok, nbad = oracle.check_gemm_bf16(c_gpu.double().numpy(), cref, bound, RTOL)
    assert ok, f"{label}: {nbad} bf16 outputs outside the tolerance interval"
    return 0.0


def _rand_q(outer, k, seed, axis=1, scale=1.0, rounding=oracle.RNE):
    x = workloads.normal(outer, k, seed) * np.float32(scale)
    x = workloads.with_outliers(x, seed + 1, p=0.01)
    return oracle.quantize(x, axis=1, rounding=rounding, seed=seed)


def test_tiny_config():
    g = workloads.TINY
    print("[gemm] tiny 128x128x256", flush=True)
    ra = oracle.quantize(g.a.generate(), axis=1)
    rb = oracle.quantize(g.b.generate(), axis=0)
    c = _gemm(_upload(ra), _upload(rb), "f32")
    _check(c, ra, rb, "f32", label="tiny")


# (64, 40000, 64): 157 tile columns in one row of tiles, the launcher keeps
# every column at 256 wide (no 128-wide remainder) and the last one is ragged
@pytest.mark.parametrize("m,n,k", [(128, 128, 128), (200, 136, 272), (257, 129, 16), (64, 300, 528),
                                   (1, 1, 16), (3, 517, 48), (384, 256, 1024), (64, 40000, 64)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_ragged_shapes(m, n, k, out):
    print(f"[gemm] {m}x{n}x{k} {out}", flush=True)
    ra, rb = _rand_q(m, k, 11), _rand_q(n, k, 12, scale=0.01)
    c = _gemm(_upload(ra), _upload(rb), out)
    _check(c, ra, rb, out, label=f"{m}x{n}x{k}")


def test_ldc_larger_than_n():
    ra, rb = _rand_q(130, 64, 21), _rand_q(70, 64, 22)
    c = _gemm(_upload(ra), _upload(rb), "f32", ldc_pad=9)
    _check(c, ra, rb, "f32", label="ldc")


def test_k_zero_and_empty():
    nv = _nv()
    z = nv.NVFP4Tensor.empty(5, 0)
    z.meta.fill_(1.0)
    w = nv.NVFP4Tensor.empty(7, 0)
    w.meta.fill_(1.0)
    c = torch.full((5, 7), 3.0, device="cuda")
    nv.nvfp4_gemm(z, w, out=c)
    torch.cuda.synchronize()
    assert torch.all(c == 0)
    e = nv.NVFP4Tensor.empty(0, 32)
    e.meta.zero_()
    ra = _upload(_rand_q(4, 32, 3))
    assert nv.nvfp4_gemm(e, ra).shape == (0, 4)
    with pytest.raises(nv.NVFP4Error, match="shape"):
        nv.nvfp4_gemm(ra, _upload(_rand_q(4, 48, 3)))


def test_extreme_scales():
    # operands whose block scales span the E4M3 range, including subnormal
    # scales (tiny blocks next to a huge one)
    x = workloads.normal(96, 256, 31)
    x[:, :16] *= 1e4
    x[5, :] = 0.0
    x[7, 32:48] = 1e-7
    ra = oracle.quantize(x, axis=1)
    assert (ra.scales < 8).any()      # subnormal E4M3 scales present
    rb = _rand_q(80, 256, 32, scale=3.0)
    c = _gemm(_upload(ra), _upload(rb), "f32")
    _check(c, ra, rb, "f32", label="extreme scales")


def test_deterministic():
    ra, rb = _rand_q(256, 512, 41), _rand_q(256, 512, 42)
    qa, qb = _upload(ra), _upload(rb)
    assert torch.equal(_gemm(qa, qb).view(torch.int32), _gemm(qa, qb).view(torch.int32))


# ------------------------------------------------------ full workloads ----

def _sample(n, count, seed):
    rng = np.random.default_rng(seed)
    base = np.array([0, n - 1])
    return np.unique(np.concatenate([base, rng.choice(n, size=min(count, n), replace=False)]))


@pytest.mark.parametrize("name", ["fprop", "dgrad", "wgrad"])
def test_full_workload_end_to_end(name):
    """GPU quantize (checked bit-exact against the oracle) -> GPU GEMM at the
    full layer shape; every element of 256+ sampled rows and 256+ sampled
    columns (which covers every tile position) checked against the oracle."""
    nv = _nv()
    g = workloads.GEMMS[name]
    print(f"[gemm] full {name} {g.mnk}", flush=True)
    ops = []
    for op in (g.a, g.b):
        x = op.generate()
        r = oracle.SR if op.rounding == "sr" else oracle.RNE
        ref = oracle.quantize(x, axis=op.axis, rounding=r, seed=workloads.SR_SEED, offset=op.sr_offset,
                              rht=op.rht, sign_mask=MASK)
        xd = x.cuda()
        if op.rht:
            q = nv.nvfp4_rht_quantize(xd, MASK, axis=op.axis, rounding=op.rounding, seed=workloads.SR_SEED,
                                      offset=op.sr_offset)
        else:
            q = nv.nvfp4_quantize(xd, axis=op.axis, rounding=op.rounding, seed=workloads.SR_SEED,
                                  offset=op.sr_offset)
        torch.cuda.synchronize()
        del xd
        assert torch.equal(q.codes.cpu(), torch.from_numpy(ref.codes)), f"{name} codes"
        assert torch.equal(q.scales.cpu(), torch.from_numpy(ref.scales)), f"{name} scales"
        ops.append((q, ref))
    (qa, ra), (qb, rb) = ops
    m, n, k = g.mnk
    c = _gemm(qa, qb, g.out)
    rows = _sample(m, 256, 1)
    cols = _sample(n, 256, 2)
    _check(c, ra, rb, g.out, rows=rows, label=f"{name} rows")
    _check(c, ra, rb, g.out, cols=cols, label=f"{name} cols")
    if g.out == "bf16":
        # the f32 result of the same launch configuration, checked strictly
        c32 = _gemm(qa, qb, "f32")
        _check(c32, ra, rb, "f32", rows=rows, label=f"{name} f32 rows")


def test_binding_rejects_bad_buffers():
    """The C ABI cannot see buffer sizes, so the binding checks every
    caller-supplied buffer before the call (nothing is launched)."""
    nv = _nv()
    qa, qb = _upload(_rand_q(64, 64, 5)), _upload(_rand_q(32, 64, 6))
    with pytest.raises(nv.NVFP4Error, match="shape"):
        nv.nvfp4_gemm(qa, qb, out=torch.empty((64, 31), device="cuda"))
    with pytest.raises(nv.NVFP4Error, match="dtype"):
        nv.nvfp4_gemm(qa, qb, out=torch.empty((64, 32), dtype=torch.float16, device="cuda"))
    with pytest.raises(nv.NVFP4Error, match="output dtype"):
        nv.nvfp4_gemm(qa, qb, torch.float16)
    with pytest.raises(nv.NVFP4Error, match="overlap"):
        nv.nvfp4_gemm(qa, qb, out=torch.empty((64, 64), device="cuda").as_strided((64, 32), (16, 1)))
    short = nv.NVFP4Tensor(qa.codes[:32], qa.scales, qa.meta, 64, 64)
    with pytest.raises(nv.NVFP4Error, match="codes"):
        nv.nvfp4_gemm(short, qb)
    with pytest.raises(nv.NVFP4Error, match="codes"):
        nv.nvfp4_quantize(torch.zeros((64, 64), device="cuda"), out=short)
    with pytest.raises(nv.NVFP4Error, match="out"):
        nv.nvfp4_dequantize(qa, out=torch.empty((64, 63), device="cuda"))
    with pytest.raises(nv.NVFP4Error, match="meta"):
        nv.nvfp4_gemm(nv.NVFP4Tensor(qa.codes, qa.scales, qa.meta.double(), 64, 64), qb)


def test_mfma_probe_runs():
    """The MFMA ceiling probe the benchmark reports beside the published
    peak: a finite rate below that peak (2.5 PFLOP/s dense f16)."""
    nv = _nv()
    rate = nv.nvfp4_probe_mfma(200)
    assert 100.0 < rate < 2600.0, rate

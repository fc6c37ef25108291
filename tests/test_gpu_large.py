"""GPU parity at the size limits: tensors whose element counts pass 2^32,
code arrays and outputs whose byte offsets pass 2^31 and 2^32, and the
largest K the GEMM accepts.

The quantizer input is too large for the oracle to process whole, so it is
built from one seeded 64-row block, scaled per 64-row slab by factors known
on the host; the tensor amax is therefore known exactly, and the oracle
quantizes the checked slices with that amax supplied and their global row
index (outer0), which gives the codes those rows have in the whole tensor
(exact for nearest rounding, and for stochastic rounding because the
element index of the counter is the whole tensor's).  Bit-exact on codes,
scales and meta; the GEMM within 1e-5 * sum |a b| on sampled rows and
columns computed by the oracle one by one.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

RTOL = 1e-5
BLK = 64                 # rows per slab
COLS = 32768
NBLK = 2049              # 131136 rows: 4.297e9 elements, 2.149e9 code bytes
FACTORS = [1.0 + (j % 7) / 8.0 for j in range(NBLK)]


@functools.lru_cache(maxsize=None)
def _nv():
    import gemm_amax_reduce_amd as nv
    nv.lib()
    return nv


@functools.lru_cache(maxsize=None)
def _base():
    return workloads.normal(BLK, COLS, seed=50)


def _slab_bf16(j, cols=slice(None)):
    """Host copy of slab j (rows 64j .. 64j+63) as bf16 bit patterns."""
    t = (torch.from_numpy(np.ascontiguousarray(_base()[:, cols])) * FACTORS[j]).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _amax():
    base = torch.from_numpy(_base())
    return max(float((base * f).to(torch.bfloat16).float().abs().max()) for f in sorted(set(FACTORS)))


@pytest.fixture(scope="module")
def big_x():
    print(f"[large] building x [{NBLK * BLK}, {COLS}] bf16 on the GPU", flush=True)
    base = torch.from_numpy(_base()).cuda()
    x = torch.empty((NBLK * BLK, COLS), dtype=torch.bfloat16, device="cuda")
    for j in range(NBLK):
        x[j * BLK:(j + 1) * BLK] = (base * FACTORS[j]).to(torch.bfloat16)
    torch.cuda.synchronize()
    yield x
    del x
    torch.cuda.empty_cache()


def _assert_rows(q, rows, ref, label):
    codes = q.codes[rows].cpu().numpy()
    scales = q.scales[rows].cpu().numpy()
    np.testing.assert_array_equal(scales, ref.scales, err_msg=f"scales {label}")
    if not np.array_equal(codes, ref.codes):
        bad = np.argwhere(codes != ref.codes)
        raise AssertionError(f"codes differ {label}: {len(bad)} bytes, first at {tuple(bad[0])}")


@pytest.mark.parametrize("rounding", ["rne", "sr"])
def test_quantize_axis1_past_2pow32_elements(big_x, rounding):
    nv = _nv()
    amax = _amax()
    print(f"[large] quantize axis 1 {rounding} rows={big_x.shape[0]}", flush=True)
    q = nv.nvfp4_quantize(big_x, axis=1, rounding=rounding, seed=0x5EED, offset=11)
    torch.cuda.synchronize()
    assert q.codes.numel() > 2 ** 31
    meta = q.meta.cpu().numpy()
    assert meta[0] == np.float32(amax), (meta[0], amax)
    r = oracle.SR if rounding == "sr" else oracle.RNE
    for j in (0, 1023, NBLK - 1):           # the last slab starts at code byte 2^31
        ref = oracle.quantize(_slab_bf16(j), axis=1, rounding=r, seed=0x5EED, offset=11, amax=amax,
                              outer0=j * BLK)
        np.testing.assert_array_equal(ref.meta.view(np.uint32), meta.view(np.uint32))
        _assert_rows(q, slice(j * BLK, (j + 1) * BLK), ref, f"slab {j}")
    del q
    torch.cuda.empty_cache()


@pytest.mark.parametrize("rounding", ["rne", "sr"])
def test_quantize_axis0_past_2pow31_code_bytes(big_x, rounding):
    nv = _nv()
    amax = _amax()
    print(f"[large] quantize axis 0 {rounding} k={big_x.shape[0]}", flush=True)
    q = nv.nvfp4_quantize(big_x, axis=0, rounding=rounding, seed=0x5EED, offset=12)
    torch.cuda.synchronize()
    assert q.outer == COLS and q.k == NBLK * BLK
    c0 = COLS - 64                          # output rows 32704.. start past code byte 2^31
    cols = slice(c0, COLS)
    xcols = np.concatenate([_slab_bf16(j, cols) for j in range(NBLK)], axis=0)
    r = oracle.SR if rounding == "sr" else oracle.RNE
    ref = oracle.quantize(xcols, axis=0, rounding=r, seed=0x5EED, offset=12, amax=amax, outer0=c0)
    meta = q.meta.cpu().numpy()
    np.testing.assert_array_equal(ref.meta.view(np.uint32), meta.view(np.uint32))
    _assert_rows(q, slice(c0, COLS), ref, "last 64 columns")
    del q
    torch.cuda.empty_cache()


def _upload(ref):
    nv = _nv()
    return nv.NVFP4Tensor(torch.from_numpy(ref.codes).cuda(), torch.from_numpy(ref.scales).cuda(),
                          torch.from_numpy(ref.meta).cuda(), ref.outer, ref.k)


def _check_sampled(c, ra, rb, rows, cols, out, label):
    cref, bound = oracle.gemm(ra, rb, rows, cols)
    got = c[torch.as_tensor(rows, device=c.device)][:, torch.as_tensor(cols, device=c.device)].cpu().double().numpy()
    if out == "f32":
        ok, worst = oracle.check_gemm_f32(got, cref, bound, RTOL)
        assert ok, f"{label}: worst |err|/bound = {worst:.3e}"
    else:
        ok, nbad = oracle.check_gemm_bf16(got, cref, bound, RTOL)
        assert ok, f"{label}: {nbad} bf16 outputs outside the tolerance interval"


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemm_output_past_2pow31_elements(out):
    nv = _nv()
    m, n, k = 65536 + 32, 32768 + 16, 256
    print(f"[large] gemm {m}x{n}x{k} {out}", flush=True)
    ra = oracle.quantize(workloads.normal(m, k, seed=51), axis=1)
    rb = oracle.quantize(workloads.normal(n, k, seed=52), axis=1)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    c = nv.nvfp4_gemm(_upload(ra), _upload(rb), dt)
    torch.cuda.synchronize()
    assert c.numel() > 2 ** 31
    rng = np.random.default_rng(53)
    rows = np.unique(np.concatenate([[0, 65535], np.arange(65536, m), rng.integers(0, m, 32)]))
    cols = np.unique(np.concatenate([np.arange(16), np.arange(32768, n), rng.integers(0, n, 48)]))
    _check_sampled(c, ra, rb, rows, cols, out, f"{m}x{n}x{k}")
    del c
    torch.cuda.empty_cache()


@pytest.mark.parametrize("k", [(1 << 25) - 256, (1 << 25) - 16])
def test_gemm_largest_k(k):
    """The largest K the launcher accepts (< 2^25; K % 64 == 0 takes the
    scale DMA, K % 64 != 0 the per-lane scale loads); one workgroup runs
    the whole reduction."""
    nv = _nv()
    print(f"[large] gemm 3x2x{k}", flush=True)
    ra = oracle.quantize(workloads.normal(3, k, seed=54), axis=1)
    rb = oracle.quantize(workloads.normal(2, k, seed=55), axis=1)
    c = nv.nvfp4_gemm(_upload(ra), _upload(rb), torch.float32)
    torch.cuda.synchronize()
    _check_sampled(c, ra, rb, np.arange(3), np.arange(2), "f32", f"k={k}")


def test_gemm_k_limit_is_an_error():
    nv = _nv()
    k = 1 << 25
    a = nv.NVFP4Tensor(torch.zeros((1, k // 2), dtype=torch.uint8, device="cuda"),
                       torch.zeros((1, k // 16), dtype=torch.uint8, device="cuda"),
                       torch.zeros(2, dtype=torch.float32, device="cuda"), 1, k)
    with pytest.raises(nv.NVFP4Error):
        nv.nvfp4_gemm(a, a, torch.float32)

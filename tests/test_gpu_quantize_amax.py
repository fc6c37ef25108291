"""GPU parity of the two passes called apart: nvfp4_amax against the oracle's
tensor amax, and nvfp4_quantize_amax against the oracle with the same
supplied amax (the true one, twice it, half of it), bit-exact on codes,
scales and meta.  Called through the C ABI."""
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


CASES = [(1, "rne", False), (1, "sr", False), (1, "sr", True), (0, "rne", False), (0, "rne", True), (0, "sr", True)]


@pytest.mark.parametrize("axis,rounding,rht", CASES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_amax_then_quantize(axis, rounding, rht, dtype):
    print(f"[amax] axis={axis} {rounding} rht={rht} {dtype}", flush=True)
    nv = _nv()
    x = workloads.mixed_rows(96, 272, 41)
    xt = torch.from_numpy(x) if dtype == "f32" else workloads.to_bf16(x)
    xd = xt.cuda()
    code = oracle.SR if rounding == "sr" else oracle.RNE
    ref = oracle.quantize(xt, axis=axis, rounding=code, seed=9, offset=2, rht=rht, sign_mask=MASK)
    a = nv.nvfp4_amax(xd, axis=axis, rht=rht, sign_mask=MASK)
    torch.cuda.synchronize()
    assert a.cpu().numpy().view(np.uint32)[0] == ref.meta.view(np.uint32)[0]
    for factor in (1.0, 2.0, 0.5):
        amax = (a * factor).contiguous()
        q = nv.nvfp4_quantize_amax(xd, amax, axis=axis, rounding=rounding, seed=9, offset=2, rht=rht,
                                   sign_mask=MASK)
        torch.cuda.synchronize()
        r = oracle.quantize(xt, axis=axis, rounding=code, seed=9, offset=2, rht=rht, sign_mask=MASK,
                            amax=float(amax.cpu()[0]))
        np.testing.assert_array_equal(q.meta.cpu().numpy().view(np.uint32), r.meta.view(np.uint32))
        np.testing.assert_array_equal(q.scales.cpu().numpy(), r.scales)
        np.testing.assert_array_equal(q.codes.cpu().numpy(), r.codes)


def test_amax_empty_is_zero():
    nv = _nv()
    a = nv.nvfp4_amax(torch.empty(0, 32, device="cuda"))
    torch.cuda.synchronize()
    assert float(a.cpu()[0]) == 0.0


@pytest.mark.parametrize("axis,rounding", [(1, "rne"), (1, "sr"), (0, "rne"), (0, "sr")])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rht_values_near_the_top_of_the_range(axis, rounding, dtype):
    """The transform on values near 1e37 (its sums stay finite), quantized
    with the computed amax and with a supplied 3e38.  With 3e38 the tensor
    scale s_enc is below 2^-115, where a bf16 encode stops taking the block
    as 4y with the scales quartered and multiplies the values by 1/4 itself:
    both forms bit-exact against the oracle."""
    print(f"[amax] near-top axis={axis} {rounding} {dtype}", flush=True)
    nv = _nv()
    x = workloads.mixed_rows(64, 160, 43)
    x = x / np.abs(x).max() * 1e37
    xt = torch.from_numpy(x.astype(np.float32)) if dtype == "f32" else workloads.to_bf16(x)
    xd = xt.cuda()
    code = oracle.SR if rounding == "sr" else oracle.RNE
    q = nv.nvfp4_rht_quantize(xd, MASK, axis=axis, rounding=rounding, seed=5, offset=3)
    torch.cuda.synchronize()
    r = oracle.quantize(xt, axis=axis, rounding=code, seed=5, offset=3, rht=True, sign_mask=MASK)
    assert np.isfinite(r.meta).all() and r.meta[0] > 1e36
    np.testing.assert_array_equal(q.meta.cpu().numpy().view(np.uint32), r.meta.view(np.uint32))
    np.testing.assert_array_equal(q.scales.cpu().numpy(), r.scales)
    np.testing.assert_array_equal(q.codes.cpu().numpy(), r.codes)
    amax = torch.tensor([3e38], dtype=torch.float32, device="cuda")
    q = nv.nvfp4_quantize_amax(xd, amax, axis=axis, rounding=rounding, seed=5, offset=3, rht=True, sign_mask=MASK)
    torch.cuda.synchronize()
    r = oracle.quantize(xt, axis=axis, rounding=code, seed=5, offset=3, rht=True, sign_mask=MASK,
                        amax=float(amax.cpu()[0]))
    assert r.scales.any()
    np.testing.assert_array_equal(q.meta.cpu().numpy().view(np.uint32), r.meta.view(np.uint32))
    np.testing.assert_array_equal(q.scales.cpu().numpy(), r.scales)
    np.testing.assert_array_equal(q.codes.cpu().numpy(), r.codes)

"""GPU parity of the dual-layout quantizer (nvfp4_quantize_dual): both outputs
bit-exact against the CPU oracle's two single quantizations on small ragged
shapes, and bit-identical to the two single-layout GPU calls on the full dY
tensor of the data- and weight-gradient workloads.  Called through the C ABI.
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


def _same(q, ref, label):
    np.testing.assert_array_equal(q.meta.cpu().numpy().view(np.uint32), ref.meta.view(np.uint32),
                                  err_msg=f"meta {label}")
    np.testing.assert_array_equal(q.scales.cpu().numpy(), ref.scales, err_msg=f"scales {label}")
    np.testing.assert_array_equal(q.codes.cpu().numpy(), ref.codes, err_msg=f"codes {label}")


@pytest.mark.parametrize("rows,cols", [(16, 16), (48, 80), (272, 528), (512, 1040)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rht0,r1,r0", [(False, "rne", "rne"), (True, "sr", "sr"), (True, "rne", "sr"),
                                        (False, "sr", "rne")])
def test_dual_matches_oracle(rows, cols, dtype, rht0, r1, r0):
    print(f"[dual] {rows}x{cols} {dtype} rht0={rht0} r1={r1} r0={r0}", flush=True)
    nv = _nv()
    x = workloads.mixed_rows(rows, cols, 77)
    xt = torch.from_numpy(x) if dtype == "f32" else workloads.to_bf16(x)
    q1, q0 = nv.nvfp4_quantize_dual(xt.cuda(), rounding1=r1, seed1=11, offset1=3, rht0=rht0, sign_mask0=MASK,
                                    rounding0=r0, seed0=12, offset0=4)
    torch.cuda.synchronize()
    code = {"rne": oracle.RNE, "sr": oracle.SR}
    ref1 = oracle.quantize(xt, axis=1, rounding=code[r1], seed=11, offset=3)
    ref0 = oracle.quantize(xt, axis=0, rounding=code[r0], seed=12, offset=4, rht=rht0, sign_mask=MASK)
    _same(q1, ref1, "axis 1")
    _same(q0, ref0, "axis 0")


def test_dual_equals_single_calls_on_dY():
    # the data-gradient (axis 1, SR, offset 0) and weight-gradient (axis 0,
    # RHT, SR, offset 1) quantizations of the 8192 x 20480 gradient
    print("[dual] dY 8192x20480 bf16", flush=True)
    nv = _nv()
    dY = workloads.DGRAD.a.generate().cuda()
    seed = workloads.SR_SEED
    q1, q0 = nv.nvfp4_quantize_dual(dY, rounding1="sr", seed1=seed, offset1=0, rht0=True, sign_mask0=MASK,
                                    rounding0="sr", seed0=seed, offset0=1)
    s1 = nv.nvfp4_quantize(dY, axis=1, rounding="sr", seed=seed, offset=0)
    s0 = nv.nvfp4_rht_quantize(dY, MASK, axis=0, rounding="sr", seed=seed, offset=1)
    torch.cuda.synchronize()
    for a, b, label in ((q1, s1, "axis 1"), (q0, s0, "axis 0")):
        assert torch.equal(a.meta, b.meta), label
        assert torch.equal(a.scales, b.scales), label
        assert torch.equal(a.codes, b.codes), label


def test_dual_zero_and_empty():
    nv = _nv()
    z = torch.zeros(32, 48, device="cuda", dtype=torch.bfloat16)
    q1, q0 = nv.nvfp4_quantize_dual(z, rht0=True, sign_mask0=MASK)
    torch.cuda.synchronize()
    for q in (q1, q0):
        assert torch.all(q.meta == 0) and torch.all(q.scales == 0) and torch.all(q.codes == 0)
    e = torch.empty(0, 32, device="cuda")
    q1, q0 = nv.nvfp4_quantize_dual(e)
    torch.cuda.synchronize()
    assert torch.all(q1.meta == 0) and torch.all(q0.meta == 0)

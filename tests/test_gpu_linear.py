"""GPU checks of the NVFP4 linear layer (autograd over the C ABI): forward and
both gradients against the oracle's quantizations and fp64 GEMM of the same
operands, within the GEMM tolerance 1e-5 * sum|a*b| (bf16 outputs by the
rounding interval), and the BF16 policy flag equal to a plain bf16 linear."""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

MASK = 0xA5C3


def _ref(qa, qb):
    c, bound = oracle.gemm(qa, qb)
    return c, bound


def _close_f32(got, c, bound, label):
    ok, worst = oracle.check_gemm_f32(got, c, bound, 1e-5)
    print(f"[linear] {label}: worst |err|/bound = {worst:.3e}", flush=True)
    assert ok, f"{label}: worst |err|/bound = {worst:.3e}"


def _within_bf16(got_bf16, c, bound, label):
    ok, nbad = oracle.check_gemm_bf16(got_bf16.double().cpu().numpy(), c, bound, 1e-5)
    assert ok, f"{label}: {nbad} bf16 outputs outside the tolerance interval"


def test_forward_and_backward_match_oracle():
    import gemm_amax_reduce_amd.linear as L
    tokens, fin, fout = 64, 96, 80
    print(f"[linear] {tokens}x{fin} -> {fout}", flush=True)
    torch.manual_seed(0)
    layer = L.NVFP4Linear(fin, fout, seed=3, sign_mask=MASK, device="cuda", dtype=torch.float32)
    x = torch.from_numpy(workloads.normal(tokens, fin, 5)).cuda().requires_grad_(True)
    y = layer(x)
    dy = torch.from_numpy(workloads.laplace(tokens, fout, 6, 1e-3)).cuda()
    y.backward(dy)
    torch.cuda.synchronize()
    xc, wc, dyc = x.detach().cpu(), layer.weight.detach().cpu(), dy.cpu()
    # forward
    c, b = _ref(oracle.quantize(xc, axis=1), oracle.quantize(wc, axis=1))
    _close_f32(y.detach().cpu().numpy(), c, b, "y")
    # data gradient: dy (axis 1, SR, offset 0) . W (axis 0)
    c, b = _ref(oracle.quantize(dyc, axis=1, rounding=oracle.SR, seed=3, offset=0), oracle.quantize(wc, axis=0))
    _close_f32(x.grad.cpu().numpy(), c, b, "dx")
    # weight gradient: dy (axis 0, RHT, SR, offset 1) . x (axis 0, RHT)
    c, b = _ref(oracle.quantize(dyc, axis=0, rounding=oracle.SR, seed=3, offset=1, rht=True, sign_mask=MASK),
                oracle.quantize(xc, axis=0, rht=True, sign_mask=MASK))
    _close_f32(layer.weight.grad.cpu().numpy(), c, b, "dW")


def test_bf16_forward_output():
    import gemm_amax_reduce_amd.linear as L
    layer = L.NVFP4Linear(64, 48, device="cuda", dtype=torch.bfloat16)
    x = workloads.to_bf16(workloads.normal(32, 64, 8)).cuda()
    y = layer(x)
    torch.cuda.synchronize()
    assert y.dtype == torch.bfloat16
    c, b = _ref(oracle.quantize(x.cpu(), axis=1), oracle.quantize(layer.weight.detach().cpu(), axis=1))
    _within_bf16(y.detach(), c, b, "y bf16")


def test_keep_bf16_policy_is_plain_linear():
    import gemm_amax_reduce_amd.linear as L
    layer = L.NVFP4Linear(64, 32, keep_bf16=True, device="cuda", dtype=torch.bfloat16)
    x = workloads.to_bf16(workloads.normal(16, 64, 9)).cuda()
    y = layer(x)
    ref = torch.nn.functional.linear(x.float(), layer.weight.detach().float())
    torch.cuda.synchronize()
    assert torch.allclose(y.detach().float(), ref, rtol=2e-2, atol=1e-2)


def test_successive_calls_draw_fresh_offsets():
    import gemm_amax_reduce_amd.linear as L
    layer = L.NVFP4Linear(64, 32, seed=1, device="cuda", dtype=torch.float32)
    x = torch.from_numpy(workloads.normal(32, 64, 10)).cuda().requires_grad_(True)
    dy = torch.from_numpy(workloads.laplace(32, 32, 11, 1e-3)).cuda()   # off-grid values: SR has work
    grads = []
    for _ in range(2):
        x.grad = None
        layer(x).backward(dy)
        grads.append(x.grad.clone())
    torch.cuda.synchronize()
    assert not torch.equal(grads[0], grads[1])     # stochastic rounding differs between steps


def test_leading_dimensions_are_tokens():
    """x [batch, seq, in] runs as the [batch*seq, in] matrix: outputs and
    both gradients bit-identical to the flattened call (same weight, seed and
    step), y shaped [batch, seq, out]; a token count that is not a multiple
    of 16 is refused."""
    import gemm_amax_reduce_amd.linear as L
    la = L.NVFP4Linear(96, 80, seed=4, sign_mask=MASK, device="cuda", dtype=torch.float32)
    lb = L.NVFP4Linear(96, 80, seed=4, sign_mask=MASK, device="cuda", dtype=torch.float32)
    with torch.no_grad():
        lb.weight.copy_(la.weight)
    x = torch.from_numpy(workloads.normal(48, 96, 12)).cuda()
    x3 = x.reshape(2, 24, 96).clone().requires_grad_(True)
    x2 = x.clone().requires_grad_(True)
    dy = torch.from_numpy(workloads.laplace(48, 80, 13, 1e-3)).cuda()
    y3, y2 = la(x3), lb(x2)
    assert y3.shape == (2, 24, 80)
    y3.backward(dy.reshape(2, 24, 80))
    y2.backward(dy)
    torch.cuda.synchronize()
    assert torch.equal(y3.detach().reshape(48, 80), y2.detach())
    assert torch.equal(x3.grad.reshape(48, 96), x2.grad)
    assert torch.equal(la.weight.grad, lb.weight.grad)
    import gemm_amax_reduce_amd as nv
    with pytest.raises(nv.NVFP4Error, match="multiple of 16"):
        la(torch.zeros(3, 5, 96, device="cuda"))


def test_full_layer_shape_bf16():
    """The layer at the benchmark's large shape (8192 tokens, 5120 -> 20480,
    bf16): y, dx and dW on sampled rows and columns against the oracle's
    quantizations of the same tensors (x N(0,1), dy Laplace(1e-3))."""
    import gemm_amax_reduce_amd.linear as L
    tokens, fin, fout = 8192, 5120, 20480
    print(f"[linear] {tokens}x{fin} -> {fout} bf16", flush=True)
    torch.manual_seed(1)
    layer = L.NVFP4Linear(fin, fout, seed=0x5EED, sign_mask=MASK, device="cuda", dtype=torch.bfloat16)
    x = workloads.to_bf16(workloads.normal(tokens, fin, 31)).cuda().requires_grad_(True)
    dy = workloads.to_bf16(workloads.laplace(tokens, fout, 32, 1e-3)).cuda()
    y = layer(x)
    y.backward(dy)
    torch.cuda.synchronize()
    xc, wc, dyc = x.detach().cpu(), layer.weight.detach().cpu(), dy.cpu()
    rng = np.random.default_rng(33)

    def pick(n):
        return np.unique(np.concatenate([[0, n - 1], rng.choice(n, 64, replace=False)]))

    def check(got, qa, qb, label):
        rows, cols = pick(qa.outer), pick(qb.outer)
        c, b = oracle.gemm(qa, qb, rows, cols)
        sub = got[torch.as_tensor(rows, device=got.device)][:, torch.as_tensor(cols, device=got.device)]
        _within_bf16(sub, c, b, label)

    check(y.detach(), oracle.quantize(xc, axis=1), oracle.quantize(wc, axis=1), "y")
    check(x.grad, oracle.quantize(dyc, axis=1, rounding=oracle.SR, seed=0x5EED, offset=0),
          oracle.quantize(wc, axis=0), "dx")
    check(layer.weight.grad, oracle.quantize(dyc, axis=0, rounding=oracle.SR, seed=0x5EED, offset=1, rht=True,
                                             sign_mask=MASK),
          oracle.quantize(xc, axis=0, rht=True, sign_mask=MASK), "dW")


def test_gradients_needed_one_at_a_time():
    """A frozen weight (only dx) or an input without grad (only dW): the
    forward quantizes each operand in the layouts its gradients need, and
    the gradient it returns is bit-identical to the one of the layer with
    both gradients (same weight, seed and step)."""
    import gemm_amax_reduce_amd.linear as L
    x0 = torch.from_numpy(workloads.normal(64, 96, 14)).cuda()
    dy = torch.from_numpy(workloads.laplace(64, 80, 15, 1e-3)).cuda()
    layers = [L.NVFP4Linear(96, 80, seed=6, sign_mask=MASK, device="cuda", dtype=torch.float32) for _ in range(3)]
    with torch.no_grad():
        for la in layers[1:]:
            la.weight.copy_(layers[0].weight)
    xa = x0.clone().requires_grad_(True)
    ya = layers[0](xa)
    ya.backward(dy)
    layers[1].weight.requires_grad_(False)
    xb = x0.clone().requires_grad_(True)
    yb = layers[1](xb)
    yb.backward(dy)
    yc = layers[2](x0.clone())
    yc.backward(dy)
    torch.cuda.synchronize()
    assert torch.equal(ya.detach(), yb.detach()) and torch.equal(ya.detach(), yc.detach())
    assert torch.equal(xa.grad, xb.grad) and layers[1].weight.grad is None
    assert torch.equal(layers[0].weight.grad, layers[2].weight.grad)

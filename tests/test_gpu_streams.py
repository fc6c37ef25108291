"""The library keeps no state between calls, so work on two streams at once
gives the same bits as the same calls in sequence: the linear-layer step
with the backward operands of the forward tensors (W on axis 0, X on axis 0
with the transform) quantized on a second stream, released once the forward
quantizations are issued, while the fprop GEMM runs on the first, the dgrad
GEMM waiting for them (the schedule the benchmark's step uses), against the
one-stream step."""
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


def test_two_stream_step_matches_one_stream():
    import gemm_amax_reduce_amd as nv
    dev = torch.device("cuda", 0)
    mask, seed = workloads.rht_sign_mask(), workloads.SR_SEED
    x = workloads.to_bf16(workloads.normal(768, 512, 71)).to(dev)            # tokens x in
    w = workloads.to_bf16(workloads.normal(1280, 512, 72, std=0.02)).to(dev)  # out x in
    dy = workloads.to_bf16(workloads.laplace(768, 1280, 73, 1e-3)).to(dev)    # tokens x out
    qx, qw = nv.NVFP4Tensor.empty(768, 512), nv.NVFP4Tensor.empty(1280, 512)
    qdy, qdyt = nv.NVFP4Tensor.empty(768, 1280), nv.NVFP4Tensor.empty(1280, 768)
    qw0, qx0 = nv.NVFP4Tensor.empty(512, 1280), nv.NVFP4Tensor.empty(512, 768)
    y = torch.empty((768, 1280), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((768, 512), dtype=torch.float32, device=dev)
    dw = torch.empty((1280, 512), dtype=torch.float32, device=dev)
    main = torch.cuda.current_stream(dev)
    side = torch.cuda.Stream(device=dev)      # default priority

    def forward_quantize():
        nv.nvfp4_quantize(x, axis=1, out=qx)
        nv.nvfp4_quantize(w, axis=1, out=qw)

    def forward_gemm():
        nv.nvfp4_gemm(qx, qw, torch.bfloat16, out=y)

    def backward_operands():
        nv.nvfp4_quantize(w, axis=0, out=qw0)
        nv.nvfp4_rht_quantize(x, mask, axis=0, out=qx0)

    def backward():
        nv.nvfp4_quantize_dual(dy, rounding1="sr", seed1=seed, offset1=0, rht0=True, sign_mask0=mask,
                               rounding0="sr", seed0=seed, offset0=1, out1=qdy, out0=qdyt)
        nv.nvfp4_gemm(qdy, qw0, torch.float32, out=dx)
        nv.nvfp4_gemm(qdyt, qx0, torch.float32, out=dw)

    def snapshot():
        return [t.clone() for t in (y, dx, dw, qx.codes, qw0.codes, qw0.scales, qw0.meta, qx0.codes, qx0.scales,
                                    qx0.meta, qdy.codes, qdyt.codes)]

    forward_quantize()
    forward_gemm()
    backward_operands()
    backward()
    torch.cuda.synchronize()
    ref = snapshot()
    for t in (y, dx, dw, qw0.codes, qx0.codes):
        t.zero_()
    torch.cuda.synchronize()

    for _ in range(3):
        forward_quantize()
        release = torch.cuda.Event()
        release.record(main)
        side.wait_event(release)
        with torch.cuda.stream(side):
            backward_operands()
        done = torch.cuda.Event()
        done.record(side)
        forward_gemm()
        main.wait_event(done)
        backward()
        torch.cuda.synchronize()
        got = snapshot()
        for i, (a, b) in enumerate(zip(ref, got)):
            assert torch.equal(a, b), f"tensor {i} differs between one-stream and two-stream steps"

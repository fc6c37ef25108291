"""The library's calls can be captured in a HIP graph (they enqueue kernels
only: no allocation, no memset, no host synchronisation): a linear-layer
step captured once and replayed several times, with eager work and
synchronisations between the replays, gives bit-identical outputs to the
eager step every time."""
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


def test_step_graph_replays_match_eager():
    import gemm_amax_reduce_amd as nv
    dev = torch.device("cuda", 0)
    mask, seed = workloads.rht_sign_mask(), workloads.SR_SEED
    x = workloads.to_bf16(workloads.normal(512, 384, 61)).to(dev)          # tokens x in
    w = workloads.to_bf16(workloads.normal(640, 384, 62, std=0.02)).to(dev)  # out x in
    dy = workloads.to_bf16(workloads.laplace(512, 640, 63, 1e-3)).to(dev)    # tokens x out
    qx, qw = nv.NVFP4Tensor.empty(512, 384), nv.NVFP4Tensor.empty(640, 384)
    qdy, qdyt = nv.NVFP4Tensor.empty(512, 640), nv.NVFP4Tensor.empty(640, 512)
    qw0, qx0 = nv.NVFP4Tensor.empty(384, 640), nv.NVFP4Tensor.empty(384, 512)
    y = torch.empty((512, 640), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((512, 384), dtype=torch.float32, device=dev)
    dw = torch.empty((640, 384), dtype=torch.float32, device=dev)

    def step():
        nv.nvfp4_quantize(x, axis=1, out=qx)
        nv.nvfp4_quantize(w, axis=1, out=qw)
        nv.nvfp4_gemm(qx, qw, torch.bfloat16, out=y)
        nv.nvfp4_quantize_dual(dy, rounding1="sr", seed1=seed, offset1=0, rht0=True, sign_mask0=mask,
                               rounding0="sr", seed0=seed, offset0=1, out1=qdy, out0=qdyt)
        nv.nvfp4_quantize(w, axis=0, out=qw0)
        nv.nvfp4_gemm(qdy, qw0, torch.float32, out=dx)
        nv.nvfp4_rht_quantize(x, mask, axis=0, out=qx0)
        nv.nvfp4_gemm(qdyt, qx0, torch.float32, out=dw)

    def snapshot():
        return [t.clone() for t in (y, dx, dw, qdy.codes, qdy.scales, qdyt.codes, qx0.codes, qx0.meta, qw0.scales)]

    step()
    torch.cuda.synchronize()
    ref = snapshot()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (y, dx, dw, qdy.codes, qdyt.codes, qx0.codes):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for i, (a, b) in enumerate(zip(ref, got)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager step"
        step()                       # eager work between replays
        torch.cuda.synchronize()

"""nvfp4_gemm_noalloc -- the GEMM on the library's own workspace, for callers
that cannot allocate -- against the entry point it varies, nvfp4_gemm_ws
with a caller workspace, through the C ABI.

Two calls in a row, the second with a smaller input (both take the split
path, which uses the workspace: 6 tiles cut 5 ways, then 1 tile cut 4
ways), each in f32 and bf16: the outputs must equal nvfp4_gemm_ws's bit for
bit, and lie within the GEMM tolerance of the float64 oracle.  A repeat of
the first shape after the smaller one checks that the array's leftover
contents from the previous call do not leak into the next.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


def _nv():
    import gemm_amax_reduce_amd as nv
    nv.lib()
    return nv


def _upload(nv, ref):
    return nv.NVFP4Tensor(torch.from_numpy(ref.codes).cuda(), torch.from_numpy(ref.scales).cuda(),
                          torch.from_numpy(ref.meta).cuda(), ref.outer, ref.k)


def _operands(m, n, k, seed):
    xa = workloads.with_outliers(workloads.normal(m, k, seed), seed + 1, p=0.01)
    xb = workloads.normal(n, k, seed + 2) * np.float32(0.02)
    return oracle.quantize(xa, axis=1), oracle.quantize(xb, axis=1)


def test_noalloc_equals_workspace_entry_point():
    nv = _nv()
    L = nv.lib()
    ws = torch.zeros(int(L.nvfp4_gemm_workspace_bytes()), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for (m, n, k), seed in (((512, 768, 5120), 91), ((256, 256, 4096), 93), ((512, 768, 5120), 95)):
        ra, rb = _operands(m, n, k, seed)
        qa, qb = _upload(nv, ra), _upload(nv, rb)
        ca, cb = qa._c(), qb._c()
        for dt, code in ((torch.float32, 0), (torch.bfloat16, 1)):
            print(f"[no_alloc] {m}x{n}x{k} {dt}", flush=True)
            want = nv.nvfp4_gemm_ws(qa, qb, dt, workspace=ws)
            got = torch.full((m, n), 7.0, dtype=dt, device="cuda")
            rc = L.nvfp4_gemm_noalloc(ctypes.byref(ca), ctypes.byref(cb), got.data_ptr(), code, n, stream)
            assert rc == 0, L.nvfp4_status_string(rc)
            torch.cuda.synchronize()
            iv = torch.int32 if code == 0 else torch.int16
            assert torch.equal(got.view(iv), want.view(iv)), f"{m}x{n}x{k} {dt}: differs from nvfp4_gemm_ws"
            cref, bound = oracle.gemm(ra, rb)
            if code == 0:
                ok, worst = oracle.check_gemm_f32(got.cpu().double().numpy(), cref, bound, 1e-5)
                assert ok, f"worst |err|/bound {worst:.3e}"
            else:
                ok, nbad = oracle.check_gemm_bf16(got.cpu().double().numpy(), cref, bound, 1e-5)
                assert ok, f"{nbad} bf16 outputs outside the tolerance"


def test_noalloc_argument_errors():
    nv = _nv()
    L = nv.lib()
    ra, rb = _operands(64, 32, 64, 97)
    qa, qb = _upload(nv, ra), _upload(nv, rb)
    ca, cb = qa._c(), qb._c()
    c = torch.empty((64, 32), device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert L.nvfp4_gemm_noalloc(None, ctypes.byref(cb), c.data_ptr(), 0, 32, s) == -1
    assert L.nvfp4_gemm_noalloc(ctypes.byref(ca), ctypes.byref(cb), c.data_ptr(), 5, 32, s) == -3
    assert L.nvfp4_gemm_noalloc(ctypes.byref(ca), ctypes.byref(cb), c.data_ptr(), 0, 31, s) == -2

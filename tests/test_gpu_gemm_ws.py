"""GPU parity of the NVFP4 GEMM with a workspace (nvfp4_gemm_ws) against the
float64 oracle, and the accuracy of both GEMM entry points on same-sign
operands.

nvfp4_gemm_ws balances the last round of 256 x 256 tiles through the
caller's workspace: grids of at least one round take the stream-K tail
(the last one to two rounds' K groups dealt out in equal ranges; a tile is
the sum of at most two ranges), smaller grids the split tail (each tile
left over cut into equal K ranges), and the rest nvfp4_gemm's grid.  Shapes
here take every branch: few tiles split up to the per-range minimum (1, 4
and 6 tiles), stream-K on a ragged grid (4600 x 5120 x 8192: 360 tiles)
and on a ragged grid with K % 64 != 0 (4200 x 4000 x 4112: 272 tiles, per-
lane scale loads), the mixed grid (340 tiles of 8 K groups: too short for
stream-K; 20 tiles of 4 groups: too short to split), f32 and bf16 output,
and the three layer shapes (all stream-K).  Tolerance as for nvfp4_gemm:
every element within 1e-5 * gA gB sum_k |(qA SA)(qB SB)| of the oracle.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

RTOL = 1e-5
FLAG_BYTES = 32 << 10           # flag region of the workspace
ERR_OFFSET = 32 << 10           # error word (waits that gave up)


@functools.lru_cache(maxsize=None)
def _nv():
    import gemm_amax_reduce_amd as nv
    nv.lib()
    return nv


def _upload(ref):
    nv = _nv()
    return nv.NVFP4Tensor(torch.from_numpy(ref.codes).cuda(), torch.from_numpy(ref.scales).cuda(),
                          torch.from_numpy(ref.meta).cuda(), ref.outer, ref.k)


def _rand_q(outer, k, seed, scale=1.0):
    x = workloads.normal(outer, k, seed) * np.float32(scale)
    x = workloads.with_outliers(x, seed + 1, p=0.01)
    return oracle.quantize(x, axis=1)


def _check(c_gpu, ra, rb, out, rows=None, cols=None, label=""):
    cref, bound = oracle.gemm(ra, rb, rows, cols)
    if rows is not None:
        c_gpu = c_gpu[torch.as_tensor(rows)]
    if cols is not None:
        c_gpu = c_gpu[:, torch.as_tensor(cols)]
    if out == "f32":
        ok, worst = oracle.check_gemm_f32(c_gpu.double().numpy(), cref, bound, RTOL)
        print(f"[gemm_ws] {label}: worst |err|/bound = {worst:.3e}", flush=True)
        assert ok, f"{label}: worst |err|/bound = {worst:.3e} > {RTOL}"
        return worst
    ok, nbad = oracle.check_gemm_bf16(c_gpu.double().numpy(), cref, bound, RTOL)
    assert ok, f"{label}: {nbad} bf16 outputs outside the tolerance interval"
    return 0.0


def _workspace_clean(ws):
    """Flags back at zero and no wait gave up."""
    head = ws[:FLAG_BYTES + 4].cpu()
    assert int(head[:FLAG_BYTES].count_nonzero()) == 0, "flags left raised"
    assert int(head[ERR_OFFSET:ERR_OFFSET + 4].view(torch.int32)[0]) == 0, "a split-tile wait gave up"


def _gemm_ws(qa, qb, out, ws):
    nv = _nv()
    dt = torch.float32 if out == "f32" else torch.bfloat16
    c = nv.nvfp4_gemm_ws(qa, qb, dt, workspace=ws)
    torch.cuda.synchronize()
    return c.cpu()


@pytest.fixture(scope="module")
def ws():
    nv = _nv()
    return torch.zeros(int(nv.lib().nvfp4_gemm_workspace_bytes()), dtype=torch.uint8, device="cuda")


# (m, n, k): 1 tile K=4096 (split 4); 4 tiles K=5120 (split 5); 6 tiles
# K=2064 (K % 64 != 0, split 2); 20 tiles K=1024 (4 groups: no split); 360
# tiles K=8192 (stream-K, ragged M); 272 tiles K=4112 (stream-K, ragged M
# and N, K % 64 != 0); 340 tiles K=2048 (8 groups: the mixed grid); small
# ragged shapes; one element
SHAPES = [(256, 256, 4096), (512, 512, 5120), (300, 700, 2064), (1024, 1280, 1024),
          (4600, 5120, 8192), (4200, 4000, 4112), (4352, 5120, 2048), (200, 136, 272), (257, 129, 16), (3, 517, 48),
          (1, 1, 16)]


@pytest.mark.parametrize("m,n,k", SHAPES)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_split_shapes(ws, m, n, k, out):
    print(f"[gemm_ws] {m}x{n}x{k} {out}", flush=True)
    ra, rb = _rand_q(m, k, 61), _rand_q(n, k, 62, scale=0.01)
    c = _gemm_ws(_upload(ra), _upload(rb), out, ws)
    if m * n > 1 << 22:
        rows, cols = np.unique(np.r_[0, m - 1, np.arange(0, m, 17)]), np.unique(np.r_[0, n - 1, np.arange(0, n, 13)])
        _check(c, ra, rb, out, rows=rows, label=f"{m}x{n}x{k} rows")
        _check(c, ra, rb, out, cols=cols, label=f"{m}x{n}x{k} cols")
    else:
        _check(c, ra, rb, out, label=f"{m}x{n}x{k}")
    _workspace_clean(ws)


@pytest.mark.parametrize("m,n,k", [(512, 512, 5120), (4600, 5120, 8192)])
def test_deterministic_and_reusable(ws, m, n, k):
    """Bit-identical results over repeated calls with one workspace (split
    and stream-K tiles add their partials in a fixed order), the workspace
    clean after each."""
    ra, rb = _rand_q(m, k, 63), _rand_q(n, k, 64)
    qa, qb = _upload(ra), _upload(rb)
    first = _gemm_ws(qa, qb, "f32", ws)
    for _ in range(3):
        assert torch.equal(_gemm_ws(qa, qb, "f32", ws).view(torch.int32), first.view(torch.int32))
        _workspace_clean(ws)


@pytest.mark.parametrize("name", ["fprop", "dgrad", "wgrad"])
def test_layer_shapes(ws, name):
    """The three layer GEMMs (all three take the stream-K tail: 320, 640 and
    1600 tiles) on the oracle's operands, sampled rows and columns (every
    tile position) against the oracle."""
    g = workloads.GEMMS[name]
    mask = workloads.rht_sign_mask()
    refs = []
    for op in (g.a, g.b):
        r = oracle.SR if op.rounding == "sr" else oracle.RNE
        refs.append(oracle.quantize(op.generate(), axis=op.axis, rounding=r, seed=workloads.SR_SEED,
                                    offset=op.sr_offset, rht=op.rht, sign_mask=mask))
    m, n, _ = g.mnk
    rng = np.random.default_rng(5)
    rows = np.unique(np.r_[0, m - 1, rng.choice(m, 256, replace=False)])
    cols = np.unique(np.r_[0, n - 1, rng.choice(n, 256, replace=False)])
    c = _gemm_ws(_upload(refs[0]), _upload(refs[1]), g.out, ws)
    _check(c, refs[0], refs[1], g.out, rows=rows, label=f"{name} {g.out} rows")
    _check(c, refs[0], refs[1], g.out, cols=cols, label=f"{name} {g.out} cols")
    _workspace_clean(ws)


def test_workspace_argument_errors(ws):
    nv = _nv()
    qa, qb = _upload(_rand_q(64, 64, 5)), _upload(_rand_q(32, 64, 6))
    with pytest.raises(nv.NVFP4Error, match="workspace"):
        nv.nvfp4_gemm_ws(qa, qb, workspace=ws[:1024])
    need = int(nv.lib().nvfp4_gemm_workspace_bytes())
    big = torch.zeros(need + 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(nv.NVFP4Error, match="misaligned"):
        nv.nvfp4_gemm_ws(qa, qb, workspace=big[16:16 + need])


# ------------------------------------------- same-sign operands ----
#
# Zero-mean data lets successive f32 rounding errors cancel; non-negative
# operands (e.g. post-activation inputs) make every partial sum grow, the
# case where accumulated rounding is largest.  These print the worst
# |err| / sum|ab| of each entry point.

def _nonneg_q(outer, k, seed):
    return oracle.quantize(np.abs(workloads.normal(outer, k, seed)), axis=1)


@pytest.mark.parametrize("entry", ["gemm", "gemm_ws"])
def test_nonnegative_operands_at_layer_k(ws, entry):
    """|N(0,1)| operands at the dgrad reduction length K = 20480, a 512 x
    512 output (one K range for nvfp4_gemm; 20 ranges per tile for
    nvfp4_gemm_ws)."""
    nv = _nv()
    ra, rb = _nonneg_q(512, 20480, 71), _nonneg_q(512, 20480, 72)
    qa, qb = _upload(ra), _upload(rb)
    c = nv.nvfp4_gemm(qa, qb) if entry == "gemm" else nv.nvfp4_gemm_ws(qa, qb, workspace=ws)
    torch.cuda.synchronize()
    _check(c.cpu(), ra, rb, "f32", label=f"nonneg K=20480 {entry}")


def test_nonnegative_operands_largest_k_split(ws):
    """|N(0,1)| operands at the largest K (2^25 - 256): nvfp4_gemm_ws cuts
    the one tile into 256 ranges of 512 groups."""
    nv = _nv()
    k = (1 << 25) - 256
    ra, rb = _nonneg_q(3, k, 73), _nonneg_q(2, k, 74)
    c = nv.nvfp4_gemm_ws(_upload(ra), _upload(rb), workspace=ws)
    torch.cuda.synchronize()
    _check(c.cpu(), ra, rb, "f32", label=f"nonneg K={k} gemm_ws")
    _workspace_clean(ws)

"""Host-side checks of the NVFP4 linear layer: shape validation, and no CPU
fallback (a CPU tensor is refused before any library call)."""
import pytest
import torch

import gemm_amax_reduce_amd as nv
import gemm_amax_reduce_amd.linear as L


def test_feature_counts_must_be_block_multiples():
    with pytest.raises(nv.NVFP4Error):
        L.NVFP4Linear(24, 32)
    with pytest.raises(nv.NVFP4Error):
        L.NVFP4Linear(32, 40)


def test_cpu_tensors_are_refused():
    layer = L.NVFP4Linear(32, 16, dtype=torch.float32)
    with pytest.raises(nv.NVFP4Error, match="GPU"):
        layer(torch.zeros(16, 32))


def test_token_count_must_be_block_multiple():
    layer = L.NVFP4Linear(32, 16, dtype=torch.float32)
    with pytest.raises(nv.NVFP4Error, match="token"):
        layer(torch.zeros(8, 32))

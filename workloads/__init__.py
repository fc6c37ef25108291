"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds only random-number generation and the workload registry
(shapes, seeds, distributions).  It contains none of the quantizer or GEMM
arithmetic, and it imports neither the product package nor the oracle.

Recipe: numpy ``default_rng(seed)`` (PCG64) draws values in float32 (normal)
or float64 (Laplace, Student-t), in fixed row chunks of ``CHUNK_ROWS`` rows,
each chunk from its own child seed ``SeedSequence(seed).spawn``; the values
are scaled, cast to float32 and rounded to bfloat16 (nearest even) by torch.
The workload shapes are the linear-layer shapes of a 5120-wide model with a
20480-wide MLP (the published recipe trains a 12B hybrid Mamba-Transformer
on GB300; no layer dimensions are given there, these are the shapes of the
benchmark configuration).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

CHUNK_ROWS = 512

# random sign vector of the Hadamard transform: bit j set => s_j = -1
def rht_sign_mask(seed: int = 4) -> int:
    return int(np.random.default_rng(seed).integers(2 ** 16)) & 0xFFFF


SR_SEED = 0x5EED


def _chunks(rows: int):
    for r0 in range(0, rows, CHUNK_ROWS):
        yield r0, min(rows, r0 + CHUNK_ROWS)


def _rngs(seed: int, rows: int):
    n = (rows + CHUNK_ROWS - 1) // CHUNK_ROWS
    kids = np.random.SeedSequence(seed).spawn(max(n, 1))
    return [np.random.default_rng(k) for k in kids]


def normal(rows: int, cols: int, seed: int, std: float = 1.0) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.float32)
    for (r0, r1), g in zip(_chunks(rows), _rngs(seed, rows)):
        out[r0:r1] = g.standard_normal((r1 - r0, cols), dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def laplace(rows: int, cols: int, seed: int, scale: float) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.float32)
    for (r0, r1), g in zip(_chunks(rows), _rngs(seed, rows)):
        out[r0:r1] = g.laplace(0.0, scale, (r1 - r0, cols)).astype(np.float32)
    return out


def student_t(rows: int, cols: int, seed: int, nu: float) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.float32)
    for (r0, r1), g in zip(_chunks(rows), _rngs(seed, rows)):
        out[r0:r1] = g.standard_t(nu, (r1 - r0, cols)).astype(np.float32)
    return out


def with_outliers(x: np.ndarray, seed: int, p: float = 1e-3, factor: float = 50.0) -> np.ndarray:
    """Scale each entry independently by ``factor`` with probability ``p``."""
    rows, cols = x.shape
    for (r0, r1), g in zip(_chunks(rows), _rngs(seed, rows)):
        mask = g.random((r1 - r0, cols)) < p
        x[r0:r1][mask] *= np.float32(factor)
    return x


def mixed_rows(rows: int, cols: int, seed: int, nu: float = 3.0) -> np.ndarray:
    """Even rows N(0,1), odd rows Student-t(nu)."""
    out = np.empty((rows, cols), dtype=np.float32)
    ev = normal((rows + 1) // 2, cols, seed)
    od = student_t(rows // 2, cols, seed + 1, nu)
    out[0::2] = ev
    out[1::2] = od
    return out


def to_bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


# --------------------------------------------------------------------------
# workload registry
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Operand:
    name: str
    rows: int
    cols: int
    dtype: str          # "f32" or "bf16"
    dist: str           # "normal", "normal_outliers", "laplace", "mixed"
    seed: int
    std: float = 1.0
    mask_seed: int = 0
    axis: int = 1       # quantization axis (K = cols for axis 1, rows for axis 0)
    rounding: str = "rne"
    rht: bool = False
    sr_offset: int = 0

    def generate(self) -> torch.Tensor:
        if self.dist == "normal":
            x = normal(self.rows, self.cols, self.seed, self.std)
        elif self.dist == "normal_outliers":
            x = with_outliers(normal(self.rows, self.cols, self.seed, self.std), self.mask_seed)
        elif self.dist == "laplace":
            x = laplace(self.rows, self.cols, self.seed, self.std)
        elif self.dist == "mixed":
            x = mixed_rows(self.rows, self.cols, self.seed)
        else:
            raise ValueError(self.dist)
        if self.dtype == "f32":
            return torch.from_numpy(x)
        return to_bf16(x)


@dataclasses.dataclass(frozen=True)
class Gemm:
    name: str
    a: Operand          # [M, K] after its quantization view
    b: Operand          # [N, K] after its quantization view
    out: str            # "f32" or "bf16"

    @property
    def mnk(self):
        def view(op):
            return (op.rows, op.cols) if op.axis == 1 else (op.cols, op.rows)
        m, k = view(self.a)
        n, k2 = view(self.b)
        assert k == k2
        return m, n, k

    @property
    def flops(self) -> int:
        m, n, k = self.mnk
        return 2 * m * n * k


_DY = dict(rows=8192, cols=20480, dtype="bf16", dist="laplace", seed=20, std=1e-3)

TINY = Gemm("tiny",
            Operand("A", 128, 256, "f32", "normal", 0, axis=1),
            Operand("B", 256, 128, "f32", "normal", 1, axis=0),
            "f32")
FPROP = Gemm("fprop",
             Operand("X", 4096, 5120, "bf16", "normal_outliers", 10, mask_seed=12),
             Operand("W", 5120, 5120, "bf16", "normal", 11, std=0.02),
             "bf16")
DGRAD = Gemm("dgrad",
             Operand("dY", **_DY, axis=1, rounding="sr", sr_offset=0),
             Operand("W", 20480, 5120, "bf16", "normal", 21, std=0.02, axis=0),
             "f32")
WGRAD = Gemm("wgrad",
             Operand("X", 8192, 5120, "bf16", "normal_outliers", 30, mask_seed=32, axis=0, rht=True),
             Operand("dY", **_DY, axis=0, rounding="sr", rht=True, sr_offset=1),
             "f32")
SWEEP = Operand("T", 32768, 8192, "bf16", "mixed", 40)

GEMMS = {g.name: g for g in (TINY, FPROP, DGRAD, WGRAD)}

"""Pins of the MXFP4 oracle (blocks of 32 E2M1 elements sharing a power-of-two
scale, [P4] "Architektura NVFP4 kontra ograniczenia mikroskalowania").

* Scale rule (reading: the smallest 2^e with amax_b / 2^e <= 6): checked in
  exact rational arithmetic on random and boundary maxima.
* Round trip: blocks of grid values times one power of two (the block
  maximum 6 * 2^k) decode back exactly.
* Elements: each decoded value is the nearest grid point of x / 2^e (ties to
  the even code), by brute force over the grid.
* Storage: 4 + 8/32 = 4.25 bits per value, the 32-block figure the NVFP4
  storage test rules out for NVFP4.
"""
from fractions import Fraction

import numpy as np

import oracle

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _exact_rule(amax: float) -> int:
    a = Fraction(float(np.float32(amax)))
    e = -127
    while e < 127 and a > 6 * Fraction(2) ** e:
        e += 1
    return e


def test_scale_rule_exact():
    rng = np.random.default_rng(0)
    vals = list(np.float32(rng.lognormal(0, 8, 4000)))
    for k in range(-130, 128, 7):
        for m in (1.0, 1.5, 3.0, 6.0):
            v = np.float32(m * 2.0 ** k)
            if np.isfinite(v) and v > 0:
                vals += [v, np.nextafter(v, np.float32(np.inf)), np.nextafter(v, np.float32(0))]
    vals += [np.float32(0.0), np.float32(1e-45), np.finfo(np.float32).max]
    for v in vals:
        assert oracle.mx_scale_exp(float(v)) == _exact_rule(float(v)), v


def test_round_trip_of_scaled_grid_blocks():
    rng = np.random.default_rng(1)
    rows, cols = 6, 128
    x = np.zeros((rows, cols), dtype=np.float32)
    for r in range(rows):
        for b in range(cols // 32):
            k = int(rng.integers(-20, 20))
            blk = rng.choice(np.concatenate([GRID, -GRID]), size=32) * 2.0 ** k
            blk[int(rng.integers(32))] = 6.0 * 2.0 ** k * rng.choice([-1, 1])
            x[r, 32 * b:32 * b + 32] = blk
    q = oracle.mxfp4_quantize(x)
    np.testing.assert_array_equal(oracle.mxfp4_decode(q), x.astype(np.float64))


def test_elements_are_nearest_grid_points():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((16, 64)) * np.exp(rng.normal(0, 3, (16, 1)))).astype(np.float32)
    q = oracle.mxfp4_quantize(x)
    dec = oracle.mxfp4_decode(q)
    for o in range(16):
        for b in range(2):
            e = int(q.scales[o, b]) - 127
            for j in range(32):
                t = float(x[o, 32 * b + j]) * 2.0 ** -e
                d = np.abs(np.abs(t) - GRID)
                best = np.flatnonzero(d == d.min())
                pick = best[0] if len(best) == 1 else [i for i in best if i % 2 == 0][0]   # ties: even code
                assert abs(dec[o, 32 * b + j]) == GRID[pick] * 2.0 ** e, (o, b, j, t)


def test_zero_block_and_storage():
    x = np.zeros((2, 64), dtype=np.float32)
    x[1, 40] = 5.0
    q = oracle.mxfp4_quantize(x)
    assert q.scales[0, 0] == 0 and q.scales[0, 1] == 0 and q.scales[1, 0] == 0
    assert q.scales[1, 1] == 127             # 5 <= 6 * 2^0
    assert not q.codes[0].any()
    bits = 8 * (q.codes.nbytes + q.scales.nbytes) / x.size
    assert bits == 4.25


def test_axis0_is_axis1_of_transpose():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 96)).astype(np.float32)
    a = oracle.mxfp4_quantize(x, axis=0)
    b = oracle.mxfp4_quantize(np.ascontiguousarray(x.T), axis=1)
    np.testing.assert_array_equal(a.codes, b.codes)
    np.testing.assert_array_equal(a.scales, b.scales)


def test_gemm_oracle_is_a_matmul_of_decoded_operands():
    rng = np.random.default_rng(4)
    a = oracle.mxfp4_quantize(rng.standard_normal((8, 64)).astype(np.float32))
    b = oracle.mxfp4_quantize(rng.standard_normal((5, 64)).astype(np.float32))
    c, bound = oracle.mxfp4_gemm(a, b)
    da, db = oracle.mxfp4_decode(a), oracle.mxfp4_decode(b)
    naive = np.array([[sum(da[i, k] * db[j, k] for k in range(64)) for j in range(5)] for i in range(8)])
    np.testing.assert_allclose(c, naive, rtol=0, atol=1e-12)
    assert np.all(bound >= np.abs(c))

"""Pins of the oracle's stochastic rounding and its counter-based generator.

Philox4x32-10 is checked against rocRAND's own implementation (a library
routine compiled for the host); stochastic rounding against its closed-form
probability, the pages' worked example and unbiasedness statistics.
"""
import math
import os
from fractions import Fraction
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import workloads

HERE = os.path.dirname(os.path.abspath(__file__))


# ---------------------------------------------------------------- Philox --

@pytest.fixture(scope="module")
def rocrand_kat(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND helper")
    exe = str(tmp_path_factory.mktemp("kat") / "kat")
    subprocess.run([hipcc, "-O1", os.path.join(HERE, "helpers", "rocrand_philox_kat.cpp"),
                    "-o", exe], check=True, capture_output=True)

    def run(cases):
        lines = "".join(f"{s:x} {c[0]:x} {c[1]:x} {c[2]:x} {c[3]:x}\n" for s, c in cases)
        out = subprocess.run([exe], input=lines, capture_output=True, text=True, check=True).stdout
        return [[int(w, 16) for w in ln.split()] for ln in out.strip().splitlines()]
    return run


def test_philox_matches_rocrand(rocrand_kat):
    rng = np.random.default_rng(123)
    cases = [(0, (0, 0, 0, 0)), (workloads.SR_SEED, (0, 0, 0, 0)), (workloads.SR_SEED, (1, 0, 1, 0)),
             (0xFFFFFFFFFFFFFFFF, (0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF))]
    for _ in range(200):
        seed = int(rng.integers(0, 2 ** 63)) * 2 + int(rng.integers(0, 2))
        ctr = tuple(int(x) for x in rng.integers(0, 2 ** 32, 4))
        cases.append((seed, ctr))
    ref = rocrand_kat(cases)
    for (seed, ctr), r in zip(cases, ref):
        got = oracle.philox4x32_10(ctr, [seed & 0xFFFFFFFF, seed >> 32])
        assert list(got) == r, (hex(seed), ctr)


def test_sr_bits_counter_layout(rocrand_kat):
    # element i takes half (i%2) of word (i%8)//2 of the block for counter i//8
    seed, off = 0x5EED, 7
    for i in (0, 1, 2, 7, 8, 9, 1 << 33, (1 << 33) + 5):
        g = i >> 3
        w = oracle.philox4x32_10([g & 0xFFFFFFFF, g >> 32, off, 0], [seed, 0])
        word = int(w[(i & 7) >> 1])
        assert oracle.sr_bits(seed, off, i) == ((word >> 16) if i & 1 else (word & 0xFFFF))


def test_philox_bytes_uniform():
    words = np.concatenate([oracle.philox4x32_10([i, 0, 0, 0], [1, 2]) for i in range(4096)])
    b = words.view(np.uint8)
    counts = np.bincount(b, minlength=256)
    exp = b.size / 256
    chi2 = float(np.sum((counts - exp) ** 2 / exp))
    # 255 degrees of freedom: mean 255, sd ~22.6; 6 sd is far in the tail
    assert chi2 < 255 + 6 * math.sqrt(2 * 255)


# ---------------------------------------------------- stochastic rounding --

def _p_up_count(v, hi):
    return sum(oracle.e2m1_value(oracle.e2m1_sr(v, r)) == hi for r in range(65536))


@pytest.mark.parametrize("v", [0.1, 0.3, 0.74, 1.2, 1.7, 2.9, 3.2, 4.5, 5.99, 1.0000001, 5.9999995])
def test_sr_probability_closed_form(v):
    # Adding u = (r16 + 1/2) / 2^16 grid steps and truncating rounds up for
    # exactly the r16 >= 2^16 (1 - frac) - 1/2, i.e. floor(frac 2^16 + 1/2)
    # of the 2^16 values: P(up) is frac rounded to 16 bits (within 2^-17).
    v = float(np.float32(v))
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    lo = max(g for g in grid if g <= v)
    hi = grid[grid.index(lo) + 1]
    frac = Fraction(v) - Fraction(lo)
    frac /= Fraction(hi) - Fraction(lo)
    count = _p_up_count(v, hi)
    assert count == math.floor(frac * 65536 + Fraction(1, 2))
    assert abs(Fraction(count, 65536) - frac) <= Fraction(1, 2 ** 17)
    # the smallest offset (r16 = 0) rounds up only when frac >= 1 - 2^-17,
    # the largest (r16 = 0xFFFF) whenever frac >= 2^-17
    assert oracle.e2m1_value(oracle.e2m1_sr(v, 0)) == (hi if frac >= 1 - Fraction(1, 2 ** 17) else lo)
    assert oracle.e2m1_value(oracle.e2m1_sr(v, 0xFFFF)) == (hi if frac >= Fraction(1, 2 ** 17) else lo)


def test_sr_brute_force_add_and_truncate():
    # The definition written as arithmetic on exact rationals: value / step +
    # u, truncated, times step, over random values in every binade and
    # random 16-bit draws.
    rng = np.random.default_rng(17)
    grid = [Fraction(g) for g in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    vals = np.concatenate([rng.uniform(0, 6.5, 3000), np.exp2(rng.uniform(-40, 2.6, 1000))]).astype(np.float32)
    for v, r in zip(vals, rng.integers(0, 65536, vals.size)):
        a = Fraction(float(v))
        if a >= 6:
            want = Fraction(6)
        else:
            lo = max(g for g in grid if g <= a)
            hi = grid[grid.index(lo) + 1]
            step = hi - lo
            t = (a - lo) / step + (Fraction(int(r)) + Fraction(1, 2)) / 65536
            want = lo + step * (1 if t >= 1 else 0)
        assert Fraction(oracle.e2m1_value(oracle.e2m1_sr(float(v), int(r)))) == want, (float(v), int(r))


def test_sr_tiny_values_stay_zero():
    # |v| far below half a grid step: frac < 2^-17, so no draw rounds it up
    for v in (1e-30, -1e-30, 2.0 ** -20, np.float32(1e-40)):
        for r in (0, 1, 0x7FFF, 0xFFFF):
            assert oracle.e2m1_value(oracle.e2m1_sr(float(v), r)) == 0.0


def test_sr_worked_example_frequencies():
    # page 3 example value 3.2 between 3 and 4: stochastic rounding stores 3
    # with probability ~0.8 and 4 with ~0.2 so the mean stays at 3.2.
    v = np.float32(3.2)
    n = 1 << 20
    vals = np.array([oracle.e2m1_value(oracle.e2m1_sr(v, oracle.sr_bits(workloads.SR_SEED, 0, i)))
                     for i in range(n)])
    p4 = float(np.mean(vals == 4.0))
    assert set(np.unique(vals)) == {3.0, 4.0}
    sd = math.sqrt(0.2 * 0.8 / n)
    assert abs(p4 - (float(v) - 3.0)) < 5 * sd
    assert abs(vals.mean() - float(v)) < 5 * sd
    # ordinary rounding keeps the whole 0.2 as a systematic error
    assert oracle.e2m1_value(oracle.e2m1_rne(v)) == 3.0


def test_sr_saturates_and_keeps_sign():
    for r in (0, 0x8000, 0xFFFF):
        assert oracle.e2m1_sr(6.0, r) == 7
        assert oracle.e2m1_sr(100.0, r) == 7
        assert oracle.e2m1_sr(-100.0, r) == 15
        assert oracle.e2m1_sr(-0.0, r) == 8


def test_sr_tensor_unbiased_vs_rne_biased():
    # A Laplace tensor (the backward-pass gradient distribution of the dgrad
    # workload) quantized with SR: mean error of the decoded values is zero
    # within 5 standard errors.  A constant block of 3.2 (scaled so that
    # m = 1) shows the bias that RNE keeps and SR removes.
    x = workloads.laplace(256, 1024, seed=99, scale=1e-3)
    q = oracle.quantize(x, axis=1, rounding=oracle.SR, seed=workloads.SR_SEED, offset=3)
    xh = oracle.dequantize(q).astype(np.float64)
    err = xh - x.astype(np.float64)
    assert abs(err.mean()) < 5 * err.std() / math.sqrt(err.size)

    blk = np.full((64, 16), np.float32(3.2), dtype=np.float32)
    blk[:, 0] = 6.0                       # amax 6 -> s_enc = 448, S = 448, m = 1
    rne = oracle.dequantize(oracle.quantize(blk, rounding=oracle.RNE))[:, 1:]
    sr = oracle.dequantize(oracle.quantize(blk, rounding=oracle.SR, seed=1))[:, 1:]
    assert abs(rne.mean() - 3.2) > 0.19      # systematic -0.2
    assert abs(sr.mean() - 3.2) < 5 * 0.4 / math.sqrt(sr.size)

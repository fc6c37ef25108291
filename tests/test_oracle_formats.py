"""Pins of the oracle's number formats (E2M1 elements, E4M3 block scales).

Each test checks the oracle against something other than itself: the pages'
worked example, the IEEE-754 definition of round-to-nearest-even, brute force
over the whole format, or torch's float8_e4m3fn cast.
"""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

E2M1_SET = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([float(t) for t in line.split()])
    return rows


# ---------------------------------------------------------------- E2M1 ----

def test_e2m1_value_set():
    vals = [oracle.e2m1_value(c) for c in range(16)]
    assert vals[:8] == E2M1_SET
    assert vals[8:] == [-v for v in E2M1_SET]
    assert np.signbit(vals[8])  # code 0x8 is -0.0


def test_e2m1_codes_round_trip():
    for c in range(16):
        v = oracle.e2m1_value(c)
        assert oracle.e2m1_rne(v) == c
        for r16 in (0, 1, 0x7FFF, 0x8000, 0xFFFF):
            assert oracle.e2m1_sr(v, r16) == c


def test_worked_rounding_example():
    # page 3, "Warum weniger Bits ...": 3.2 is stored as 3, error 0.2
    lo, hi, value, stored, err = _golden("rounding_example.txt")[0]
    assert lo in E2M1_SET and hi in E2M1_SET
    assert E2M1_SET.index(hi) == E2M1_SET.index(lo) + 1  # 3 and 4 are neighbours
    code = oracle.e2m1_rne(np.float32(value))
    assert oracle.e2m1_value(code) == stored
    assert abs((float(np.float32(value)) - stored) - err) < 1e-6


def _ieee_e2m1(v: np.ndarray) -> np.ndarray:
    """E2M1 rounding derived from IEEE-754 float32 arithmetic: adding 2^22,
    2^23 or 2^24 leaves a float whose unit in the last place is the E2M1
    spacing of the binade (0.5 below 2, 1 in [2,4), 2 in [4,8)), so the
    hardware's round-to-nearest-even rounds |v| onto the grid with ties to
    the even mantissa bit; then saturate at 6."""
    a = np.minimum(np.abs(v.astype(np.float32)), np.float32(6.0))
    magic = np.where(a < 2, np.float32(2 ** 22), np.where(a < 4, np.float32(2 ** 23), np.float32(2 ** 24))).astype(np.float32)
    r = ((a + magic) - magic).astype(np.float32)
    idx = np.searchsorted(np.array(E2M1_SET, dtype=np.float32), r)
    assert np.all(np.array(E2M1_SET, dtype=np.float32)[idx] == r)
    return (idx | (np.signbit(v).astype(np.int64) << 3)).astype(np.uint8)


def _all_bf16_finite_f32():
    bits = np.arange(65536, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    return v[np.isfinite(v)]


def test_e2m1_rne_matches_ieee_on_all_bf16():
    v = _all_bf16_finite_f32()
    got = np.array([oracle.e2m1_rne(x) for x in v], dtype=np.uint8)
    np.testing.assert_array_equal(got, _ieee_e2m1(v))


def test_e2m1_rne_midpoints_and_neighbours():
    grid = np.array(E2M1_SET, dtype=np.float32)
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)
    pts = []
    for m in list(mids) + [np.float32(6.0), np.float32(7.0)]:
        pts += [np.nextafter(m, np.float32(0)), m, np.nextafter(m, np.float32(100))]
    pts = np.array(pts, dtype=np.float32)
    pts = np.concatenate([pts, -pts])
    got = np.array([oracle.e2m1_rne(x) for x in pts], dtype=np.uint8)
    np.testing.assert_array_equal(got, _ieee_e2m1(pts))


def test_e2m1_rne_ties_go_to_even_code():
    expect = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0,
              6.5: 6.0, 1e30: 6.0}
    for x, y in expect.items():
        assert oracle.e2m1_value(oracle.e2m1_rne(x)) == y
        assert oracle.e2m1_value(oracle.e2m1_rne(-x)) == -y


def test_e2m1_rne_sign_of_zero():
    assert oracle.e2m1_rne(-0.0) == 0x8
    assert oracle.e2m1_rne(-1e-30) == 0x8
    assert oracle.e2m1_rne(0.0) == 0x0


# ---------------------------------------------------------------- E4M3 ----

def _torch_e4m3_values():
    codes = torch.arange(256, dtype=torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()


def test_e4m3_decode_all_codes_vs_torch():
    ref = _torch_e4m3_values()
    got = np.array([oracle.e4m3_value(b) for b in range(256)], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def _torch_e4m3_rne(t: np.ndarray) -> np.ndarray:
    return torch.from_numpy(t.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_vs_torch():
    vals = _torch_e4m3_values()[:0x7F].astype(np.float64)  # 0 .. 448
    mids = (vals[:-1] + vals[1:]) / 2
    pts = []
    for m in mids:
        m32 = np.float32(m)
        pts += [np.nextafter(m32, np.float32(0)), m32, np.nextafter(m32, np.float32(1000))]
    rng = np.random.default_rng(7)
    pts += list(vals.astype(np.float32))
    pts += list((rng.random(20000) * 463.0).astype(np.float32))
    pts += list(np.exp2(rng.uniform(-14, 8.85, 20000)).astype(np.float32))
    pts += [np.float32(2.0 ** -10), np.float32(1e-30), np.float32(463.99)]
    pts = np.array(pts, dtype=np.float32)
    pts = pts[(pts >= 0) & (pts < 464)]
    got = np.array([oracle.e4m3_rne_sat(x) for x in pts], dtype=np.uint8)
    np.testing.assert_array_equal(got, _torch_e4m3_rne(pts))


def test_e4m3_encode_saturates():
    for t in (448.0, 463.0, 464.0, 470.0, 1e6, 3e38):
        assert oracle.e4m3_rne_sat(t) == 0x7E
    assert oracle.e4m3_rne_sat(0.0) == 0


def test_e4m3_encode_brute_force():
    vals = np.array([oracle.e4m3_value(b) for b in range(0x7F)], dtype=np.float64)
    rng = np.random.default_rng(11)
    pts = np.concatenate([rng.random(3000) * 470, np.exp2(rng.uniform(-12, 9, 3000))]).astype(np.float32)
    for t in pts:
        d = np.abs(vals - float(t))
        best = np.flatnonzero(d == d.min())
        # ties: even mantissa (even code) wins; beyond 448 saturate
        b = best[0] if best.size == 1 else [x for x in best if x % 2 == 0][0]
        assert oracle.e4m3_rne_sat(t) == b, (t, b)

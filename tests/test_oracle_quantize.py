"""Pins of the oracle's whole-tensor quantizer, dequantizer and GEMM.

Invariants that the format description fixes (16-element blocks, E4M3 block
scale, FP32 tensor level), special cases with exact answers, the storage
figure printed on the pages, a per-element error bound, library E4M3
rounding of the block scale, and exact rational brute force for the GEMM.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _codes_unpacked(q):
    lo = q.codes & 15
    hi = q.codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(q.outer, q.k)


def _view(x, axis):
    return x if axis == 1 else x.T


def _as_f32(x):
    if isinstance(x, torch.Tensor):
        return x.float().numpy()
    return x


# ------------------------------------------------------------ invariants --

@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("rht", [False, True])
def test_scale_invariants(axis, rht):
    x = workloads.with_outliers(workloads.normal(64, 96, 3), 4, p=0.01)
    q = oracle.quantize(x, axis=axis, rht=rht, sign_mask=0x3C5A)
    amax, g = q.amax, q.g
    y = _view(x, axis)
    if not rht:
        assert amax == np.abs(x).max()
    assert g == np.float32(np.float32(amax) / np.float32(2688.0))
    S = np.array([[oracle.e4m3_value(b) for b in row] for row in q.scales])
    assert S.max() == 448.0 and np.all(S <= 448.0)
    # the block holding the tensor maximum gets S = 448 and its maximum
    # element the largest code
    codes = _codes_unpacked(q)
    if not rht:
        o, k = np.unravel_index(np.argmax(np.abs(y)), y.shape)
        assert q.scales[o, k // 16] == 0x7E
        assert codes[o, k] & 7 == 7


def test_block_scale_is_library_e4m3_of_block_max():
    x = workloads.mixed_rows(32, 256, 21)
    q = oracle.quantize(x)
    bmax = np.abs(x).reshape(32, 16, 16).max(axis=2).astype(np.float32)
    k = np.float32(np.float32(448.0) / np.float32(q.amax))
    t = (bmax * k).astype(np.float32)
    ref = torch.from_numpy(np.minimum(t, np.float32(448.0))).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(q.scales, ref)


def test_zero_tensor():
    q = oracle.quantize(np.zeros((16, 32), dtype=np.float32))
    assert q.amax == 0.0 and q.g == 0.0
    assert not q.codes.any() and not q.scales.any()
    assert not oracle.dequantize(q).any()


def test_zero_block_in_nonzero_tensor():
    x = np.zeros((2, 32), dtype=np.float32)
    x[0, :16] = np.linspace(-3, 3, 16)
    x[1, 16] = -0.0
    q = oracle.quantize(x)
    assert q.scales[1, 0] == 0 and q.scales[1, 1] == 0
    c = _codes_unpacked(q)
    assert np.all(c[1] & 7 == 0)
    assert c[1, 16] == 8  # -0.0 keeps its sign bit
    assert np.all(oracle.dequantize(q)[1] == 0)


def test_worked_example_full_tensor():
    # page 3 "Warum weniger Bits ...": 3.2 between 3 and 4 is stored as 3.
    # With a block [6, 3.2, 0, ...] and tensor amax 6: s_enc = 448 and
    # S = 448 exactly, so the element multiplier is 1 and 3.2 -> code 5 (3).
    x = np.zeros((1, 16), dtype=np.float32)
    x[0, 0], x[0, 1] = 6.0, 3.2
    q = oracle.quantize(x)
    assert q.scales[0, 0] == 0x7E
    c = _codes_unpacked(q)
    assert c[0, 1] == 5
    xh = oracle.dequantize(q)
    # decode multiplies by g = fl(6/2688), itself rounded: 3 within 2 ulp
    assert abs(float(xh[0, 1]) - 3.0) <= 2 * 2.0 ** -22
    assert abs((float(x[0, 1]) - float(xh[0, 1])) - 0.2) < 1e-6


def test_exact_round_trip_construction():
    # every block holds a +-5.25, so amax = 5.25: g = 2^-9, s_enc = 512,
    # every S = 448, and entries +-q * 0.875 decode back bit-exactly
    rng = np.random.default_rng(2)
    qv = rng.choice(np.concatenate([GRID, -GRID]), size=(8, 64))
    x = (qv * 0.875).astype(np.float32)
    x[:, ::16] = np.where(rng.random((8, 4)) < 0.5, 5.25, -5.25)
    q = oracle.quantize(x)
    assert q.g == 2.0 ** -9 and np.all(q.scales == 0x7E)
    np.testing.assert_array_equal(oracle.dequantize(q), x)


def test_storage_ratio_matches_pages():
    # page 3 "Drei Formate, ein Trainingslauf": about 3.6x fewer bits than BF16
    with open(os.path.join(GOLDEN, "storage_ratio.txt")) as f:
        bf16_bits, factor, block = [float(t) for t in
                                    [ln for ln in f if ln.strip() and not ln.startswith("#")][0].split()]
    x = workloads.normal(64, 512, 1)
    q = oracle.quantize(x)
    bits_per_value = 8 * (q.codes.nbytes + q.scales.nbytes) / x.size
    assert bits_per_value == 4 + 8 / block == 4.5
    assert round(bf16_bits / bits_per_value, 1) == factor
    # a 32-element block with an 8-bit scale would not give 3.6
    assert round(bf16_bits / (4 + 8 / 32), 1) != factor


@pytest.mark.parametrize("rht", [False, True])
def test_axis0_is_axis1_of_transpose(rht):
    x = workloads.normal(48, 80, 13)
    a = oracle.quantize(x, axis=0, rht=rht, sign_mask=0x0F0F, rounding=oracle.SR, seed=5)
    b = oracle.quantize(np.ascontiguousarray(x.T), axis=1, rht=rht, sign_mask=0x0F0F, rounding=oracle.SR, seed=5)
    np.testing.assert_array_equal(a.codes, b.codes)
    np.testing.assert_array_equal(a.scales, b.scales)
    np.testing.assert_array_equal(a.meta, b.meta)


def test_bf16_input_equals_f32_of_same_values():
    x = workloads.to_bf16(workloads.normal(32, 64, 17))
    a = oracle.quantize(x)
    b = oracle.quantize(x.float())
    np.testing.assert_array_equal(a.codes, b.codes)
    np.testing.assert_array_equal(a.scales, b.scales)


def _rne_error_bound_ok(x, q, rht=False, mask=0):
    y = _view(_as_f32(x), 1).astype(np.float64)
    if rht:
        y = np.stack([np.concatenate([oracle.rht16(r[16 * b:16 * b + 16], mask)
                                      for b in range(r.size // 16)]) for r in y.astype(np.float32)]).astype(np.float64)
    xh = oracle.dequantize(q).astype(np.float64)
    S = np.array([[oracle.e4m3_value(b) for b in row] for row in q.scales]).repeat(16, axis=1)
    unit = S * q.g          # one grid unit in input scale
    v = np.abs(y) / np.where(unit > 0, unit, 1)
    # half the E2M1 spacing at |v|, plus any saturation overshoot past 6
    half = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0))
    allow = (half + np.maximum(0, v - 6)) * unit + 1e-5 * np.abs(y) + 1e-30
    return np.all(np.abs(y - xh) <= allow)


@settings(max_examples=25, deadline=None)
@given(outer=st.integers(1, 40), nb=st.integers(1, 12), logscale=st.floats(-20, 20),
       axis=st.integers(0, 1), seed=st.integers(0, 2 ** 31))
def test_rne_error_bound_property(outer, nb, logscale, axis, seed):
    rng = np.random.default_rng(seed)
    y = (rng.standard_normal((outer, 16 * nb)) * 2.0 ** logscale).astype(np.float32)
    x = y if axis == 1 else np.ascontiguousarray(y.T)
    q = oracle.quantize(x, axis=axis)
    assert _rne_error_bound_ok(y, q)
    assert np.all(np.array([[oracle.e4m3_value(b) for b in row] for row in q.scales]) <= 448)


def test_rht_error_bound():
    x = workloads.with_outliers(workloads.normal(32, 128, 31), 32, p=0.01)
    m = workloads.rht_sign_mask()
    assert _rne_error_bound_ok(x, oracle.quantize(x, rht=True, sign_mask=m), rht=True, mask=m)


def test_nonfinite_reported_in_meta():
    x = np.ones((4, 32), dtype=np.float32)
    x[2, 5] = np.inf
    assert np.isinf(oracle.quantize(x).amax)
    x[1, 1] = np.nan
    assert np.isnan(oracle.quantize(x).amax)


def test_rejects_bad_k():
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((4, 24), dtype=np.float32))


def test_dequantize_is_one_rounding_of_exact_product():
    x = workloads.normal(16, 64, 41)
    q = oracle.quantize(x)
    xh = oracle.dequantize(q)
    codes = _codes_unpacked(q)
    S = np.array([[Fraction(oracle.e4m3_value(b)) for b in row] for row in q.scales])
    g = Fraction(float(q.g))
    for o in range(0, 16, 5):
        for k in range(0, 64, 7):
            c = int(codes[o, k])
            exact = Fraction(oracle.e2m1_value(c)) * S[o, k // 16] * g
            assert xh[o, k] == np.float32(float(exact))  # float(Fraction) is correctly rounded
    bf = oracle.dequantize(q, oracle.BF16)
    ref = torch.from_numpy(xh).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bf, ref)


# ----------------------------------------------------------------- GEMM --

def test_gemm_matches_exact_rational_brute_force():
    rng = np.random.default_rng(3)
    a = (rng.standard_normal((5, 32)) * 3).astype(np.float32)
    b = (rng.standard_normal((32, 4)) * 0.01).astype(np.float32)
    qa = oracle.quantize(a, axis=1)
    qb = oracle.quantize(b, axis=0)
    c, bound = oracle.gemm(qa, qb)
    ca, cb = _codes_unpacked(qa), _codes_unpacked(qb)
    for m in range(5):
        for n in range(4):
            tot = Fraction(0)
            tab = Fraction(0)
            for k in range(32):
                va = Fraction(oracle.e2m1_value(int(ca[m, k]))) * Fraction(oracle.e4m3_value(int(qa.scales[m, k // 16]))) * Fraction(float(qa.g))
                vb = Fraction(oracle.e2m1_value(int(cb[n, k]))) * Fraction(oracle.e4m3_value(int(qb.scales[n, k // 16]))) * Fraction(float(qb.g))
                tot += va * vb
                tab += abs(va * vb)
            assert abs(Fraction(c[m, n]) - tot) <= Fraction(2 ** -50) * tab
            assert abs(Fraction(bound[m, n]) - tab) <= Fraction(2 ** -50) * tab


def test_gemm_equals_matmul_of_dequantized_within_f32_rounding():
    g = workloads.TINY
    A, B = g.a.generate(), g.b.generate()
    qa = oracle.quantize(A, axis=1)
    qb = oracle.quantize(B, axis=0)
    c, bound = oracle.gemm(qa, qb)
    da = oracle.dequantize(qa).astype(np.float64)
    db = oracle.dequantize(qb).astype(np.float64)
    # dequantized values carry one f32 rounding each, so the two agree to
    # ~2^-23 of the absolute sum
    assert np.all(np.abs(da @ db.T - c) <= 2 * 2 ** -23 * bound + 1e-30)


def test_block_partials_exact_in_f32():
    # (q_A S_A)(q_B S_B) has at most 12 significant bits and a 16-term block
    # sum at most 16 more bits of range: every block partial is exact in f32,
    # so an f32 accumulation only rounds once per 16-block.
    rng = np.random.default_rng(4)
    vals = np.array([oracle.e2m1_value(c) for c in range(16)])
    svals = np.array([oracle.e4m3_value(b) for b in range(0x7F)])
    for _ in range(2000):
        qa, qb = rng.choice(vals, 16), rng.choice(vals, 16)
        sa, sb = rng.choice(svals), rng.choice(svals)
        terms = (qa * sa) * (qb * sb)
        f32 = np.float32(0)
        for t in terms.astype(np.float32):
            f32 = np.float32(f32 + t)
        assert float(f32) == float(np.sum(terms))


def test_tolerance_checker_catches_planted_error():
    g = workloads.TINY
    qa = oracle.quantize(g.a.generate(), axis=1)
    qb = oracle.quantize(g.b.generate(), axis=0)
    c, bound = oracle.gemm(qa, qb)
    ok, _ = oracle.check_gemm_f32(c.astype(np.float32), c, bound)
    assert ok
    bad = c.copy()
    bad[3, 4] += 2e-5 * bound[3, 4]
    assert not oracle.check_gemm_f32(bad, c, bound)[0]
    ok16, _ = oracle.check_gemm_bf16(torch.from_numpy(c).to(torch.bfloat16).double().numpy(), c, bound)
    assert ok16


@pytest.mark.parametrize("axis", [0, 1])
def test_sr_counter_is_output_layout_index(axis):
    # Every element 3.2 in blocks whose maximum is 6 (so m = 1): each code is
    # 3 or 4, decided by the 16 random bits of output index i = o*K + k.
    outer, K, seed, off = 3, 48, 0xABC, 9
    y = np.full((outer, K), np.float32(3.2), dtype=np.float32)
    y[:, ::16] = 6.0
    x = y if axis == 1 else np.ascontiguousarray(y.T)
    q = oracle.quantize(x, axis=axis, rounding=oracle.SR, seed=seed, offset=off)
    c = _codes_unpacked(q)
    frac = Fraction(float(np.float32(3.2))) - 3
    for o in range(outer):
        for k in range(K):
            if k % 16 == 0:
                continue
            r = oracle.sr_bits(seed, off, o * K + k)
            up = frac + (Fraction(r) + Fraction(1, 2)) / 65536 >= 1
            assert c[o, k] == (6 if up else 5), (o, k)

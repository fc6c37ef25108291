"""Pins of the oracle's supplied-amax quantization (the tensor scale level
given by the caller instead of computed in step 2), by closed forms on the
exact round-trip construction: every block holds a +-5.25 and the other
entries are +-q * 0.875 for grid values q.

* amax supplied = the true amax: identical to the computed path.
* amax supplied = 10.5 (twice the true one): g = 2^-8, s_enc = 256, every
  block scale rounds to exactly 224 (E4M3 0x76) and every element still
  decodes back bit-exactly (q * 224 * 2^-8 = q * 0.875).
* amax supplied = 2.625 (half): g = 2^-10, s_enc = 1024, block scales
  saturate at 448, elements map to 2q and saturate at 6, so the decoded
  tensor is exactly clip(x, -2.625, 2.625).
"""
import numpy as np

import oracle

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)


def _fixture(seed=2, rows=8, cols=64):
    rng = np.random.default_rng(seed)
    qv = rng.choice(np.concatenate([GRID, -GRID]), size=(rows, cols))
    x = (qv * 0.875).astype(np.float32)
    x[:, ::16] = np.where(rng.random((rows, cols // 16)) < 0.5, 5.25, -5.25)
    return x


def test_supplied_true_amax_is_the_computed_path():
    x = _fixture()
    for rounding in (oracle.RNE, oracle.SR):
        a = oracle.quantize(x, rounding=rounding, seed=5)
        b = oracle.quantize(x, rounding=rounding, seed=5, amax=5.25)
        np.testing.assert_array_equal(a.codes, b.codes)
        np.testing.assert_array_equal(a.scales, b.scales)
        np.testing.assert_array_equal(a.meta, b.meta)


def test_supplied_larger_amax_round_trips():
    x = _fixture()
    q = oracle.quantize(x, amax=10.5)
    assert q.meta[0] == 10.5 and q.g == 2.0 ** -8
    assert np.all(q.scales == 0x76)          # 224 = 1.75 * 2^7
    np.testing.assert_array_equal(oracle.dequantize(q), x)


def test_supplied_smaller_amax_saturates_at_it():
    x = _fixture()
    q = oracle.quantize(x, amax=2.625)
    assert q.g == 2.0 ** -10
    assert np.all(q.scales == 0x7E)          # saturated at 448
    np.testing.assert_array_equal(oracle.dequantize(q), np.clip(x, -2.625, 2.625))

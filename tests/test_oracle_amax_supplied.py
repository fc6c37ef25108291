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


def test_slice_with_outer0_reproduces_its_rows():
    """A slice of output rows, quantized with the whole tensor's amax and its
    first row's global index, gets exactly the codes of those rows in the
    whole tensor (both axes, SR): the SR element index is the output-layout
    index o*K + k of the whole tensor."""
    import workloads
    x = workloads.normal(96, 160, seed=21)
    full = oracle.quantize(x, axis=1, rounding=oracle.SR, seed=9, offset=3)
    sub = oracle.quantize(x[40:72], axis=1, rounding=oracle.SR, seed=9, offset=3, amax=full.amax, outer0=40)
    np.testing.assert_array_equal(sub.codes, full.codes[40:72])
    np.testing.assert_array_equal(sub.scales, full.scales[40:72])
    full0 = oracle.quantize(x, axis=0, rounding=oracle.SR, seed=9, offset=3)
    sub0 = oracle.quantize(np.ascontiguousarray(x[:, 32:80]), axis=0, rounding=oracle.SR, seed=9, offset=3,
                           amax=full0.amax, outer0=32)
    np.testing.assert_array_equal(sub0.codes, full0.codes[32:80])
    # without the offset the draws differ
    sub_wrong = oracle.quantize(x[40:72], axis=1, rounding=oracle.SR, seed=9, offset=3, amax=full.amax)
    assert not np.array_equal(sub_wrong.codes, full.codes[40:72])


def test_outer0_shifts_the_counter_by_whole_rows():
    """One row at a large global index: each code equals the SR primitive
    applied with the Philox bits of element outer0*K + k."""
    x = np.full((1, 32), 0.3, dtype=np.float32)
    x[0, 0] = 6.0                       # amax 6: s_enc = 448, the block max maps to 6
    outer0 = (1 << 33) + 5              # element indices above 2^35: the counter's second word is used
    q = oracle.quantize(x, rounding=oracle.SR, seed=0x5EED, offset=7, amax=6.0, outer0=outer0)
    # second block: m_b = s_enc / S_b in binary32
    m = np.float32(448.0) / np.float32(oracle.e4m3_value(int(q.scales[0, 1])))
    for k in range(16, 32):
        v = np.float32(0.3) * m
        want = oracle.e2m1_sr(float(v), oracle.sr_bits(0x5EED, 7, outer0 * 32 + k))
        got = (q.codes[0, k // 2] >> (4 * (k & 1))) & 0xF
        assert got == want, (k, got, want)

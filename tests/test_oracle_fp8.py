"""Pins of the oracle's e4m3 arithmetic against the OCP 8-bit float definition: the code table's
closed-form values, round trips, ties to even, the range ends, and the per-row scaling."""
import numpy as np
import pytest

from oracle import dit_oracle as o


def test_e4m3_table_closed_forms():
    d = o.e4m3_decode
    assert d(0x00) == 0.0 and d(0x80) == 0.0
    assert d(0x38) == 1.0 and d(0x40) == 2.0 and d(0xB8) == -1.0
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0             # largest finite: 2^8 * 1.75
    assert d(0x08) == 2.0 ** -6                                 # smallest normal
    assert d(0x01) == 2.0 ** -9                                 # smallest subnormal: 2^-6 / 8
    assert d(0x07) == 7 * 2.0 ** -9
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0x3C) == 1.5 and d(0x3F) == 1.875


def test_e4m3_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    np.testing.assert_array_equal(o.e4m3_encode(o.e4m3_decode(codes)), codes)


def test_e4m3_rounding_ties_to_even_and_subnormals():
    e = o.e4m3_encode
    # 1.0625 lies halfway between 1.0 (code 0x38, even) and 1.125 (0x39): to 1.0
    assert e(1.0625) == 0x38
    # 1.1875 lies halfway between 1.125 (0x39) and 1.25 (0x3A, even): to 1.25
    assert e(1.1875) == 0x3A
    assert e(1.07) == 0x39 and e(-1.07) == 0xB9
    # half the smallest subnormal is a tie with zero (even): 0; just above it rounds up
    assert e(2.0 ** -10) == 0x00 and e(1.01 * 2.0 ** -10) == 0x01
    assert e(448.0) == 0x7E and e(449.0) == 0x7E and e(463.9) == 0x7E
    # rounding keeps the sign: a negative value below half the smallest subnormal becomes -0
    assert e(-1e-5) == 0x80 and e(1e-5) == 0x00 and e(-0.0) == 0x80 and e(0.0) == 0x00
    with pytest.raises(ValueError):
        e(464.0)


def test_quantize_rows_maps_the_row_max_to_448_and_bounds_the_error():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((6, 100)).astype(np.float32) * np.float32(3.0)
    x[2] = 0.0
    q, s = o.quantize_fp8_rows(x)
    assert s[2] == 1.0 and np.all(q[2] == 0)
    for r in (0, 1, 3, 4, 5):
        j = np.argmax(np.abs(x[r]))
        assert abs(o.e4m3_decode(q[r, j])) == 448.0
        # relative error of a normal e4m3 value: at most 2^-4 (half a unit of the 3-bit mantissa)
        back = o.e4m3_decode(q[r]) * s[r]
        big = np.abs(x[r]) >= 2.0 ** -6 * s[r]
        assert np.all(np.abs(back - x[r])[big] <= 2.0 ** -4 * np.abs(x[r])[big] * (1 + 1e-6))


def test_linear_fp8_brute_force():
    rng = np.random.default_rng(2)
    xq = rng.integers(0, 0x7E, size=(3, 5)).astype(np.uint8)
    wq = (rng.integers(0, 0x7E, size=(4, 5)) | 0x80 * rng.integers(0, 2, size=(4, 5))).astype(np.uint8)
    sx, sw = np.array([0.5, 2.0, 1.25]), np.array([1.0, 0.25, 3.0, 0.125])
    want = np.array([[sum(o.e4m3_decode(xq[i, k]) * o.e4m3_decode(wq[j, k]) for k in range(5)) * sx[i] * sw[j]
                      for j in range(4)] for i in range(3)])
    np.testing.assert_allclose(o.linear_fp8(xq, sx, wq, sw), want, rtol=1e-15)


def _representable_rows(rng, rows, cols):
    """Rows of e4m3 values times a power of two per row, each row holding +-448 * 2^k once, so the
    per-row scale is exactly 2^k and every scaled value is an e4m3 value."""
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    vals = o.e4m3_decode(rng.choice(finite, size=(rows, cols)))
    vals[:, rng.integers(0, cols, rows)] = 0.0
    vals[np.arange(rows), rng.integers(0, cols, rows)] = 448.0 * rng.choice([-1.0, 1.0], rows)
    return vals * np.power(2.0, rng.integers(-12, 4, rows))[:, None]


def test_fp8_product_is_exact_on_representable_operands():
    # e4m3 values scaled by powers of two survive the per-row quantisation unchanged, so the fp8
    # product must equal the exact one there (up to float64 summation order)
    rng = np.random.default_rng(7)
    x, w = _representable_rows(rng, 9, 64), _representable_rows(rng, 5, 64)
    np.testing.assert_allclose(o._product(x, w, True), x @ w.T, rtol=1e-12, atol=0)
    np.testing.assert_array_equal(o._product(x, w, False), x @ w.T)


def test_fp8_product_error_within_e4m3_rounding_bound():
    # each operand element moves by at most half an e4m3 step: 2^-4 of its magnitude in the normal
    # range, 2^-10 of its row scale in the subnormal range -- so the product error is bounded by
    # sum_k (ex |w| + |x| ew + ex ew); a dropped scale, a transposed operand or a wrong row's scale
    # breaks it
    rng = np.random.default_rng(8)
    x = rng.standard_normal((12, 96)) * np.exp(rng.uniform(-3, 3, (12, 1)))
    w = rng.standard_normal((10, 96)) * 0.02
    sx = np.max(np.abs(x), axis=1, keepdims=True) / 448.0
    sw = np.max(np.abs(w), axis=1, keepdims=True) / 448.0
    ex = np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * sx) * (1 + 1e-6)
    ew = np.maximum(2.0 ** -4 * np.abs(w), 2.0 ** -10 * sw) * (1 + 1e-6)
    bound = ex @ np.abs(w).T + np.abs(x) @ ew.T + ex @ ew.T
    err = np.abs(o._product(x, w, True) - x @ w.T)
    assert np.all(err <= bound)
    assert np.max(err / bound) > 0.05          # the bound is not vacuous
    # and the fp8 block differs from the exact block only through these products
    y = o._product(x, w, True)
    assert not np.allclose(y, x @ w.T, rtol=1e-3)

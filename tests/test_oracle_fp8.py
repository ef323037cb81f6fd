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


# --- fp8 joint attention -------------------------------------------------------------------------

def _codes(rng, shape, lo=0x30, hi=0x78):
    return (rng.integers(lo, hi, size=shape) | (rng.integers(0, 2, size=shape) << 7)).astype(np.uint8)


def test_fp8_attention_brute_force():
    # plain loops with math.exp on the decoded values: per-token q scales, per-head k and v scales,
    # head slicing, the softmax scale -- a scale applied on the wrong axis or head fails here
    import math
    rng = np.random.default_rng(11)
    n, H, D = 5, 2, 4
    q8, k8, v8 = _codes(rng, (n, H * D)), _codes(rng, (n, H * D)), _codes(rng, (n, H * D))
    sq = rng.uniform(0.001, 0.01, (n, H)).astype(np.float32)
    sk = np.array([0.004, 0.007], np.float32)
    sv = np.array([0.5, 0.25], np.float32)
    scale = 0.37
    dec = o.e4m3_decode
    want = np.zeros((n, H * D))
    for h in range(H):
        for i in range(n):
            s = [sum(float(sq[i, h]) * dec(q8[i, h * D + c]) * float(sk[h]) * dec(k8[j, h * D + c])
                     for c in range(D)) * scale for j in range(n)]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            for c in range(D):
                want[i, h * D + c] = sum(w[j] * float(sv[h]) * dec(v8[j, h * D + c]) for j in range(n)) / sum(w)
    got = o.joint_attention_fp8(q8, sq, k8, sk, v8, sv, H, D, scale=scale)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-15)
    rows = np.array([3, 0])
    np.testing.assert_allclose(o.joint_attention_fp8(q8, sq, k8, sk, v8, sv, H, D, scale=scale, q_rows=rows),
                               want[rows], rtol=1e-12, atol=1e-15)


def test_fp8_attention_equal_scores_give_the_mean_of_v():
    # identical keys: every weight is exactly 1 (e4m3 holds 1), so both forms return mean(V)
    rng = np.random.default_rng(12)
    n, H, D = 9, 2, 8
    q8, v8 = _codes(rng, (n, H * D)), _codes(rng, (n, H * D))
    k8 = np.repeat(_codes(rng, (1, H * D)), n, axis=0)
    sq = rng.uniform(0.001, 0.01, (n, H))
    sk, sv = np.array([0.01, 0.02]), np.array([0.5, 3.0])
    v = o.e4m3_decode(v8) * np.repeat(sv, D)[None, :]
    for round_p in (False, True):
        got = o.joint_attention_fp8(q8, sq, k8, sk, v8, sv, H, D, round_p=round_p)
        np.testing.assert_allclose(got, np.broadcast_to(v.mean(axis=0), got.shape), rtol=1e-14)


def test_fp8_attention_dominant_key_and_constant_v():
    rng = np.random.default_rng(13)
    n, H, D = 6, 1, 8
    # key 2 equals the query direction scaled up: its score exceeds every other by > 30, so its
    # weight is 1 and every other weight is below 2^-40 -- O is V_2 (exact form), and the rounded
    # model drops the others entirely (they round to 0): O = V_2 / (1 + tiny)
    q8 = np.full((n, D), 0x38, np.uint8)                      # all ones
    k8 = _codes(rng, (n, D), 0x30, 0x38)                      # |k| in [0.5, 1)
    k8 &= 0x7F                                                # positive
    k8[2] = 0x58                                              # 8.0
    v8 = _codes(rng, (n, D))
    sq, sk, sv = np.ones((n, 1)), np.array([1.0]), np.array([0.125])
    for rp in (False, True):
        got = o.joint_attention_fp8(q8, sq, k8, sk, v8, sv, H, D, scale=1.0, round_p=rp)
        np.testing.assert_allclose(got, np.broadcast_to(0.125 * o.e4m3_decode(v8[2]), got.shape), rtol=1e-12)
    # V constant per feature: the exact form returns that row for every query, whatever the scores
    v8c = np.repeat(_codes(rng, (1, D)), n, axis=0)
    got = o.joint_attention_fp8(_codes(rng, (n, D)), rng.uniform(0.01, 0.1, (n, 1)), _codes(rng, (n, D)),
                                np.array([0.05]), v8c, np.array([2.0]), H, D)
    np.testing.assert_allclose(got, np.broadcast_to(2.0 * o.e4m3_decode(v8c[0]), got.shape), rtol=1e-13)


def test_fp8_attention_rounded_weights_closed_form():
    # two keys with scaled scores 0 and ln 0.3: weights 1 and 0.3; e4m3 holds 1 and rounds 0.3 =
    # 1.2 * 2^-2 to 1.25 * 2^-2 = 0.3125, the normaliser stays 1.3:
    # O = (V_1 + 0.3125 V_2) / 1.3 for the rounded model, (V_1 + 0.3 V_2) / 1.3 exactly
    import math
    rng = np.random.default_rng(15)
    D = 8
    q8 = np.full((2, D), 0x38, np.uint8)                      # ones
    k8 = np.zeros((2, D), np.uint8)
    k8[1] = 0x38                                              # key 1: q.k = 8, key 0: 0
    v8 = _codes(rng, (2, D))
    v = 0.5 * o.e4m3_decode(v8)
    args = (q8, np.ones((2, 1)), k8, np.array([1.0]), v8, np.array([0.5]), 1, D)
    scale = math.log(0.3) / 8
    got = o.joint_attention_fp8(*args, scale=scale, round_p=True, q_rows=np.array([0]))
    np.testing.assert_allclose(got[0], (v[0] + 0.3125 * v[1]) / 1.3, rtol=1e-13)
    got = o.joint_attention_fp8(*args, scale=scale, q_rows=np.array([0]))
    np.testing.assert_allclose(got[0], (v[0] + 0.3 * v[1]) / 1.3, rtol=1e-13)


def test_fp8_attention_rounding_shift():
    # a whole shift is a power-of-two scaling, exact in e4m3's normal range: shift 3 rounds the
    # closed-form pair above the same way (0.3 * 8 = 2.4 -> 2.5 = 0.3125 * 8); a shift of
    # log2(1.25) turns the largest weight 1 into 1.25 (exact) and 0.3 into 0.375 (exact): no
    # rounding at all, so the model equals the exact form
    import math
    rng = np.random.default_rng(16)
    D = 8
    q8 = np.full((2, D), 0x38, np.uint8)
    k8 = np.zeros((2, D), np.uint8)
    k8[1] = 0x38
    v8 = _codes(rng, (2, D))
    v = 0.5 * o.e4m3_decode(v8)
    args = (q8, np.ones((2, 1)), k8, np.array([1.0]), v8, np.array([0.5]), 1, D)
    scale = math.log(0.3) / 8
    got = o.joint_attention_fp8(*args, scale=scale, round_p=True, q_rows=np.array([0]), p_shift=np.array([[3.0]]))
    np.testing.assert_allclose(got[0], (v[0] + 0.3125 * v[1]) / 1.3, rtol=1e-13)
    got = o.joint_attention_fp8(*args, scale=scale, round_p=True, q_rows=np.array([0]),
                                p_shift=np.array([[math.log2(1.25)]]))
    np.testing.assert_allclose(got[0], (v[0] + 0.3 * v[1]) / 1.3, rtol=1e-13)


def test_fp8_attention_scale_moves_between_factors():
    # s = sq sk scale q.k: moving a factor of 2 from sk to scale, or from sq to sk, changes nothing
    rng = np.random.default_rng(14)
    n, H, D = 7, 2, 16
    q8, k8, v8 = _codes(rng, (n, H * D)), _codes(rng, (n, H * D)), _codes(rng, (n, H * D))
    sq = rng.uniform(0.001, 0.01, (n, H))
    sk, sv = np.array([0.01, 0.02]), np.array([0.5, 3.0])
    a = o.joint_attention_fp8(q8, sq, k8, sk, v8, sv, H, D, scale=0.3)
    np.testing.assert_allclose(o.joint_attention_fp8(q8, sq, k8, sk * 2, v8, sv, H, D, scale=0.15), a, rtol=1e-12)
    np.testing.assert_allclose(o.joint_attention_fp8(q8, sq * 2, k8, sk / 2, v8, sv, H, D, scale=0.3), a,
                               rtol=1e-12)


def test_fp8_attention_rounded_weights_within_the_e4m3_bound():
    # each weight w in (0, 1] moves by at most max(2^-4 w, 2^-10) (half a step, normal or
    # subnormal), so |O_round - O| <= sum_j max(2^-4 w_j, 2^-10) |V_j| / sum_j w_j per element
    import dit_inputs as di
    x = di.fp8_attention_inputs(96, 2, seed=3)
    H, D = 2, 128
    exact = o.joint_attention_fp8(x["q8"], x["sq"], x["k8"], x["sk"], x["v8"], x["sv"], H, D)
    rnd = o.joint_attention_fp8(x["q8"], x["sq"], x["k8"], x["sk"], x["v8"], x["sv"], H, D, round_p=True)
    q = o.e4m3_decode(x["q8"]) * np.repeat(x["sq"].astype(np.float64), D, axis=1)
    k = o.e4m3_decode(x["k8"]) * np.repeat(x["sk"].astype(np.float64), D)[None, :]
    v = o.e4m3_decode(x["v8"]) * np.repeat(x["sv"].astype(np.float64), D)[None, :]
    worst = 0.0
    for h in range(H):
        c = slice(h * D, (h + 1) * D)
        s = q[:, c] @ k[:, c].T / np.sqrt(D)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        bound = np.maximum(2.0 ** -4 * w, 2.0 ** -10) @ np.abs(v[:, c]) / w.sum(axis=1, keepdims=True)
        err = np.abs(rnd[:, c] - exact[:, c])
        assert np.all(err <= bound * (1 + 1e-9))
        worst = max(worst, float(np.max(err / bound)))
    assert worst > 0.05                    # the bound is not vacuous
    assert not np.allclose(rnd, exact, rtol=1e-3)


# --- the fp8 blocks' attention operands -----------------------------------------------------------

def test_fp8_attention_operands_scales_and_codes():
    rng = np.random.default_rng(21)
    n, H, D = 10, 3, 16
    q = rng.standard_normal((n, H * D)) * np.exp(rng.uniform(-2, 2, (n, 1)))
    k = rng.standard_normal((n, H * D)) * 0.3
    v = rng.standard_normal((n, H * D)) * np.repeat(np.array([0.5, 0.0, 7.0]), D)[None, :]
    kmax = 1.25
    q8, sq, k8, sk, v8, sv = o.fp8_attention_operands(q, k, v, H, D, kmax)
    for h in range(H):
        c = slice(h * D, (h + 1) * D)
        # q: every (token, head) row's largest magnitude lands on +-448
        np.testing.assert_array_equal(np.max(np.abs(o.e4m3_decode(q8[:, c])), axis=1), 448.0)
        np.testing.assert_allclose(sq[:, h], np.max(np.abs(q[:, c]), axis=1) / 448.0, rtol=1e-6)
    # k: one static scale per head from the weight bound
    np.testing.assert_array_equal(sk, np.float32(np.float32(1.25) * np.float32(np.sqrt(128.0) / 448.0)))
    # v: the zero head gets scale 1 and zero codes, the others map their max to 448
    assert sv[1] == 1.0 and np.all(o.e4m3_decode(v8[:, D:2 * D]) == 0.0)
    for h in (0, 2):
        c = slice(h * D, (h + 1) * D)
        assert np.max(np.abs(o.e4m3_decode(v8[:, c]))) == 448.0
    # every operand within half an e4m3 step of its value (normal range) or of the scale's subnormal step
    for x, codes, scale in ((q, q8, np.repeat(sq, D, axis=1)), (k, k8, sk[0]), (v, v8, np.repeat(sv, D)[None, :])):
        back = o.e4m3_decode(codes) * scale
        tol = np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * scale) * (1 + 1e-5)
        assert np.all(np.abs(back - x) <= tol)


def test_fp8_attention_k_bound_is_tight():
    # the worst case of the bound: a one-hot head vector, RMS-normed at position 0 (no rotation),
    # times the largest weight, reaches sqrt(128) * max|w| (less eps): its code is 448 (0x7E)
    H, D = 1, 128
    w = np.ones((1, 2, D))
    w[0, 1, 0] = 1.5                        # k weight, dim 0 the largest
    x = np.zeros((1, D))
    x[0, 0] = 3.0
    pos = np.zeros((1, 4), np.int32)
    q, k = o.qk_rmsnorm_rope(x.copy(), x.copy(), H, D, w, 1, 1e-6, pos, (32, 32, 32, 32), 1e4)
    assert abs(k[0, 0] - np.sqrt(128.0) * 1.5) < 1e-3        # eps shaves 7e-6 relative
    _, _, k8, sk, _, _ = o.fp8_attention_operands(q, k, np.zeros((1, D)), H, D, 1.5)
    assert k8[0, 0] == 0x7E
    # random normed, rotated k never leaves the range
    rng = np.random.default_rng(22)
    n = 64
    wr = 1.0 + 0.3 * rng.standard_normal((1, 2, D))
    kk = rng.standard_normal((n, D)) * np.exp(rng.uniform(-3, 3, (n, 1)))
    kk[np.arange(n) % 7 == 0] *= 0
    kk[np.arange(n) % 7 == 0, rng.integers(0, D, (n + 6) // 7)] = 1.0       # one-hot rows
    posr = rng.integers(0, 64, (n, 4)).astype(np.int32)
    _, kn = o.qk_rmsnorm_rope(kk.copy(), kk.copy(), H, D, wr, n, 1e-6, posr, (32, 32, 32, 32), 1e4)
    kw = float(np.max(np.abs(wr[0, 1])))
    s_k = np.float32(np.float32(kw) * o.K_BOUND_PER_WEIGHT)
    assert np.max(np.abs(kn)) / s_k <= 448.0 * (1 + 1e-6)
    _, _, k8r, _, _, _ = o.fp8_attention_operands(kn, kn, np.zeros_like(kn), H, D, kw)
    assert not np.any(np.isnan(o.e4m3_decode(k8r)))

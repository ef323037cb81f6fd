"""Pins of the oracle's 2-D convolution: a 1x1 kernel is a per-pixel linear layer, the centre-tap
identity kernel copies the input, brute force on a tiny image, the zero border, and translation in
the interior."""
import numpy as np

from oracle import dit_oracle as o


def test_1x1_is_a_linear_layer():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 3, 4, 5))
    w = rng.standard_normal((6, 1, 1, 5))
    b = rng.standard_normal(6)
    np.testing.assert_allclose(o.conv2d_nhwc(x, w, b), o.linear(x.reshape(-1, 5), w.reshape(6, 5)).reshape(2, 3, 4, 6) + b,
                               rtol=1e-13)


def test_centre_tap_identity_copies_the_input():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((1, 5, 6, 4))
    w = np.zeros((4, 3, 3, 4))
    w[:, 1, 1, :] = np.eye(4)
    np.testing.assert_array_equal(o.conv2d_nhwc(x, w), x)


def test_brute_force_tiny():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 4, 5, 3))
    w = rng.standard_normal((2, 3, 3, 3))
    b = np.array([0.5, -1.0])
    y = o.conv2d_nhwc(x, w, b)
    for bb in range(2):
        for h in range(4):
            for ww in range(5):
                for co in range(2):
                    acc = b[co]
                    for i in range(3):
                        for j in range(3):
                            hh, wj = h + i - 1, ww + j - 1
                            if 0 <= hh < 4 and 0 <= wj < 5:
                                acc += float(np.dot(x[bb, hh, wj], w[co, i, j]))
                    assert abs(y[bb, h, ww, co] - acc) < 1e-12


def test_zero_border_single_pixel_spreads_the_flipped_kernel():
    # one unit pixel at (0, 0): output (h, w) sees it through tap (1 - h, 1 - w), nothing else
    x = np.zeros((1, 4, 4, 1))
    x[0, 0, 0, 0] = 1.0
    w = np.arange(1.0, 10.0).reshape(1, 3, 3, 1)
    y = o.conv2d_nhwc(x, w)[0, :, :, 0]
    want = np.zeros((4, 4))
    want[0, 0], want[0, 1], want[1, 0], want[1, 1] = w[0, 1, 1, 0], w[0, 1, 0, 0], w[0, 0, 1, 0], w[0, 0, 0, 0]
    np.testing.assert_array_equal(y, want)


def test_translation_in_the_interior():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, 8, 9, 2))
    w = rng.standard_normal((3, 3, 3, 2))
    y = o.conv2d_nhwc(x, w)
    y2 = o.conv2d_nhwc(np.roll(x, 1, axis=2), w)
    np.testing.assert_allclose(y2[:, 1:7, 2:8], y[:, 1:7, 1:7], rtol=1e-13)


# ---- causal 3-D convolution ----------------------------------------------------------------------

def test_causal3d_with_one_frame_tap_is_the_2d_convolution_per_frame():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((2, 3, 4, 5, 3))
    w = rng.standard_normal((4, 1, 3, 3, 3))
    b = rng.standard_normal(4)
    y = o.conv3d_causal_nhwc(x, w, b)
    y2 = o.conv2d_nhwc(x.reshape(6, 4, 5, 3), w[:, 0], b).reshape(2, 3, 4, 5, 4)
    np.testing.assert_allclose(y, y2, rtol=1e-13, atol=1e-13)


def test_causal3d_ignores_future_frames():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((1, 5, 3, 4, 2))
    w = rng.standard_normal((3, 3, 3, 3, 2))
    y = o.conv3d_causal_nhwc(x, w)
    for t in range(5):
        x2 = x.copy()
        x2[:, t + 1:] = rng.standard_normal(x2[:, t + 1:].shape)
        np.testing.assert_array_equal(o.conv3d_causal_nhwc(x2, w)[:, :t + 1], y[:, :t + 1])
    # and frame t does depend on frame t - KT + 1
    x3 = x.copy()
    x3[:, 1] += 1.0
    assert not np.allclose(o.conv3d_causal_nhwc(x3, w)[:, 3], y[:, 3])


def test_causal3d_temporal_one_hot_shifts_frames():
    # only tap s = KT-1-d is nonzero: output frame t is the 2-D convolution of frame t - d
    # (zeros for t < d)
    rng = np.random.default_rng(13)
    x = rng.standard_normal((1, 4, 3, 3, 2))
    w2 = rng.standard_normal((2, 3, 3, 2))
    for d in range(3):
        w = np.zeros((2, 3, 3, 3, 2))
        w[:, 2 - d] = w2
        y = o.conv3d_causal_nhwc(x, w)
        for t in range(4):
            want = np.zeros((1, 3, 3, 2)) if t < d else o.conv2d_nhwc(x[:, t - d], w2)
            np.testing.assert_allclose(y[:, t], want, rtol=1e-13, atol=1e-13)


def test_causal3d_brute_force_tiny():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((1, 3, 3, 4, 2))
    w = rng.standard_normal((2, 2, 3, 1, 2))          # KT = 2, KH = 3, KW = 1
    b = np.array([0.25, -0.5])
    y = o.conv3d_causal_nhwc(x, w, b)
    for t in range(3):
        for h in range(3):
            for ww in range(4):
                for co in range(2):
                    acc = b[co]
                    for s in range(2):
                        for i in range(3):
                            tt, hh = t + s - 1, h + i - 1
                            if tt >= 0 and 0 <= hh < 3:
                                acc += float(np.dot(x[0, tt, hh, ww], w[co, s, i, 0]))
                    assert abs(y[0, t, h, ww, co] - acc) < 1e-12

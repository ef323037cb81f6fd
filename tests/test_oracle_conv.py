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

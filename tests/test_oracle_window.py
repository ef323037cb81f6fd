"""Pins of the oracle's neighborhood (windowed) attention: the boundary rule of the windows, the
page's statement that an axis narrower than the window is attended in full, the single-key window,
and brute force on a tiny grid."""
import numpy as np

from oracle import dit_oracle as o


def test_window_start_rule():
    # interior: centred; near the edges: shifted inwards, never shrunk
    assert [o.window_start(i, 3, 8) for i in range(8)] == [0, 0, 1, 2, 3, 4, 5, 5]
    assert [o.window_start(i, 5, 6) for i in range(6)] == [0, 0, 0, 1, 1, 1]
    # an axis narrower than the window: the whole axis (start 0, width = extent)
    assert [o.window_start(i, 7, 4) for i in range(4)] == [0, 0, 0, 0]
    for n in (1, 2, 5, 9, 16):
        for k in (1, 3, 5, 11):
            for i in range(n):
                s = o.window_start(i, k, n)
                ke = min(k, n)
                assert 0 <= s and s + ke <= n and s <= i < s + ke


def _qkv(n, heads, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, heads * 128)) for _ in range(3))


def test_window_wider_than_every_axis_is_full_attention():
    # the page's edge case: grid [1, 4, 4], kernel [3, 7, 7] clamps every axis
    q, k, v = _qkv(16, 2, 1)
    got = o.neighborhood_attention(q, k, v, (1, 4, 4), (3, 7, 7), 2, 128)
    np.testing.assert_allclose(got, o.joint_attention(q, k, v, 2, 128), rtol=1e-12, atol=1e-12)


def test_single_key_window_returns_v():
    q, k, v = _qkv(2 * 3 * 4, 1, 2)
    np.testing.assert_allclose(o.neighborhood_attention(q, k, v, (2, 3, 4), (1, 1, 1), 1, 128), v, rtol=0, atol=0)


def test_brute_force_tiny_grid():
    grid, kernel = (2, 5, 6), (1, 3, 5)
    q, k, v = _qkv(60, 1, 3)
    got = o.neighborhood_attention(q, k, v, grid, kernel, 1, 128, q_rows=[0, 7, 29, 59])
    T, H, W = grid
    for r_i, r in enumerate([0, 7, 29, 59]):
        t, h, w = r // (H * W), (r // W) % H, r % W
        # window by enumeration: the kernel[a] consecutive positions that contain the query,
        # centred when both halves fit, otherwise flush with the nearer edge
        keys = []
        for kt in range(T):
            for kh in range(H):
                for kw in range(W):
                    ok = True
                    for i, j, kk, n in ((t, kt, kernel[0], T), (h, kh, kernel[1], H), (w, kw, kernel[2], W)):
                        ke = min(kk, n)
                        lo = i - kk // 2
                        if lo < 0:
                            lo = 0
                        if lo + ke > n:
                            lo = n - ke
                        ok &= lo <= j < lo + ke
                    if ok:
                        keys.append((kt * H + kh) * W + kw)
        s = np.array([float(np.dot(q[r], k[j])) / np.sqrt(128.0) for j in keys])
        p = np.exp(s - s.max())
        p /= p.sum()
        want = sum(pi * v[j] for pi, j in zip(p, keys))
        np.testing.assert_allclose(got[r_i], want, rtol=1e-12, atol=1e-12)
        assert len(keys) == min(kernel[0], T) * min(kernel[1], H) * min(kernel[2], W)


def test_translation_inside_the_interior():
    # far from the edges a window is the centred box: shifting the whole grid content by one
    # column shifts the output of an interior query by one column
    grid, kernel = (1, 9, 12), (1, 3, 3)
    q, k, v = _qkv(108, 1, 4)
    r = 4 * 12 + 5
    a = o.neighborhood_attention(q, k, v, grid, kernel, 1, 128, q_rows=[r])
    roll = lambda x: np.roll(x.reshape(9, 12, -1), 1, axis=1).reshape(108, -1)
    b = o.neighborhood_attention(roll(q), roll(k), roll(v), grid, kernel, 1, 128, q_rows=[r + 1])
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)

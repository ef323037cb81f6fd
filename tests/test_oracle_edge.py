"""Pins of the oracle's layers either side of the block stack (timestep embedding, MLP embedder,
linear, LayerNorm, final layer): closed forms, invariants and brute force on tiny inputs."""
import math

import numpy as np

from oracle import dit_oracle as o


def test_timestep_embedding_t0_is_cos_one_sin_zero():
    e = o.timestep_embedding(0.0, 256)
    assert e.shape == (256,)
    np.testing.assert_array_equal(e[:128], np.ones(128))
    np.testing.assert_array_equal(e[128:], np.zeros(128))


def test_timestep_embedding_closed_form_dim4():
    # half = 2, frequencies 1 and max_period^(-1/2) = 0.1 for max_period = 100
    t, tf = 0.37, 1000.0
    s = tf * t
    want = [math.cos(s), math.cos(0.1 * s), math.sin(s), math.sin(0.1 * s)]
    np.testing.assert_allclose(o.timestep_embedding(t, 4, max_period=100.0, time_factor=tf), want,
                               rtol=0, atol=1e-12)


def test_timestep_embedding_pairs_have_unit_norm_and_first_frequency_is_one():
    e = o.timestep_embedding(0.731, 256)
    np.testing.assert_allclose(e[:128] ** 2 + e[128:] ** 2, np.ones(128), rtol=0, atol=1e-12)
    assert abs(e[0] - math.cos(731.0)) < 1e-9 and abs(e[128] - math.sin(731.0)) < 1e-9
    # the last frequency is max_period^(-(half-1)/half)
    f_last = 10000.0 ** (-127 / 128)
    assert abs(e[127] - math.cos(731.0 * f_last)) < 1e-12


def _brute_matvec(w, v):
    out = []
    for r in range(len(w)):
        acc = 0.0
        for k in range(len(v)):
            acc += float(w[r][k]) * float(v[k])
        out.append(acc)
    return np.array(out)


def test_mlp_embedder_brute_force_and_identity():
    rng = np.random.default_rng(1)
    v = rng.standard_normal(6)
    w_in = rng.standard_normal((5, 6))
    w_out = rng.standard_normal((5, 5))
    h = _brute_matvec(w_in, v)
    h = [x / (1.0 + math.exp(-x)) for x in h]
    np.testing.assert_allclose(o.mlp_embedder(v, w_in, w_out), _brute_matvec(w_out, h), rtol=1e-12, atol=1e-12)
    # identity weights: SiLU(v) itself
    eye = np.eye(6)
    np.testing.assert_allclose(o.mlp_embedder(v, eye, eye), [x / (1.0 + math.exp(-x)) for x in v], rtol=1e-14)


def test_conditioning_vector_closed_forms():
    """Closed forms of c = W_t,out SiLU(W_t,in emb(t)) [+ W_g,out SiLU(W_g,in emb(g))]."""
    sig1 = 1.0 / (1.0 + math.exp(-1.0))               # SiLU(1) = sigma(1) = 0.7310585786300049
    # t = 0: emb = [1, 1, 0, 0] (cosines of 0 first); W_in picks emb[0] and emb[2] -> hidden (1, 0)
    w_in = np.array([[1.0, 0, 0, 0], [0, 0, 1.0, 0]])
    w_out = np.array([[2.0, 0], [0, 3.0]])
    np.testing.assert_allclose(o.conditioning_vector(0.0, w_in, w_out, 4), [2.0 * sig1, 0.0], rtol=0, atol=1e-15)
    # t = 0.25, factor 1000, max_period 100, dim 4: s = 250, frequencies 1 and 0.1
    # emb = [cos 250, cos 25, sin 250, sin 25]; identity MLP weights give SiLU(emb) itself
    e = [math.cos(250.0), math.cos(25.0), math.sin(250.0), math.sin(25.0)]
    eye = np.eye(4)
    ct = o.conditioning_vector(0.25, eye, eye, 4, max_period=100.0)
    # (the oracle's frequency 100^(-1/2) carries a rounding of ~1e-17, times s = 250: atol 1e-12)
    np.testing.assert_allclose(ct, [v / (1.0 + math.exp(-v)) for v in e], rtol=0, atol=1e-12)
    # guidance g = 0.5 (s = 500) through its own weights: W_g,in selects sin(500 * 0.1) = sin 50 into
    # hidden 0, W_g,out doubles it into output 3
    wg_in = np.zeros((4, 4)); wg_in[0, 3] = 1.0
    wg_out = np.zeros((4, 4)); wg_out[3, 0] = 2.0
    both = o.conditioning_vector(0.25, eye, eye, 4, g=0.5, w_g_in=wg_in, w_g_out=wg_out, max_period=100.0)
    s50 = math.sin(50.0)
    want = [v / (1.0 + math.exp(-v)) for v in e]
    want[3] += 2.0 * s50 / (1.0 + math.exp(-s50))
    np.testing.assert_allclose(both, want, rtol=0, atol=1e-12)


def test_linear_brute_force_and_one_hot_rows():
    rng = np.random.default_rng(3)
    x, w = rng.standard_normal((3, 7)), rng.standard_normal((4, 7))
    want = np.array([[sum(x[i, k] * w[j, k] for k in range(7)) for j in range(4)] for i in range(3)])
    np.testing.assert_allclose(o.linear(x, w), want, rtol=1e-12, atol=1e-12)
    sel = np.zeros((2, 7)); sel[0, 5] = 1.0; sel[1, 2] = 1.0      # row j of W picks input column
    np.testing.assert_array_equal(o.linear(x, sel), x[:, [5, 2]])


def test_layer_norm_closed_form_and_moments():
    np.testing.assert_allclose(o.layer_norm(np.array([1.0, 2.0, 3.0]), 0.0),
                               [-math.sqrt(1.5), 0.0, math.sqrt(1.5)], rtol=1e-14)
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 64)) * 3.0 + 1.5
    y = o.layer_norm(x, 0.0)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose((y ** 2).mean(axis=1), 1.0, rtol=1e-12)
    # affine invariance (eps = 0): LN(a x + b) = LN(x) for a > 0
    np.testing.assert_allclose(o.layer_norm(2.5 * x - 7.0, 0.0), y, rtol=1e-12, atol=1e-12)
    # a constant row normalises to zero (eps > 0)
    np.testing.assert_array_equal(o.layer_norm(np.full((1, 8), 3.0), 1e-6), np.zeros((1, 8)))


def test_final_layer_zero_modulation_and_chunk_order():
    rng = np.random.default_rng(5)
    d, p = 8, 4
    x = rng.standard_normal((3, d))
    cond = rng.standard_normal(6)
    w_out = rng.standard_normal((p, d))
    ln = o.layer_norm(x, 1e-6)
    # zero modulation: LayerNorm then the projection
    np.testing.assert_allclose(o.final_layer(x, cond, np.zeros((2 * d, 6)), w_out), ln @ w_out.T, rtol=1e-12)
    # shift chunk first: only the first d rows of W_mod set, shift_i = SiLU(c_0) for every i
    w_mod = np.zeros((2 * d, 6)); w_mod[:d, 0] = 1.0
    sh = cond[0] / (1.0 + math.exp(-cond[0]))
    np.testing.assert_allclose(o.final_layer(x, cond, w_mod, w_out), (ln + sh) @ w_out.T, rtol=1e-12)
    # scale = -1 (second chunk) leaves only the shift: y = shift W_out^T for every row
    w_mod = np.zeros((2 * d, 6)); w_mod[d:, 1] = 1.0; w_mod[:d, 0] = 1.0
    c = cond.copy(); c[1] = -50.0    # SiLU(-50) ~ -1.9e-21: scale ~ 0 -> plain (LN + shift)
    np.testing.assert_allclose(o.final_layer(x, c, w_mod, w_out), (ln + sh) @ w_out.T, rtol=1e-12)
    w_id = np.eye(d)
    m = np.zeros((2 * d, 6)); m[d:, 2] = 1.0
    c2 = np.zeros(6); c2[2] = 1.0
    scale = 1.0 / (1.0 + math.exp(-1.0))
    np.testing.assert_allclose(o.final_layer(x, c2, m, w_id), (1.0 + scale) * ln, rtol=1e-12)

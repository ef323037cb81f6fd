"""Pins of the fp64 oracle against facts fixed outside it (CPU only).

Each test checks a closed form, an invariant of the definition, a library
routine on a special case, or brute force on a tiny input, so that a plausible
mistake in the oracle (a dropped term, a wrong sign, index or axis, a swapped
operand or chunk) fails at least one of them.  ``test_oracle_mutations.py``
plants such mistakes and checks that they are caught.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import dit_inputs as di
from oracle import dit_oracle as o

GOLD = os.path.join(os.path.dirname(__file__), "golden")
AXES = (32, 32, 32, 32)
THETA = 1e4


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _val(tok, g):
    return {"cos1": g["cos1"], "sin1": g["sin1"], "-sin1": -g["sin1"], "1": 1.0}[tok]


def tiny_cfg(**kw):
    base = dict(name="tiny", dtype="f32", d=256, n_heads=2, ffn_inner=768, n_txt=3,
                grid_h=2, grid_w=3)
    base.update(kw)
    return di.BlockConfig(**base)


# --- storage ----------------------------------------------------------------------

def test_widen_bf16_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x3C23], dtype=np.uint16)
    want = np.array([1.0, -1.0, 3.140625, 0.0, 0.0099487304688])
    np.testing.assert_allclose(o.widen(bits, "bf16"), want, rtol=0, atol=1e-13)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(o.widen(bits, "bf16"), t)


# --- SiLU / SwiGLU / AdaLN ------------------------------------------------------------

def test_silu_closed_forms():
    g = _load("elementwise_closed_forms.json")
    for z, want in g["silu"]:
        assert o.silu(np.array([z]))[0] == pytest.approx(want, abs=1e-15)


def test_silu_vs_library():
    z = np.linspace(-30, 30, 2001)
    ref = torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    np.testing.assert_allclose(o.silu(z), ref, rtol=1e-14, atol=1e-300)


def test_swiglu_gate_is_first_argument():
    g = np.array([1.0, -1.0, 0.0])
    u = np.array([2.0, 3.0, 5.0])
    np.testing.assert_allclose(o.swiglu(g, u), [2 * 0.7310585786300049, -3 * 0.2689414213699951, 0.0],
                               rtol=1e-15)


def test_adaln_modulation_one_hot_rows():
    # row r of W_mod picks cond[j] with weight w -> m_r = w * SiLU(cond[j])
    d_c = 5
    cond = np.array([0.0, 1.0, -1.0, 2.0, 1.0986122886681098])
    w = np.zeros((6, d_c))
    w[0, 1] = 1.0
    w[1, 2] = -2.0
    w[2, 4] = 4.0
    w[3, 0] = 7.0
    w[4, 3] = 0.5
    w[5, 1] = 1.0
    w[5, 2] = 1.0
    m = o.adaln_modulation(w, cond)
    want = [0.7310585786300049, 2 * 0.2689414213699951, 4 * 0.8239592165010823, 0.0,
            0.5 * 2 / (1 + math.exp(-2)), 0.7310585786300049 - 0.2689414213699951]
    np.testing.assert_allclose(m, want, rtol=1e-14, atol=1e-16)


def test_adaln_modulate_chunks_and_identity():
    rng = np.random.default_rng(1)
    d, d_c = 8, 4
    cond = rng.standard_normal(d_c)
    x = rng.standard_normal((3, d))
    w = np.zeros((3 * d, d_c))
    m, a = o.adaln_modulate(cond, w, 3, d, x=x, shift_chunk=0, scale_chunk=1, eps=1e-6)
    np.testing.assert_array_equal(m, 0)
    np.testing.assert_allclose(a, o.rms_norm(x, 1e-6), rtol=1e-15)
    # shift = chunk 0, scale = chunk 1 (identity for scale = 0, affine otherwise)
    w[:d, 0] = 1.0          # shift_k = SiLU(c0)
    w[d:2 * d, 1] = 1.0     # scale_k = SiLU(c1)
    m, a = o.adaln_modulate(cond, w, 3, d, x=x, eps=1e-6)
    s0, s1 = o.silu(cond[0]), o.silu(cond[1])
    np.testing.assert_allclose(a, (1 + s1) * o.rms_norm(x, 1e-6) + s0, rtol=1e-14)


# --- RMSNorm ---------------------------------------------------------------------------

def test_rmsnorm_closed_form_1_to_128():
    g = _load("elementwise_closed_forms.json")["rmsnorm_1_to_128"]
    x = np.arange(1, 129, dtype=np.float64)
    np.testing.assert_allclose(o.rms_norm(x, 1e-6), x / math.sqrt(g["mean_square"] + 1e-6), rtol=1e-15)


def test_rmsnorm_unit_rms_scale_invariance_and_eps():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 128))
    eps = 1e-6
    n = o.rms_norm(x, eps)
    ms = np.mean(x * x, axis=1)
    np.testing.assert_allclose(np.sqrt(np.mean(n * n, axis=1)), np.sqrt(ms / (ms + eps)), rtol=1e-13)
    np.testing.assert_allclose(o.rms_norm(1000 * x, 0.0), o.rms_norm(x, 0.0), rtol=1e-13)
    # eps inside the square root: a row with mean square == eps has RMS 1/sqrt(2)
    tiny = np.full((1, 128), 1e-3)
    assert np.sqrt(np.mean(o.rms_norm(tiny, 1e-6) ** 2)) == pytest.approx(1 / math.sqrt(2), rel=1e-12)


def test_rmsnorm_vs_library():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((40, 3072)) * 3
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (3072,), eps=1e-6).numpy()
    np.testing.assert_allclose(o.rms_norm(x, 1e-6), ref, rtol=1e-13)


# --- RoPE ---------------------------------------------------------------------------------

def test_rope_frequencies_closed_form():
    g = _load("rope_closed_forms.json")
    om = o.rope_frequencies(32, THETA)
    assert om.shape == (16,)
    for j, want in g["omega"].items():
        assert om[int(j)] == pytest.approx(want, rel=1e-14)


def test_rope_basis_vectors_closed_form():
    g = _load("rope_closed_forms.json")
    for case in g["cases"]:
        x = np.zeros((1, 128))
        x[0, case["in_dim"]] = 1.0
        y = o.rope_rotate(x, np.array([case["pos"]]), AXES, THETA)[0]
        want = np.zeros(128)
        for dim, tok in case["out"].items():
            want[int(dim)] = _val(tok, g)
        np.testing.assert_allclose(y, want, rtol=0, atol=1e-12, err_msg=case["note"])


def test_rope_general_angle_closed_form():
    # axis 1, pair 2 (dims 36, 37), row 2: angle 2 * 10^(-1/2)
    x = np.zeros((1, 128))
    x[0, 36], x[0, 37] = 0.6, -0.8
    y = o.rope_rotate(x, np.array([[0, 2, 0, 0]]), AXES, THETA)[0]
    phi = 2 * 10 ** -0.5
    assert y[36] == pytest.approx(0.6 * math.cos(phi) + 0.8 * math.sin(phi), abs=1e-14)
    assert y[37] == pytest.approx(0.6 * math.sin(phi) - 0.8 * math.cos(phi), abs=1e-14)
    assert np.count_nonzero(np.abs(y) > 1e-15) == 2


def test_rope_norm_identity_composition():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, 3, 128))
    p1 = rng.integers(0, 600, size=(64, 4))
    p2 = rng.integers(0, 600, size=(64, 4))
    y = o.rope_rotate(x, p1, AXES, THETA)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)
    np.testing.assert_array_equal(o.rope_rotate(x, np.zeros((64, 4), int), AXES, THETA), x)
    np.testing.assert_allclose(o.rope_rotate(y, p2, AXES, THETA), o.rope_rotate(x, p1 + p2, AXES, THETA),
                               rtol=0, atol=1e-11)


def test_rope_axis_ownership_and_interleaving():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((1, 128))
    for a in range(4):
        pos = np.zeros((1, 4), int)
        pos[0, a] = 5
        y = o.rope_rotate(x, pos, AXES, THETA)
        changed = np.nonzero(np.abs(y - x)[0] > 1e-12)[0]
        assert changed.min() >= 32 * a and changed.max() < 32 * (a + 1)
    # pair (2j, 2j+1): e_{2j} rotates into e_{2j+1} only (not into e_{j+16})
    e = np.zeros((1, 128))
    e[0, 6] = 1
    y = o.rope_rotate(e, np.array([[3, 0, 0, 0]]), AXES, THETA)[0]
    assert set(np.nonzero(np.abs(y) > 1e-15)[0]) == {6, 7}


def test_rope_relative_position_property():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((20, 128))
    k = rng.standard_normal((30, 128))
    pq = rng.integers(0, 100, size=(20, 4))
    pk = rng.integers(0, 100, size=(30, 4))
    s0 = o.rope_rotate(q, pq, AXES, THETA) @ o.rope_rotate(k, pk, AXES, THETA).T
    for a in range(4):
        sh = np.zeros(4, int)
        sh[a] = 37
        s1 = o.rope_rotate(q, pq + sh, AXES, THETA) @ o.rope_rotate(k, pk + sh, AXES, THETA).T
        np.testing.assert_allclose(s1, s0, rtol=0, atol=1e-10)


def test_qk_rmsnorm_rope_sets_and_weights():
    rng = np.random.default_rng(8)
    n, H, D = 6, 2, 128
    q = rng.standard_normal((n, H * D))
    k = rng.standard_normal((n, H * D))
    w = np.empty((2, 2, D))
    w[0, 0], w[0, 1], w[1, 0], w[1, 1] = 2.0, 3.0, 5.0, 7.0
    pos = np.zeros((n, 4), int)
    qo, ko = o.qk_rmsnorm_rope(q, k, H, D, w, 2, 1e-6, pos, AXES, THETA)
    rq = np.sqrt(np.mean(qo.reshape(n, H, D) ** 2, axis=-1))
    rk = np.sqrt(np.mean(ko.reshape(n, H, D) ** 2, axis=-1))
    np.testing.assert_allclose(rq[:2], 2.0, rtol=1e-6)
    np.testing.assert_allclose(rq[2:], 5.0, rtol=1e-6)
    np.testing.assert_allclose(rk[:2], 3.0, rtol=1e-6)
    np.testing.assert_allclose(rk[2:], 7.0, rtol=1e-6)
    # per-head normalisation: scaling one head leaves the result unchanged
    q2 = q.copy()
    q2[:, :D] *= 50
    qo2, _ = o.qk_rmsnorm_rope(q2, k, H, D, w, 2, 0.0, pos, AXES, THETA)
    qo0, _ = o.qk_rmsnorm_rope(q, k, H, D, w, 2, 0.0, pos, AXES, THETA)
    np.testing.assert_allclose(qo2, qo0, rtol=1e-13)


# --- attention -----------------------------------------------------------------------------

def _brute_attention(q, k, v, scale):
    n, m, dv = len(q), len(k), len(v[0])
    out = []
    for i in range(n):
        s = [scale * sum(q[i][t] * k[j][t] for t in range(len(q[i]))) for j in range(m)]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        z = sum(e)
        out.append([sum(e[j] / z * v[j][c] for j in range(m)) for c in range(dv)])
    return np.array(out)


def test_attention_brute_force_tiny():
    rng = np.random.default_rng(9)
    for n in (1, 2, 3, 4):
        q = rng.standard_normal((n, 2 * 128))
        k = rng.standard_normal((n, 2 * 128))
        v = rng.standard_normal((n, 2 * 128))
        got = o.joint_attention(q, k, v, 2, 128)
        for h in range(2):
            c = slice(h * 128, (h + 1) * 128)
            want = _brute_attention(q[:, c].tolist(), k[:, c].tolist(), v[:, c].tolist(), 1 / math.sqrt(128))
            np.testing.assert_allclose(got[:, c], want, rtol=1e-12, atol=1e-14)


def test_attention_softmax_closed_form():
    g = _load("elementwise_closed_forms.json")["softmax_ln123"]
    q = np.zeros((1, 128))
    q[0, 0] = math.sqrt(128)
    k = np.zeros((3, 128))
    k[:, 0] = g["scores"]
    v = np.zeros((3, 128))
    v[:, 5] = [6.0, 12.0, 18.0]
    out = o.joint_attention(q, k, v, 1, 128)
    want = sum(p * x for p, x in zip(g["probs"], [6.0, 12.0, 18.0]))
    assert out[0, 5] == pytest.approx(want, rel=1e-14)
    np.testing.assert_allclose(o.softmax_rows(np.array(g["scores"])), g["probs"], rtol=1e-14)


def test_attention_constant_scores_single_key_and_library():
    rng = np.random.default_rng(10)
    n, H = 37, 3
    v = rng.standard_normal((n, H * 128))
    k = rng.standard_normal((n, H * 128))
    out = o.joint_attention(np.zeros((n, H * 128)), k, v, H, 128)
    np.testing.assert_allclose(out, np.broadcast_to(v.mean(axis=0), out.shape), rtol=1e-12)
    out1 = o.joint_attention(rng.standard_normal((5, H * 128)), k[:1], v[:1], H, 128)
    np.testing.assert_allclose(out1, np.broadcast_to(v[0], out1.shape), rtol=1e-14)
    q = rng.standard_normal((n, H * 128)) * 2
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.reshape(n, H, 128).transpose(1, 0, 2).copy()),
        torch.from_numpy(k.reshape(n, H, 128).transpose(1, 0, 2).copy()),
        torch.from_numpy(v.reshape(n, H, 128).transpose(1, 0, 2).copy())).numpy()
    np.testing.assert_allclose(o.joint_attention(q, k, v, H, 128),
                               ref.transpose(1, 0, 2).reshape(n, H * 128), rtol=1e-11, atol=1e-13)
    rows = np.array([0, 5, 36])
    np.testing.assert_allclose(o.joint_attention(q, k, v, H, 128, q_rows=rows),
                               o.joint_attention(q, k, v, H, 128)[rows], rtol=0, atol=1e-13)


# --- inputs ------------------------------------------------------------------------------------

def test_positions_layout():
    p = di.positions(3, 2, 3)
    np.testing.assert_array_equal(p[:3], [[0, 0, 0, 0], [0, 0, 0, 1], [0, 0, 0, 2]])
    np.testing.assert_array_equal(p[3:], [[0, 0, 0, 0], [0, 0, 1, 0], [0, 0, 2, 0],
                                          [0, 1, 0, 0], [0, 1, 1, 0], [0, 1, 2, 0]])


# --- block-level special cases -------------------------------------------------------------------

@pytest.fixture(scope="module")
def tiny_inputs():
    cfg = tiny_cfg()
    return cfg, di.double_block_inputs(cfg, seed=3, qk_norm="random")


def _zero(inp, stream, name):
    inp = dict(inp)
    inp[stream] = dict(inp[stream])
    inp[stream][name] = np.zeros_like(inp[stream][name])
    return inp


def test_block_zero_modulation_is_identity(tiny_inputs):
    cfg, inp = tiny_inputs
    z = _zero(_zero(inp, "txt", "w_mod"), "img", "w_mod")
    out = o.double_block(cfg, z)
    np.testing.assert_array_equal(out["y_txt"], o.widen(inp["x_txt"], "f32"))
    np.testing.assert_array_equal(out["y_img"], o.widen(inp["x_img"], "f32"))
    scfg = cfg
    sinp = di.single_block_inputs(scfg, seed=4)
    sinp["w"] = dict(sinp["w"], w_mod=np.zeros_like(sinp["w"]["w_mod"]))
    np.testing.assert_array_equal(o.single_block(scfg, sinp)["y"], o.widen(sinp["x"], "f32"))


def _mods(cfg, rng, **fix):
    m = {}
    for s in ("txt", "img"):
        mm = rng.standard_normal((6, cfg.d)) * 0.5
        for idx, val in fix.items():
            mm[int(idx[1:])] = val
        m[s] = mm
    return m


def test_block_gate_chunks(tiny_inputs):
    cfg, inp = tiny_inputs
    rng = np.random.default_rng(11)
    out = o.double_block(cfg, inp, mods=_mods(cfg, rng, c2=0.0), keep=True)
    np.testing.assert_array_equal(out["h_txt"], o.widen(inp["x_txt"], "f32"))   # gate1 = 0 -> h = x
    assert np.abs(out["y_txt"] - out["h_txt"]).max() > 1e-3
    out = o.double_block(cfg, inp, mods=_mods(cfg, rng, c5=0.0), keep=True)
    np.testing.assert_array_equal(out["y_img"], out["h_img"])                  # gate2 = 0 -> y = h


def test_block_zero_up_half_gives_y_equal_h(tiny_inputs):
    cfg, inp = tiny_inputs
    z = dict(inp)
    for s in ("txt", "img"):
        w = inp[s]["w_ffn_in"].copy()
        w[cfg.ffn_inner:] = 0
        z[s] = dict(inp[s], w_ffn_in=w)
    out = o.double_block(cfg, z, keep=True)
    np.testing.assert_array_equal(out["y_txt"], out["h_txt"])
    np.testing.assert_array_equal(out["y_img"], out["h_img"])


def test_block_constant_scores_is_joint_mean(tiny_inputs):
    # W_q = 0 in both streams -> q = 0 -> every score 0 -> each output row is the
    # mean of V over ALL text and image tokens (one joint softmax).
    cfg, inp = tiny_inputs
    z = dict(inp)
    for s in ("txt", "img"):
        w = inp[s]["w_qkv"].copy()
        w[:cfg.d] = 0
        z[s] = dict(inp[s], w_qkv=w)
    out = o.double_block(cfg, z, keep=True)
    mean_v = out["v"].mean(axis=0)
    np.testing.assert_allclose(out["o_txt"], np.broadcast_to(mean_v, out["o_txt"].shape), rtol=1e-12)
    np.testing.assert_allclose(out["o_img"], np.broadcast_to(mean_v, out["o_img"].shape), rtol=1e-12)
    per_stream = out["v"][:cfg.n_txt].mean(axis=0)
    assert np.abs(per_stream - mean_v).max() > 1e-3


def test_block_scale_minus_one_closed_chain():
    # scale1 = -1 in both streams and shared (shift1, W_v): a = shift1 for every
    # token, v identical for all tokens, O = v, so h - x = gate1 * (v W_o^T),
    # the same for every row of a stream.
    cfg = tiny_cfg()
    inp = di.double_block_inputs(cfg, seed=12)
    inp["img"] = dict(inp["img"])
    wq = inp["img"]["w_qkv"].copy()
    wq[2 * cfg.d:] = inp["txt"]["w_qkv"][2 * cfg.d:]
    inp["img"]["w_qkv"] = wq
    rng = np.random.default_rng(13)
    m = _mods(cfg, rng, c1=-1.0)
    m["img"][0] = m["txt"][0]
    out = o.double_block(cfg, inp, mods=m, keep=True)
    v_row = m["txt"][0] @ o.widen(inp["txt"]["w_qkv"], "f32")[2 * cfg.d:].T
    for s in ("txt", "img"):
        want = o.widen(inp["x_" + s], "f32") + m[s][2] * (v_row @ o.widen(inp[s]["w_o"], "f32").T)
        np.testing.assert_allclose(out["h_" + s], want, rtol=1e-12, atol=1e-12)


def test_block_one_hot_routing_layout():
    # q = k = 0 (W_q = W_k = 0): O = mean of v.  One-hot rows of W_v route
    # input feature i to v column c (head c // 128); one-hot W_o routes O
    # column c to output column j.  This pins the q|k|v column blocks and the
    # head-major layout inside them.
    cfg = tiny_cfg()
    inp = di.double_block_inputs(cfg, seed=14)
    d = cfg.d
    rng = np.random.default_rng(15)
    m = _mods(cfg, rng)
    for s in ("txt", "img"):
        m[s][0] = 0.0
        m[s][1] = 0.0       # a = RMSNorm(x)
        m[s][2] = 1.0       # gate1 = 1
        m[s][5] = 0.0       # no FFN term
    i, c, j = 17, 200, 9
    for s in ("txt", "img"):
        w = np.zeros((3 * d, d), np.float32)
        w[2 * d + c, i] = 1.0
        wo = np.zeros((d, d), np.float32)
        wo[j, c] = 1.0
        inp[s] = dict(inp[s], w_qkv=w, w_o=wo)
    out = o.double_block(cfg, inp, mods=m, keep=True)
    a_all = np.concatenate([o.rms_norm(o.widen(inp["x_txt"], "f32"), cfg.eps),
                            o.rms_norm(o.widen(inp["x_img"], "f32"), cfg.eps)])
    want = a_all[:, i].mean()
    for s in ("txt", "img"):
        dh = out["h_" + s] - o.widen(inp["x_" + s], "f32")
        np.testing.assert_allclose(dh[:, j], want, rtol=1e-12)
        assert np.abs(np.delete(dh, j, axis=1)).max() == 0


def test_block_swiglu_halves_routing():
    # b = RMSNorm(h); W_in gate row r reads feature 0, up row F+r reads feature 1:
    # f_r = SiLU(b0) * b1, not SiLU(b1) * b0.
    cfg = tiny_cfg()
    inp = di.double_block_inputs(cfg, seed=16)
    d, F = cfg.d, cfg.ffn_inner
    rng = np.random.default_rng(17)
    m = _mods(cfg, rng)
    for s in ("txt", "img"):
        m[s][3] = 0.0
        m[s][4] = 0.0
    for s in ("txt", "img"):
        w = np.zeros((2 * F, d), np.float32)
        w[3, 0] = 1.0
        w[F + 3, 1] = 1.0
        inp[s] = dict(inp[s], w_ffn_in=w)
    out = o.double_block(cfg, inp, mods=m, keep=True)
    for s in ("txt", "img"):
        b = o.rms_norm(out["h_" + s], cfg.eps)
        np.testing.assert_allclose(out["f_" + s][:, 3], o.silu(b[:, 0]) * b[:, 1], rtol=1e-12)
        assert np.abs(np.delete(out["f_" + s], 3, axis=1)).max() == 0


def test_block_token_permutation_equivariance():
    cfg = tiny_cfg(grid_h=3, grid_w=3)
    inp = di.double_block_inputs(cfg, seed=18, qk_norm="random")
    out = o.double_block(cfg, inp)
    perm = np.random.default_rng(19).permutation(cfg.n_img)
    p2 = dict(inp)
    p2["x_img"] = inp["x_img"][perm]
    pos = inp["pos"].copy()
    pos[cfg.n_txt:] = inp["pos"][cfg.n_txt:][perm]
    p2["pos"] = pos
    out2 = o.double_block(cfg, p2)
    np.testing.assert_allclose(out2["y_img"], out["y_img"][perm], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(out2["y_txt"], out["y_txt"], rtol=1e-11, atol=1e-12)


def test_block_row_sampling_matches_full():
    cfg = tiny_cfg()
    inp = di.double_block_inputs(cfg, seed=20)
    full = o.double_block(cfg, inp)
    rt, ri = np.array([2, 0]), np.array([5, 1])
    part = o.double_block(cfg, inp, rows_txt=rt, rows_img=ri)
    np.testing.assert_allclose(part["y_txt"], full["y_txt"][rt], rtol=1e-6)
    np.testing.assert_allclose(part["y_img"], full["y_img"][ri], rtol=1e-6)
    sinp = di.single_block_inputs(cfg, seed=21)
    sf = o.single_block(cfg, sinp)
    sp = o.single_block(cfg, sinp, rows=np.array([7, 1]))
    np.testing.assert_allclose(sp["y"], sf["y"][[7, 1]], rtol=1e-6)


def test_single_block_layout_routing():
    # single block: W_1 rows [q|k|v|gate|up]; W_2 input columns [O|f].
    cfg = tiny_cfg()
    d, F = cfg.d, cfg.ffn_inner
    inp = di.single_block_inputs(cfg, seed=22)
    m = np.zeros((3, d))
    m[2] = 1.0                                   # gate = 1, a = RMSNorm(x)
    w1 = np.zeros((3 * d + 2 * F, d), np.float32)
    w1[2 * d + 4, 8] = 1.0                       # v column 4 <- feature 8
    w1[3 * d + 6, 2] = 1.0                       # gate row 6 <- feature 2
    w1[3 * d + F + 6, 3] = 1.0                   # up row 6 <- feature 3
    w2 = np.zeros((d, d + F), np.float32)
    w2[0, 4] = 1.0                               # y col 0 <- O col 4
    w2[1, d + 6] = 1.0                           # y col 1 <- f col 6
    inp["w"] = dict(inp["w"], w_1=w1, w_2=w2)
    out = o.single_block(cfg, inp, mods=m, keep=True)
    x = o.widen(inp["x"], "f32")
    a = o.rms_norm(x, cfg.eps)
    dy = out["y"] - x
    np.testing.assert_allclose(dy[:, 0], a[:, 8].mean(), rtol=1e-12)      # q = k = 0 -> mean of v
    np.testing.assert_allclose(dy[:, 1], o.silu(a[:, 2]) * a[:, 3], rtol=1e-12)
    assert np.abs(dy[:, 2:]).max() == 0


def test_block_scale2_minus_one_makes_ffn_input_constant():
    # scale2 = -1: b = shift2 for every token of a stream, so the FFN term
    # gate2 * (f W_down^T) is one row vector per stream: y - h is constant
    # over the rows of a stream and equals the closed chain below.
    cfg = tiny_cfg()
    inp = di.double_block_inputs(cfg, seed=24)
    rng = np.random.default_rng(25)
    m = _mods(cfg, rng, c4=-1.0)
    out = o.double_block(cfg, inp, mods=m, keep=True)
    F = cfg.ffn_inner
    for s in ("txt", "img"):
        gu = m[s][3] @ o.widen(inp[s]["w_ffn_in"], "f32").T
        f = gu[:F] / (1 + np.exp(-gu[:F])) * gu[F:]
        want = m[s][5] * (f @ o.widen(inp[s]["w_ffn_out"], "f32").T)
        dy = out["y_" + s] - out["h_" + s]
        np.testing.assert_allclose(dy, np.broadcast_to(want, dy.shape), rtol=1e-10, atol=1e-12)

"""Brute-force pins of the oracle's composed blocks (CPU).

A second, independent evaluation of the double-stream and single-stream blocks on tiny inputs
with random weights, in plain scalar Python loops over explicit indices (no numpy arithmetic, no
reshapes or transposes), following the block's definition step by step:
  AdaLN vectors m = W_mod SiLU(c), chunks shift, scale, gate (x2 for a double block);
  a = (1 + scale) x / sqrt(mean x^2 + eps) + shift;  [q|k|v] = a W_qkv^T, head h = columns 128h..;
  per-head RMSNorm of q and k times the stream's weight, then RoPE with 4 axes of 32 dims:
  the pair (2j', 2j'+1) of axis a (j' = 0..15) rotated by pos[a] * theta^(-2j'/32), computed here as
  a complex product z * exp(i phi);  joint softmax attention over [text; image] per head with
  scale 1/sqrt(128);  h = x + gate1 (O W_o^T);  b = (1 + scale2) RMSNorm(h) + shift2;
  [g|u] = b W_in^T;  y = h + gate2 ((SiLU(g) u) W_down^T);
  single block: [q|k|v|g|u] = a W_1^T, y = x + gate ([O | SiLU(g) u] W_2^T).
The oracle (numpy, vectorised) must agree to 1e-10 relative.  A transposed operand, a wrong head
or column offset, a dropped term or a flipped RoPE sign in either implementation fails this."""
import cmath
import math

import numpy as np

import dit_inputs as di
from oracle import dit_oracle as o

CFG = di.BlockConfig("brute_tiny", "f32", d=256, n_heads=2, ffn_inner=768, n_txt=2, grid_h=2, grid_w=2)


def _mat(a):
    """numpy array -> nested lists of Python floats (exact widening of float32)."""
    return np.asarray(a, np.float64).tolist()


def _matvec(w, v):
    return [sum(w[r][k] * v[k] for k in range(len(v))) for r in range(len(w))]


def _silu(z):
    return z / (1.0 + math.exp(-z))


def _rms_norm(v, eps):
    ms = sum(t * t for t in v) / len(v)
    r = 1.0 / math.sqrt(ms + eps)
    return [t * r for t in v]


def _rope(vec, pos, theta, axes=(32, 32, 32, 32)):
    out = list(vec)
    base = 0
    for a, width in enumerate(axes):
        for jp in range(width // 2):
            phi = pos[a] * theta ** (-2.0 * jp / width)
            i0 = base + 2 * jp
            z = complex(vec[i0], vec[i0 + 1]) * cmath.exp(1j * phi)
            out[i0], out[i0 + 1] = z.real, z.imag
        base += width
    return out


def _attention(q, k, v, n_heads, hd=128):
    n = len(q)
    out = [[0.0] * (n_heads * hd) for _ in range(n)]
    sc = 1.0 / math.sqrt(hd)
    for h in range(n_heads):
        c0 = h * hd
        for i in range(n):
            s = [sc * sum(q[i][c0 + e] * k[j][c0 + e] for e in range(hd)) for j in range(n)]
            mx = max(s)
            p = [math.exp(t - mx) for t in s]
            tot = sum(p)
            for e in range(hd):
                out[i][c0 + e] = sum(p[j] * v[j][c0 + e] for j in range(n)) / tot
    return out


def _qk_rope(row, d, n_heads, wq, wk, pos, cfg):
    """Row [q|k|v] of one token -> (q, k, v) with QK-norm + RoPE applied to q and k."""
    q, k, v = row[:d], row[d:2 * d], row[2 * d:3 * d]
    qo, ko = [], []
    for h in range(n_heads):
        hq = _rms_norm(q[h * 128:(h + 1) * 128], cfg.eps_qk)
        hk = _rms_norm(k[h * 128:(h + 1) * 128], cfg.eps_qk)
        qo += _rope([hq[e] * wq[e] for e in range(128)], pos, cfg.theta)
        ko += _rope([hk[e] * wk[e] for e in range(128)], pos, cfg.theta)
    return qo, ko, v


def brute_double_block(cfg, inp):
    d, F, H = cfg.d, cfg.ffn_inner, cfg.n_heads
    cond = _mat(inp["cond"])
    pos = inp["pos"].tolist()
    streams = {"txt": _mat(inp["x_txt"]), "img": _mat(inp["x_img"])}
    W = {s: {k: _mat(v) for k, v in inp[s].items()} for s in ("txt", "img")}
    sc = [_silu(c) for c in cond]
    mods, qs, ks, vs, order = {}, [], [], [], []
    for s in ("txt", "img"):
        m = _matvec(W[s]["w_mod"], sc)
        mods[s] = [m[i * d:(i + 1) * d] for i in range(6)]
        for t, x in enumerate(streams[s]):
            n = t if s == "txt" else cfg.n_txt + t
            xn = _rms_norm(x, cfg.eps)
            a = [(1.0 + mods[s][1][j]) * xn[j] + mods[s][0][j] for j in range(d)]
            q, k, v = _qk_rope(_matvec(W[s]["w_qkv"], a), d, H, W[s]["qk_norm_w"][0], W[s]["qk_norm_w"][1],
                               pos[n], cfg)
            qs.append(q); ks.append(k); vs.append(v); order.append((s, t))
    att = _attention(qs, ks, vs, H)
    out = {"txt": [], "img": []}
    for (s, t), o_row in zip(order, att):
        x = streams[s][t]
        m = mods[s]
        proj = _matvec(W[s]["w_o"], o_row)
        h = [x[j] + m[2][j] * proj[j] for j in range(d)]
        hn = _rms_norm(h, cfg.eps)
        b = [(1.0 + m[4][j]) * hn[j] + m[3][j] for j in range(d)]
        gu = _matvec(W[s]["w_ffn_in"], b)
        f = [_silu(gu[i]) * gu[F + i] for i in range(F)]
        dn = _matvec(W[s]["w_ffn_out"], f)
        out[s].append([h[j] + m[5][j] * dn[j] for j in range(d)])
    return np.array(out["txt"]), np.array(out["img"])


def brute_single_block(cfg, inp):
    d, F, H = cfg.d, cfg.ffn_inner, cfg.n_heads
    cond, pos, xs = _mat(inp["cond"]), inp["pos"].tolist(), _mat(inp["x"])
    W = {k: _mat(v) for k, v in inp["w"].items()}
    m = _matvec(W["w_mod"], [_silu(c) for c in cond])
    shift, scale, gate = m[:d], m[d:2 * d], m[2 * d:3 * d]
    qs, ks, vs, fs = [], [], [], []
    for n, x in enumerate(xs):
        xn = _rms_norm(x, cfg.eps)
        a = [(1.0 + scale[j]) * xn[j] + shift[j] for j in range(d)]
        row = _matvec(W["w_1"], a)
        q, k, v = _qk_rope(row[:3 * d], d, H, W["qk_norm_w"][0], W["qk_norm_w"][1], pos[n], cfg)
        qs.append(q); ks.append(k); vs.append(v)
        fs.append([_silu(row[3 * d + i]) * row[3 * d + F + i] for i in range(F)])
    att = _attention(qs, ks, vs, H)
    y = []
    for n, x in enumerate(xs):
        z = _matvec(W["w_2"], att[n] + fs[n])
        y.append([x[j] + gate[j] * z[j] for j in range(d)])
    return np.array(y)


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / np.sqrt(np.mean(b ** 2)))


def test_double_block_matches_brute_force_scalar_loops():
    inp = di.double_block_inputs(CFG, seed=11, qk_norm="random")
    ref = o.double_block(CFG, inp)
    bt, bi = brute_double_block(CFG, inp)
    assert _rel(ref["y_txt"], bt) < 1e-10 and _rel(ref["y_img"], bi) < 1e-10
    # the block does change its input (the comparison above is not between two copies of x)
    assert _rel(o.widen(inp["x_img"], "f32"), bi) > 1e-3


def test_single_block_matches_brute_force_scalar_loops():
    inp = di.single_block_inputs(CFG, seed=12, qk_norm="random")
    ref = o.single_block(CFG, inp)["y"]
    y = brute_single_block(CFG, inp)
    assert _rel(ref, y) < 1e-10
    assert _rel(o.widen(inp["x"], "f32"), y) > 1e-3

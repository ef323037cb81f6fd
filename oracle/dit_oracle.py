"""fp64 CPU oracle for the FLUX-style joint text+image DiT block forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s CPU-baseline leg may import this module.  The product path
(``attention_dit_block_amd``) never imports, calls or falls back to it, and it
shares no code with that path: the only common code is ``dit_inputs`` (seeded
draws, no arithmetic of the method).

What it computes is the plain definition of each stage, in float64, reading
the same storage bits the GPU gets (bf16 widened exactly, or float32) and
never rounding in between: intermediate results stay exact float64.  numpy's
matmul serves as the matrix-product primitive; everything else is written out.

Sources (the "CUDA codepath !" thread, antirez/iris.c issue #15):
  * the cuBLAS/custom-kernel reply lists the operations of the transformer:
    QKV projections, FFN, attention scores (matrix products) and RMSNorm,
    RoPE, AdaLN modulation, softmax and activations;
  * the GGML update, item 3, fixes RoPE: 4 axes of [32, 32, 32, 32] dims,
    separate text/image positions, pairs formed by repeat-interleave;
  * the GGML update's bottom line names the block: AdaLN + custom RoPE +
    joint attention.
The remaining details are the FLUX double-/single-stream block convention
(the readings are listed in the design notes and in each function below):
SiLU before the modulation linear, chunk order shift/scale/gate, modulation
(1 + scale) * RMSNorm(x) + shift, no biases, per-head RMSNorm of q and k with
a per-stream weight, RoPE frequency theta^(-2j/dim_axis) with theta = 1e4 and
rotation by +angle on interleaved pairs, softmax scale 1/sqrt(head_dim), no
mask, text tokens first, SwiGLU with the gate half first.

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``,
``tests/test_oracle_edge.py`` or ``tests/test_oracle_fp8.py`` (closed forms, invariants, library
special cases, brute force) except the
composition of the whole block, which is pinned only through its stages and
block-level special cases (identity modulation, constant scores, zero FFN).
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np

F64 = np.float64


# --- storage -----------------------------------------------------------------

def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage (bf16 bit pattern as uint16, float16 or float32) -> exact float64."""
    if dtype == "bf16":
        u = np.ascontiguousarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(F64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(F64)
    if dtype == "f16":
        return np.asarray(a, dtype=np.float16).astype(F64)
    if dtype == "f64":
        return np.asarray(a, dtype=F64)
    raise ValueError(dtype)


# --- elementwise ---------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z)) (the thread's 'activations')."""
    z = np.asarray(z, dtype=F64)
    return z / (1.0 + np.exp(-z))


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """SwiGLU gating f = SiLU(g) * u, g being the first half of the FFN-in output."""
    return silu(g) * u


# --- AdaLN ------------------------------------------------------------------------

def adaln_modulation(w_mod: np.ndarray, cond: np.ndarray) -> np.ndarray:
    """m = W_mod . SiLU(c).  W_mod is [n_chunks*d, d_cond] ([out, in]); the result
    is read as n_chunks vectors of d in the order shift, scale, gate (repeated)."""
    return np.asarray(w_mod, F64) @ silu(cond)


def rms_norm(x: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) over the last axis; no learnable weight."""
    x = np.asarray(x, F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps)


def modulate(x: np.ndarray, shift: np.ndarray, scale: np.ndarray, eps: float) -> np.ndarray:
    """AdaLN modulation of a pre-norm: (1 + scale) * RMSNorm(x) + shift.
    shift = scale = 0 gives the plain RMSNorm (identity modulation)."""
    return (1.0 + np.asarray(scale, F64)) * rms_norm(x, eps) + np.asarray(shift, F64)


def adaln_modulate(cond, w_mod, n_chunks: int, d: int, x=None, shift_chunk: int = 0,
                   scale_chunk: int = 1, eps: float = 1e-6):
    """Counterpart of the library's standalone AdaLN call: returns the modulation
    vectors m [n_chunks, d] and, if x is given, (1+scale)*RMSNorm(x)+shift."""
    m = adaln_modulation(w_mod, cond).reshape(n_chunks, d)
    if x is None:
        return m, None
    return m, modulate(x, m[shift_chunk], m[scale_chunk], eps)


# --- RoPE ---------------------------------------------------------------------------

def rope_frequencies(axis_dim: int, theta: float) -> np.ndarray:
    """omega_j = theta^(-2j/axis_dim), j = 0 .. axis_dim/2 - 1."""
    j = np.arange(axis_dim // 2, dtype=F64)
    return np.power(F64(theta), -2.0 * j / axis_dim)


def rope_angles(pos: np.ndarray, axes_dim: Sequence[int], theta: float) -> np.ndarray:
    """phi[n, p] for every pair p of the head (pairs of all axes, in axis order):
    phi = pos[n, a] * omega_j for the pair j of axis a."""
    pos = np.asarray(pos, dtype=F64)
    cols = []
    for a, dim in enumerate(axes_dim):
        cols.append(pos[:, a:a + 1] * rope_frequencies(dim, theta)[None, :])
    return np.concatenate(cols, axis=1)


def rope_rotate(x: np.ndarray, pos: np.ndarray, axes_dim: Sequence[int], theta: float) -> np.ndarray:
    """Rotate every interleaved pair (x[2p], x[2p+1]) of the last axis by +phi[n, p]:
    (u, v) -> (u cos - v sin, u sin + v cos).  x is [n, ..., head_dim] with the
    token on axis 0; axis a of the position owns dims [sum(axes_dim[:a]), +axes_dim[a])."""
    x = np.asarray(x, F64)
    phi = rope_angles(pos, axes_dim, theta)               # [n, head_dim/2]
    shape = (x.shape[0],) + (1,) * (x.ndim - 2) + (phi.shape[1],)
    c = np.cos(phi).reshape(shape)
    s = np.sin(phi).reshape(shape)
    u = x[..., 0::2]
    v = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = u * c - v * s
    out[..., 1::2] = u * s + v * c
    return out


def qk_rmsnorm_rope(q, k, n_heads: int, head_dim: int, qk_w, n_first: int, eps: float,
                    pos, axes_dim: Sequence[int], theta: float):
    """Per token and head: q <- RoPE(RMSNorm(q_head) * w_q), k likewise with w_k.
    q, k are [n, n_heads*head_dim]; qk_w is [2 sets, 2 (q, k), head_dim]: rows
    n < n_first use set 0 (text), the others set 1 (image)."""
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    n = q.shape[0]
    w = np.asarray(qk_w, F64).reshape(-1, 2, head_dim)
    set_of_row = np.where(np.arange(n) < n_first, 0, min(1, w.shape[0] - 1))
    outs = []
    for which, t in ((0, q), (1, k)):
        th = t.reshape(n, n_heads, head_dim)
        wrow = w[set_of_row, which, :][:, None, :]         # [n, 1, head_dim]
        normed = rms_norm(th, eps) * wrow
        outs.append(rope_rotate(normed, pos, axes_dim, theta).reshape(n, n_heads * head_dim))
    return outs[0], outs[1]


# --- attention ----------------------------------------------------------------------

def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Exact softmax over the last axis (max-subtracted)."""
    s = np.asarray(s, F64)
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def joint_attention(q, k, v, n_heads: int, head_dim: int, scale: Optional[float] = None,
                    q_rows: Optional[np.ndarray] = None) -> np.ndarray:
    """For every head h: O_h = softmax(Q_h K_h^T * scale) V_h over ALL tokens
    (text and image in one softmax, no mask).  q, k, v are [n, n_heads*head_dim]
    with head h in columns h*head_dim .. h*head_dim + head_dim - 1.
    ``q_rows`` restricts the query rows (the keys and values are always all)."""
    if scale is None:
        scale = 1.0 / np.sqrt(F64(head_dim))
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    if q_rows is not None:
        q = q[q_rows]
    out = np.empty((q.shape[0], n_heads * head_dim), dtype=F64)
    for h in range(n_heads):
        c = slice(h * head_dim, (h + 1) * head_dim)
        p = softmax_rows((q[:, c] @ k[:, c].T) * scale)
        out[:, c] = p @ v[:, c]
    return out


# --- blocks ---------------------------------------------------------------------------

def _w(ws: Dict[str, np.ndarray], name: str, dtype: str) -> np.ndarray:
    return widen(ws[name], dtype)


def _product(x: np.ndarray, w: np.ndarray, fp8: bool) -> np.ndarray:
    """x w^T.  fp8: both operands first quantised per row to OCP e4m3 (``quantize_fp8_rows``: each
    row scaled by its max |value| / 448 and rounded to the nearest e4m3 value), the product then
    exact (``linear_fp8``) -- the fp8 variant of a weight product."""
    if not fp8:
        return x @ w.T
    xq, sx = quantize_fp8_rows(x)
    wq, sw = quantize_fp8_rows(w)
    return linear_fp8(xq, sx, wq, sw)


def double_block(cfg, inputs: Dict[str, object], rows_txt=None, rows_img=None,
                 mods=None, keep: bool = False, fp8: bool = False) -> Dict[str, np.ndarray]:
    """Double-stream block (text and image keep their own weights, attention is joint).

    1. m_s = W_mod,s . SiLU(c) -> shift1, scale1, gate1, shift2, scale2, gate2
    2. a_s = (1 + scale1) * RMSNorm(x_s) + shift1
    3. [q | k | v]_s = a_s W_qkv,s^T
    4. q, k <- RMSNorm per head * w_{q,k},s ; RoPE at the token's position
    5. O = joint attention over [text; image]
    6. h_s = x_s + gate1 * (O_s W_o,s^T)
    7. b_s = (1 + scale2) * RMSNorm(h_s) + shift2 ; [g | u] = b_s W_in,s^T
    8. y_s = h_s + gate2 * ((SiLU(g) * u) W_down,s^T)

    Every step is exact float64 arithmetic on the stored inputs.  The inputs x_s
    are read in their own storage type (``x_dtype``: the workload type for a
    first block, float32 for a block fed by another block's output).
    ``rows_txt`` / ``rows_img`` select output rows (index arrays within each
    stream); all tokens still enter the keys and values.  ``mods`` replaces
    the AdaLN vectors by given [6, d] arrays (special-case pins).  ``keep``
    returns the intermediates too.  ``fp8`` quantises both operands of the four weight
    products (QKV, out-projection, FFN-in, FFN-down) to e4m3 per row (``_product``) and runs the
    attention on e4m3 q, k, v (``fp8_attention_operands``, ``joint_attention_fp8``); the
    values are rounded to float32 just before each quantisation (the quantisers' input
    precision), everything else stays exact."""
    t = cfg.dtype
    d, H, D, F = cfg.d, cfg.n_heads, cfg.head_dim, cfg.ffn_inner
    nt, ni = cfg.n_txt, cfg.n_img
    xdt = inputs.get("x_dtype", t)
    cond = widen(inputs["cond"], t)
    xs = {"txt": widen(inputs["x_txt"], xdt), "img": widen(inputs["x_img"], xdt)}
    pos = np.asarray(inputs["pos"])
    ws = {"txt": inputs["txt"], "img": inputs["img"]}
    m = {}
    for s in ("txt", "img"):
        if mods is not None:
            m[s] = np.asarray(mods[s], F64).reshape(6, d)
        else:
            m[s] = adaln_modulation(_w(ws[s], "w_mod", t), cond).reshape(6, d)
    qkv = {}
    for s in ("txt", "img"):
        a = modulate(xs[s], m[s][0], m[s][1], cfg.eps)
        qkv[s] = _product(a, _w(ws[s], "w_qkv", t), fp8)
    q = np.concatenate([qkv["txt"][:, :d], qkv["img"][:, :d]], axis=0)
    k = np.concatenate([qkv["txt"][:, d:2 * d], qkv["img"][:, d:2 * d]], axis=0)
    v = np.concatenate([qkv["txt"][:, 2 * d:], qkv["img"][:, 2 * d:]], axis=0)
    qk_w = np.stack([widen(ws["txt"]["qk_norm_w"], t).reshape(2, D),
                     widen(ws["img"]["qk_norm_w"], t).reshape(2, D)])
    q, k = qk_rmsnorm_rope(q, k, H, D, qk_w, nt, cfg.eps_qk, pos, cfg.axes_dim, cfg.theta)
    rows = {"txt": np.arange(nt) if rows_txt is None else np.asarray(rows_txt),
            "img": np.arange(ni) if rows_img is None else np.asarray(rows_img)}
    q_rows = np.concatenate([rows["txt"], nt + rows["img"]])
    if fp8:
        kmax = float(np.max(np.abs(qk_w[:, 1, :])))
        o = joint_attention_fp8(*fp8_attention_operands(q, k, v, H, D, kmax), H, D, q_rows=q_rows)
    else:
        o = joint_attention(q, k, v, H, D, q_rows=q_rows)
    o_s = {"txt": o[:len(rows["txt"])], "img": o[len(rows["txt"]):]}
    out: Dict[str, np.ndarray] = {}
    for s in ("txt", "img"):
        x_r = xs[s][rows[s]]
        h = x_r + m[s][2] * _product(o_s[s], _w(ws[s], "w_o", t), fp8)
        b = modulate(h, m[s][3], m[s][4], cfg.eps)
        gu = _product(b, _w(ws[s], "w_ffn_in", t), fp8)
        f = swiglu(gu[:, :F], gu[:, F:])
        y = h + m[s][5] * _product(f, _w(ws[s], "w_ffn_out", t), fp8)
        out["y_" + s] = y
        if keep:
            out.update({"mod_" + s: m[s], "h_" + s: h, "f_" + s: f, "o_" + s: o_s[s]})
    if keep:
        out.update({"q": q, "k": k, "v": v, "qkv_txt": qkv["txt"], "qkv_img": qkv["img"]})
    return out


def single_block(cfg, inputs: Dict[str, object], rows=None, mods=None,
                 keep: bool = False, fp8: bool = False) -> Dict[str, np.ndarray]:
    """Single-stream block over the concatenated sequence x = [text; image]:

    m = W_mod . SiLU(c) -> shift, scale, gate
    a = (1 + scale) * RMSNorm(x) + shift
    [q | k | v | g | u] = a W_1^T
    q, k <- RMSNorm per head * w ; RoPE ; O = joint attention
    y = x + gate * ([O | SiLU(g) * u] W_2^T)

    Exact float64 arithmetic as in ``double_block``; x is read in ``x_dtype``.  ``fp8``
    quantises both operands of the two weight products (W_1 per output row, each activation row
    over its full width) to e4m3 and runs the attention on e4m3 q, k, v, as
    ``double_block(fp8=True)`` does."""
    t = cfg.dtype
    d, H, D, F = cfg.d, cfg.n_heads, cfg.head_dim, cfg.ffn_inner
    n = cfg.n_tok
    cond = widen(inputs["cond"], t)
    x = widen(inputs["x"], inputs.get("x_dtype", t))
    pos = np.asarray(inputs["pos"])
    ws = inputs["w"]
    if mods is not None:
        m = np.asarray(mods, F64).reshape(3, d)
    else:
        m = adaln_modulation(_w(ws, "w_mod", t), cond).reshape(3, d)
    a = modulate(x, m[0], m[1], cfg.eps)
    w1 = _w(ws, "w_1", t)
    qkv = _product(a, w1[:3 * d], fp8)
    q, k, v = qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:]
    qk_w = widen(ws["qk_norm_w"], t).reshape(1, 2, D)
    q, k = qk_rmsnorm_rope(q, k, H, D, qk_w, n, cfg.eps_qk, pos, cfg.axes_dim, cfg.theta)
    r = np.arange(n) if rows is None else np.asarray(rows)
    if fp8:
        kmax = float(np.max(np.abs(qk_w[:, 1, :])))
        o = joint_attention_fp8(*fp8_attention_operands(q, k, v, H, D, kmax), H, D, q_rows=r)
    else:
        o = joint_attention(q, k, v, H, D, q_rows=r)
    gu = _product(a[r], w1[3 * d:], fp8)
    f = swiglu(gu[:, :F], gu[:, F:])
    y = x[r] + m[2] * _product(np.concatenate([o, f], axis=1), _w(ws, "w_2", t), fp8)
    out = {"y": y}
    if keep:
        out.update({"mod": m, "q": q, "k": k, "v": v, "o": o, "f": f, "a": a})
    return out


# --- the steps either side of the block stack ------------------------------------------
# The pages name the denoising step's transformer (FLUX Klein) but print none of these layers;
# they follow the FLUX model's conventions, without biases like the block (readings listed in the
# design notes).

def timestep_embedding(t: float, dim: int, max_period: float = 10000.0,
                       time_factor: float = 1000.0) -> np.ndarray:
    """Sinusoidal embedding of a scalar: s = time_factor * t, half = dim / 2,
    f_j = max_period^(-j / half) for j = 0 .. half-1, emb = [cos(s f_j) ..., sin(s f_j) ...]
    (the cosine half first)."""
    half = dim // 2
    j = np.arange(half, dtype=F64)
    f = np.exp(-math.log(max_period) * j / half)
    a = F64(time_factor) * F64(t) * f
    return np.concatenate([np.cos(a), np.sin(a)])


def mlp_embedder(v: np.ndarray, w_in: np.ndarray, w_out: np.ndarray) -> np.ndarray:
    """Two linear layers with a SiLU between: W_out . SiLU(W_in . v)."""
    return np.asarray(w_out, F64) @ silu(np.asarray(w_in, F64) @ np.asarray(v, F64))


def conditioning_vector(t: float, w_t_in, w_t_out, freq_dim: int, g: Optional[float] = None,
                        w_g_in=None, w_g_out=None, max_period: float = 10000.0,
                        time_factor: float = 1000.0) -> np.ndarray:
    """c = MLP_t(emb(t)) (+ MLP_g(emb(g)) when a guidance value and its weights are given)."""
    c = mlp_embedder(timestep_embedding(t, freq_dim, max_period, time_factor), w_t_in, w_t_out)
    if g is not None:
        c = c + mlp_embedder(timestep_embedding(g, freq_dim, max_period, time_factor), w_g_in, w_g_out)
    return c


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = x W^T with W [out, in] (patch and text embedding, final projection)."""
    return np.asarray(x, F64) @ np.asarray(w, F64).T


def layer_norm(x: np.ndarray, eps: float) -> np.ndarray:
    """(x - mean) / sqrt(var + eps) over the last axis (population variance), no affine."""
    x = np.asarray(x, F64)
    mu = np.mean(x, axis=-1, keepdims=True)
    var = np.mean((x - mu) ** 2, axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def final_layer(x: np.ndarray, cond: np.ndarray, w_mod: np.ndarray, w_out: np.ndarray,
                eps: float = 1e-6) -> np.ndarray:
    """Last layer of the model: [shift, scale] = W_mod . SiLU(c);
    y = ((1 + scale) * LayerNorm(x) + shift) W_out^T."""
    d = np.asarray(x).shape[-1]
    m = adaln_modulation(w_mod, cond).reshape(2, d)
    return linear((1.0 + m[1]) * layer_norm(x, eps) + m[0], w_out)


# --- windowed (neighborhood) attention ---------------------------------------------------
# The diffusion-VAE decoder page ports a neighborhood-attention kernel: every query attends to the
# keys of a 3-D window (odd size per axis) around its grid position, with the boundary rule of
# NATTEN -- near an edge the window shifts inwards instead of shrinking, and an axis narrower
# than the requested window is attended in full (the effective size per axis is min(k, extent)).

def window_start(i: int, k: int, n: int) -> int:
    """First position of the window of size min(k, n) along an axis of extent n for query
    position i: centred on i where it fits, shifted to stay inside [0, n)."""
    ke = min(k, n)
    return min(max(i - k // 2, 0), n - ke)


def neighborhood_attention(q, k, v, grid: Sequence[int], kernel: Sequence[int], n_heads: int, head_dim: int,
                           scale: Optional[float] = None, q_rows=None) -> np.ndarray:
    """O = softmax(q K_W^T * scale) V_W per head, K_W / V_W the tokens of the query's window.
    Tokens are the grid positions (t, h, w) in row-major order (w fastest); q, k, v are
    [T*H*W, n_heads*head_dim].  Returns the rows q_rows (all by default)."""
    q, k, v = (np.asarray(a, F64) for a in (q, k, v))
    T, H, W = grid
    scale = head_dim ** -0.5 if scale is None else scale
    rows = np.arange(T * H * W) if q_rows is None else np.asarray(q_rows)
    eff = [min(kk, n) for kk, n in zip(kernel, grid)]
    out = np.empty((len(rows), n_heads * head_dim), F64)
    for r_i, r in enumerate(rows):
        t, h, w = r // (H * W), (r // W) % H, r % W
        st = [window_start(i, kk, n) for i, kk, n in zip((t, h, w), kernel, grid)]
        tt, hh, ww = np.meshgrid(np.arange(st[0], st[0] + eff[0]), np.arange(st[1], st[1] + eff[1]),
                                 np.arange(st[2], st[2] + eff[2]), indexing="ij")
        keys = ((tt * H + hh) * W + ww).ravel()
        for hd in range(n_heads):
            sl = slice(hd * head_dim, (hd + 1) * head_dim)
            p = softmax_rows((q[r, sl] @ k[keys, sl].T * scale)[None, :])[0]
            out[r_i, sl] = p @ v[keys, sl]
    return out


# --- fp8 (OCP e4m3) GEMM variant -----------------------------------------------------------
# The pages weigh speed against accuracy ("slight (invisible) loss of accuracy", the cuBLAS
# reply's follow-up); this variant runs the block's products on 8-bit floats: OCP e4m3 (1 sign,
# 4 exponent bits with bias 7, 3 mantissa bits; largest finite 448, no infinities), one fp32 scale
# per row of each operand.  The quantised code is an integer decided by floating point, so the
# oracle takes that decision in the kernel's precision (float32), as the GPU does.

E4M3_MAX = 448.0


def _e4m3_value(code) -> np.ndarray:
    """Value of e4m3 byte(s): (-1)^s 2^(e-7) (1 + m/8) for e > 0, (-1)^s 2^-6 (m/8) for e = 0;
    0x7f / 0xff are NaN."""
    c = np.asarray(code, dtype=np.int64)
    sgn = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    v = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.power(2.0, e - 7))
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return sgn * v


_E4M3_TABLE = _e4m3_value(np.arange(256))       # value of every byte
_E4M3_POS = _E4M3_TABLE[:0x7f]                  # the 127 finite non-negative values, ascending
_E4M3_MID = (_E4M3_POS[:-1] + _E4M3_POS[1:]) / 2  # the 126 midpoints between neighbours (exact in float64)


def e4m3_decode(code) -> np.ndarray:
    """Value of e4m3 byte(s), by the closed form above (tabulated once for the 256 bytes)."""
    return _E4M3_TABLE[np.asarray(code, dtype=np.int64)]


def e4m3_encode(x) -> np.ndarray:
    """Round float values to the nearest e4m3 value, ties to the even code (even mantissa), keeping
    the sign (e4m3 has +0 and -0).  Magnitudes from 448 up to (not including) 464, halfway to the next binade step, round to 448;
    larger ones have no finite code and are refused (the callers scale into range).
    The non-negative codes 0..126 are the finite values in ascending order, so the code of |x| is
    the number of midpoints below it, moved up by one at an exact midpoint whose lower neighbour is
    odd."""
    x = np.asarray(x, dtype=F64)
    a = np.abs(x)
    if np.any(a >= 464.0):
        raise ValueError("value beyond the e4m3 range")
    code = np.searchsorted(_E4M3_MID, a, side="left")       # midpoints strictly below a
    at_mid = _E4M3_MID[np.minimum(code, len(_E4M3_MID) - 1)] == a
    code = code + (at_mid & (code % 2 == 1))
    # the sign survives rounding, so a negative value that rounds to zero is -0 (code 0x80)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def quantize_fp8_rows(x: np.ndarray):
    """Per-row e4m3 quantisation: s = max|x_row| / 448 in float32 (1 for an all-zero row), codes of
    float32(x / s).  Returns (codes [rows, cols] uint8, scales [rows] float32)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1)
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = (x / s[:, None]).astype(np.float32)
    return e4m3_encode(y), s


def linear_fp8(xq, sx, wq, sw) -> np.ndarray:
    """y = diag(sx) (dec(xq) dec(wq)^T) diag(sw), exact in float64."""
    return (np.asarray(sx, F64)[:, None] * (e4m3_decode(xq) @ e4m3_decode(wq).T)) * np.asarray(sw, F64)[None, :]


def joint_attention_fp8(q8, sq, k8, sk, v8, sv, n_heads: int, head_dim: int, scale: Optional[float] = None,
                        q_rows: Optional[np.ndarray] = None, round_p: bool = False,
                        p_shift: Optional[np.ndarray] = None) -> np.ndarray:
    """Joint attention with e4m3 operands (the fp8 variant of the attention's two products).
    q8, k8, v8 are [n, n_heads*head_dim] e4m3 codes, head h in columns h*head_dim ..; the scales are
    float32: sq [n, n_heads] one per token and head, sk [n_heads] and sv [n_heads] one per head.  The
    operands are Q_h = diag(sq[:, h]) dec(q8_h), K_h = sk[h] dec(k8_h), V_h = sv[h] dec(v8_h),
    exactly, and O_h = softmax(Q_h K_h^T * scale) V_h in float64.

    round_p adds a model of the probabilities passing through e4m3 on their way into the PV product:
    with s the scaled scores of a row and w_j = exp(s_j - max s) (the largest weight is 1), the
    weights become dec(e4m3(w_j)) while the normaliser stays the exact sum:
    O = sum_j dec(e4m3(w_j)) V_j / sum_j w_j.  Weights below 2^-6 land on e4m3's subnormal grid
    (steps of 2^-9).  p_shift [rows, n_heads] (log2 units, 0 <= shift <= 8) rounds the weights of
    a row relative to a max lower than the row's by that much instead: dec(e4m3(w_j 2^shift)) 2^-shift
    -- an online softmax whose running max lags the row max by shift."""
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    q = e4m3_decode(q8)
    k = e4m3_decode(k8)
    v = e4m3_decode(v8)
    sq = np.asarray(sq, F64).reshape(q.shape[0], n_heads)
    sk = np.asarray(sk, F64).reshape(n_heads)
    sv = np.asarray(sv, F64).reshape(n_heads)
    if q_rows is not None:
        q, sq = q[q_rows], sq[q_rows]
    out = np.empty((q.shape[0], n_heads * head_dim), dtype=F64)
    for h in range(n_heads):
        c = slice(h * head_dim, (h + 1) * head_dim)
        s = (sq[:, h:h + 1] * q[:, c]) @ (sk[h] * k[:, c]).T * scale
        w = np.exp(s - np.max(s, axis=1, keepdims=True))
        if round_p:
            f = np.ones((w.shape[0], 1)) if p_shift is None else np.exp2(np.asarray(p_shift, F64)[:, h:h + 1])
            wq = e4m3_decode(e4m3_encode(w * f)) / f
        else:
            wq = w
        out[:, c] = (wq @ (sv[h] * v[:, c])) / np.sum(w, axis=1, keepdims=True)
    return out


# Bound of a QK-normed, rotated head vector's elements relative to its weight: after RMSNorm the
# 128 values have sum of squares 128 * ms / (ms + eps) < 128, so each has |x| < sqrt(128); the
# weight multiplies it by at most max|w|, and a rotation of a pair (x, y) keeps sqrt(x^2 + y^2).
K_BOUND_PER_WEIGHT = np.float32(math.sqrt(128.0) / E4M3_MAX)


def fp8_attention_operands(q, k, v, n_heads: int, head_dim: int, k_weight_absmax: float):
    """The e4m3 operands of the fp8 blocks' attention (float32 decisions, as the kernels take them):
    q per (token, head) row by ``quantize_fp8_rows``; k per head with the static scale
    s_k = float32(max|w_k| * float32(sqrt(128) / 448)), max over the k-norm weights the block uses
    (every |k| stays below 448 s_k, see K_BOUND_PER_WEIGHT), codes e4m3(float32(k) / s_k); v per
    head with s_v = max over the head's |v| / 448 (1 for an all-zero head), codes
    e4m3(float32(v) / s_v).  Returns (q8, sq [n, H], k8, sk [H], v8, sv [H])."""
    n, D, H = q.shape[0], head_dim, n_heads
    q32, k32, v32 = (np.asarray(t, F64).astype(np.float32) for t in (q, k, v))
    q8 = np.empty((n, H * D), np.uint8)
    sq = np.empty((n, H), np.float32)
    for h in range(H):
        q8[:, h * D:(h + 1) * D], sq[:, h] = quantize_fp8_rows(q32[:, h * D:(h + 1) * D])
    s_k = np.float32(np.float32(k_weight_absmax) * K_BOUND_PER_WEIGHT)
    sk = np.full(H, s_k, np.float32)
    k8 = e4m3_encode((k32 / s_k).astype(np.float32))
    vmax = np.max(np.abs(v32).reshape(n, H, D), axis=(0, 2))
    sv = np.where(vmax > 0, vmax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    v8 = e4m3_encode((v32 / np.repeat(sv, D)[None, :]).astype(np.float32))
    return q8, sq, k8, sk, v8, sv


# --- 2-D convolution (the diffusion-VAE decoder's layers) ----------------------------------------

def conv2d_nhwc(x: np.ndarray, w: np.ndarray, bias=None) -> np.ndarray:
    """y[b, h, w, co] = bias[co] + sum_{i, j, ci} x[b, h + i - KH//2, w + j - KW//2, ci] W[co, i, j, ci],
    x [B, H, W, Cin] (NHWC), W [Cout, KH, KW, Cin], stride 1, zeros outside the image (odd KH, KW
    keep the output the input's size)."""
    x = np.asarray(x, F64)
    w = np.asarray(w, F64)
    B, H, W_, Cin = x.shape
    Cout, KH, KW, _ = w.shape
    ph, pw = KH // 2, KW // 2
    xp = np.zeros((B, H + 2 * ph, W_ + 2 * pw, Cin), F64)
    xp[:, ph:ph + H, pw:pw + W_, :] = x
    y = np.zeros((B, H, W_, Cout), F64)
    for i in range(KH):
        for j in range(KW):
            y += xp[:, i:i + H, j:j + W_, :] @ w[:, i, j, :].T
    if bias is not None:
        y += np.asarray(bias, F64)
    return y


def conv3d_causal_nhwc(x: np.ndarray, w: np.ndarray, bias=None) -> np.ndarray:
    """Causal 3-D convolution over video frames (the video-VAE decoder's layers):
    y[b, t, h, w, co] = bias[co] + sum_{s, i, j, ci} x[b, t + s - (KT-1), h + i - KH//2, w + j - KW//2, ci]
                                                    W[co, s, i, j, ci],
    x [B, T, H, W, Cin], W [Cout, KT, KH, KW, Cin]; frames before the first and pixels outside the
    image are zeros, so output frame t sees frames t-KT+1 .. t only and keeps the input's size."""
    x = np.asarray(x, F64)
    w = np.asarray(w, F64)
    B, T, H, W_, Cin = x.shape
    Cout, KT, KH, KW, _ = w.shape
    pt, ph, pw = KT - 1, KH // 2, KW // 2
    xp = np.zeros((B, T + pt, H + 2 * ph, W_ + 2 * pw, Cin), F64)
    xp[:, pt:, ph:ph + H, pw:pw + W_, :] = x
    y = np.zeros((B, T, H, W_, Cout), F64)
    for s_ in range(KT):
        for i in range(KH):
            for j in range(KW):
                y += xp[:, s_:s_ + T, i:i + H, j:j + W_, :] @ w[:, s_, i, j, :].T
    if bias is not None:
        y += np.asarray(bias, F64)
    return y

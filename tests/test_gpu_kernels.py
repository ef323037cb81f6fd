"""Per-entry-point parity of the HIP path against the fp64 oracle (GPU).

Each test draws seeded inputs, runs one C-ABI entry point through the binding, and
compares element by element with the oracle stage it implements (exact float64 on the
same input bits).  Bars, derived from the arithmetic of each call:
  * fp32 outputs: max|gpu - oracle| / RMS(oracle) <= 1e-4;
  * 16-bit outputs (bf16, fp16): the output is the exact value rounded once to the output
    type, up to fp32 arithmetic (which can flip a rounding that falls within ~1e-6 of a
    tie), so every element must lie within tol_ulp ulps of the exact value.  A max/RMS bar
    cannot resolve this: one bf16 ulp at the largest magnitudes of these tensors is
    already ~2% of their RMS;
  * attention (16-bit): the probabilities enter the PV product rounded (fp16: 2^-11
    relative; bf16: two terms, 2^-16), which adds at most that fraction of
    attention(q, k, |v|) -- a quantity the oracle computes exactly.
Every test also checks that the library really launched (dit_launch_count).
"""
import numpy as np
import pytest
import torch

import dit_inputs as di
from oracle import dit_oracle as o
from gpu_util import dev, host, metric, ulp, say, tdtype

pytestmark = pytest.mark.gpu

AXES = (32, 32, 32, 32)


@pytest.fixture(scope="module")
def dit():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import attention_dit_block_amd as m
    return m


def _cfg(dtype, n_txt, gh, gw, heads):
    return di.BlockConfig("t", dtype, d=128 * heads, n_heads=heads, ffn_inner=3 * 128 * heads,
                          n_txt=n_txt, grid_h=gh, grid_w=gw)


def check(gpu, ref, dtype, tol_ulp=0.6, what=""):
    m = metric(gpu, ref)
    if dtype == "f32":
        assert m <= 1e-4, f"{what}: max/RMS {m:.3e} > 1e-4"
        return m
    err = np.abs(gpu - ref)
    bound = tol_ulp * ulp(ref, dtype) + 1e-6 * np.sqrt(np.mean(ref ** 2))
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} elements beyond {tol_ulp} ulp, worst "
                           f"{np.max(err / bound):.2f}x at {np.unravel_index(np.argmax(err / bound), err.shape)}")
    return m


def check_attention(gpu, ref, ref_abs, dtype, what="O"):
    rel = 2.0 ** -11 if dtype == "f16" else 2.0 ** -16
    perr = (rel + 1e-5) * ref_abs
    bound = 0.5 * ulp(np.abs(ref) + perr, dtype) * 1.001 + perr
    err = np.abs(gpu - ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} elements beyond the bound, worst "
                           f"{np.max(err / bound):.2f}x at {np.unravel_index(np.argmax(err / bound), err.shape)}")
    say(f"  {what}: max err/bound {np.max(err / bound):.3f}, max|gpu-oracle|/RMS {metric(gpu, ref):.2e}")


ROPE_CASES = [
    # (q/k dtype, weight dtype, n_txt, grid h, grid w, heads)
    ("f32", "f32", 16, 8, 8, 2),        # the fp32 workload's shape
    ("f16", "bf16", 512, 64, 64, 24),   # the bf16 block: fp16 activations, bf16 QK-norm weights
    ("bf16", "bf16", 512, 64, 64, 24),
    ("f16", "bf16", 5, 3, 7, 3),        # ragged
    ("bf16", "bf16", 1, 1, 1, 1),       # one text and one image token
    ("f16", "f16", 0, 2, 3, 2),         # image only
]


@pytest.mark.parametrize("dtype,wdt,n_txt,gh,gw,heads", ROPE_CASES)
def test_qk_rmsnorm_rope(dit, dtype, wdt, n_txt, gh, gw, heads):
    say(f"qk_rmsnorm_rope {dtype} w={wdt} n_txt={n_txt} grid={gh}x{gw} heads={heads}")
    cfg = _cfg("f32" if wdt == "f16" else wdt, n_txt, gh, gw, heads)
    n, d = cfg.n_tok, cfg.d
    qkv = di.draw((n, 3 * d), 1.5, dtype, 7, "q")
    w = np.stack([di._qk_norm_weights(cfg, 7, 0, "txt", "random"),
                  di._qk_norm_weights(cfg, 7, 0, "img", "random")])   # [2 sets][2][128]
    if wdt == "f16":
        w = w.astype(np.float16)
    pos = di.positions(n_txt, gh, gw)
    t = dev(qkv, dtype)
    before = dit.launch_count()
    dit.qk_rmsnorm_rope(t[:, :d], t[:, d:2 * d], heads, dev(w, wdt), n_txt, dev(pos, "i32"), eps=1e-6)
    torch.cuda.synchronize()
    assert dit.launch_count() == before + 1
    out = host(t)
    x = o.widen(qkv, dtype)
    rq, rk = o.qk_rmsnorm_rope(x[:, :d], x[:, d:2 * d], heads, 128, o.widen(w, wdt), n_txt, 1e-6, pos, AXES, 1e4)
    check(out[:, :d], rq, dtype, what="q")
    check(out[:, d:2 * d], rk, dtype, what="k")
    np.testing.assert_array_equal(out[:, 2 * d:], x[:, 2 * d:])       # v untouched


def test_qk_rmsnorm_rope_large_positions(dit):
    # positions far beyond the workloads (angles up to ~2e4 rad): the angle is reduced in double
    say("qk_rmsnorm_rope large positions")
    n, heads = 64, 2
    d = 128 * heads
    q = di.draw((n, d), 1.0, "f32", 8, "q")
    k = di.draw((n, d), 1.0, "f32", 8, "k")
    pos = np.random.default_rng(8).integers(0, 20000, size=(n, 4)).astype(np.int32)
    w = np.ones((2, 2, 128), np.float32)
    tq, tk = dev(q, "f32"), dev(k, "f32")
    dit.qk_rmsnorm_rope(tq, tk, heads, dev(w, "f32"), n, dev(pos, "i32"), eps=1e-6)
    rq, rk = o.qk_rmsnorm_rope(q, k, heads, 128, w, n, 1e-6, pos, AXES, 1e4)
    check(host(tq), rq, "f32", what="q")
    check(host(tk), rk, "f32", what="k")


ADALN_CASES = [
    # (weight dtype, x dtype, out dtype, d, chunks, rows)
    ("f32", "f32", "f32", 256, 6, 80),
    ("bf16", "bf16", "f16", 3072, 6, 4608),   # the bf16 block's first pre-norm
    ("bf16", "f32", "f16", 3072, 6, 600),     # fp32 input (the residual stream h)
    ("bf16", "bf16", "bf16", 3072, 6, 512),
    ("bf16", "bf16", "f16", 3072, 3, 37),     # single-stream block: 3 chunks, ragged rows
    ("bf16", "bf16", "f16", 264, 6, 5),       # d not a multiple of 512
    ("bf16", "bf16", "f16", 8192, 3, 3),      # the widest rows (16 chunks per lane, 64 KB of LDS)
    ("bf16", "f32", "bf16", 4104, 3, 9),      # 16 chunks per lane, the last partly filled
]


@pytest.mark.parametrize("wdt,xdt,odt,d,chunks,rows", ADALN_CASES)
def test_adaln_modulate(dit, wdt, xdt, odt, d, chunks, rows):
    say(f"adaln_modulate w={wdt} x={xdt} out={odt} d={d} chunks={chunks} rows={rows}")
    cond = di.draw((d,), 1.0, wdt, 9, "cond")
    w = di.draw((chunks * d, d), 0.02, wdt, 9, "w_mod")
    x = di.draw((rows, d), 1.0, xdt, 9, "x")
    mod = torch.empty(chunks * d, dtype=torch.float32, device="cuda")
    xo = torch.empty(rows, d, dtype=tdtype(odt), device="cuda")
    before = dit.launch_count()
    dit.adaln_modulate(dev(cond, wdt), dev(w, wdt), chunks, d, mod, x=dev(x, xdt), x_out=xo,
                       shift_chunk=chunks - 3, scale_chunk=chunks - 2, eps=1e-6)
    torch.cuda.synchronize()
    assert dit.launch_count() == before + 2
    m_ref, a_ref = o.adaln_modulate(o.widen(cond, wdt), o.widen(w, wdt), chunks, d, x=o.widen(x, xdt),
                                    shift_chunk=chunks - 3, scale_chunk=chunks - 2, eps=1e-6)
    m_gpu = host(mod).reshape(chunks, d)
    assert metric(m_gpu, m_ref) <= 1e-5
    # the output rounds the modulated value once; the fp32 vectors add < 1e-5 relative
    check(host(xo), a_ref, odt, tol_ulp=0.75, what="x_out")


def test_adaln_gemv_only(dit):
    say("adaln_modulate GEMV only")
    d = 3072
    cond = di.draw((d,), 1.0, "bf16", 10, "cond")
    w = di.draw((6 * d, d), 0.02, "bf16", 10, "w_mod")
    mod = torch.empty(6 * d, dtype=torch.float32, device="cuda")
    before = dit.launch_count()
    dit.adaln_modulate(dev(cond, "bf16"), dev(w, "bf16"), 6, d, mod)
    torch.cuda.synchronize()
    assert dit.launch_count() == before + 1
    ref = o.adaln_modulation(o.widen(w, "bf16"), o.widen(cond, "bf16"))
    assert metric(host(mod), ref) <= 1e-5


@pytest.mark.parametrize("wdt", ["bf16", "f32"])
def test_adaln_gemv_long_cond(dit, wdt):
    """A conditioning vector longer than one staging pass of SiLU(c) (4096 values) and not a whole
    number of 64-lane slices: the GEMV's multi-pass staging and partial last slice."""
    say(f"adaln_modulate GEMV, 9000-long cond, {wdt}")
    d_cond, d = 9000, 264
    cond = di.draw((d_cond,), 1.0, wdt, 11, "cond")
    w = di.draw((2 * d, d_cond), 0.02, wdt, 11, "w_mod")
    mod = torch.empty(2 * d, dtype=torch.float32, device="cuda")
    dit.adaln_modulate(dev(cond, wdt), dev(w, wdt), 2, d, mod)
    torch.cuda.synchronize()
    ref = o.adaln_modulation(o.widen(w, wdt), o.widen(cond, wdt))
    assert metric(host(mod), ref) <= 1e-5


ATTN_CASES = [
    ("f32", 80, 2),
    ("f32", 333, 1),
    ("f16", 80, 2),
    ("f16", 1, 3),
    ("f16", 77, 2),
    ("f16", 64, 1),         # exactly one key tile
    ("f16", 128, 1),        # two full tiles, no tail
    ("f16", 130, 1),        # two full tiles + a 2-key tail
    ("bf16", 200, 1),       # three full tiles + an 8-key tail
    ("f16", 1536, 24),
    ("f16", 4608, 24),
    ("bf16", 77, 2),
    ("bf16", 4608, 24),
]


@pytest.mark.parametrize("dtype,n,heads", ATTN_CASES)
def test_joint_attention(dit, dtype, n, heads):
    say(f"joint_attention {dtype} n={n} heads={heads}")
    d = 128 * heads
    qkv = di.draw((n, 3 * d), 1.0, dtype, 11, "q")
    t = dev(qkv, dtype)
    o_t = torch.empty(n, d, dtype=tdtype(dtype), device="cuda")
    before = dit.launch_count()
    dit.joint_attention(t[:, :d], t[:, d:2 * d], t[:, 2 * d:], o_t, heads)
    torch.cuda.synchronize()
    assert dit.launch_count() == before + 1
    x = o.widen(qkv, dtype)
    rows = None
    if n > 2000:
        rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(n).choice(n, 300, replace=False)]))
    ref = o.joint_attention(x[:, :d], x[:, d:2 * d], x[:, 2 * d:], heads, 128, q_rows=rows)
    got = host(o_t) if rows is None else host(o_t)[rows]
    if dtype == "f32":
        check(got, ref, dtype, what="O")
    else:
        ref_abs = o.joint_attention(x[:, :d], x[:, d:2 * d], np.abs(x[:, 2 * d:]), heads, 128, q_rows=rows)
        check_attention(got, ref, ref_abs, dtype)


def test_joint_attention_strided_output_and_canary(dit):
    # output written into the first d columns of a wider buffer (the single-stream layout);
    # the columns beyond must stay untouched.
    say("joint_attention strided output")
    n, heads = 300, 4
    d = 128 * heads
    qkv = di.draw((n, 3 * d), 1.0, "f16", 12, "q")
    t = dev(qkv, "f16")
    buf = torch.full((n, d + 640), float("nan"), dtype=torch.float16, device="cuda")
    dit.joint_attention(t[:, :d], t[:, d:2 * d], t[:, 2 * d:], buf[:, :d], heads)
    torch.cuda.synchronize()
    out = host(buf)
    assert np.isnan(out[:, d:]).all()
    x = o.widen(qkv, "f16")
    ref = o.joint_attention(x[:, :d], x[:, d:2 * d], x[:, 2 * d:], heads, 128)
    ref_abs = o.joint_attention(x[:, :d], x[:, d:2 * d], np.abs(x[:, 2 * d:]), heads, 128)
    check_attention(out[:, :d], ref, ref_abs, "f16")


def test_joint_attention_constant_scores_mean(dit):
    # q = 0: every score equal -> each output row is the mean of v over all tokens
    say("joint_attention constant scores")
    n, heads = 1000, 2
    d = 128 * heads
    v = di.draw((n, d), 1.0, "f16", 13, "v")
    q = torch.zeros(n, d, dtype=torch.float16, device="cuda")
    k = dev(di.draw((n, d), 1.0, "f16", 13, "k"), "f16")
    out = torch.empty(n, d, dtype=torch.float16, device="cuda")
    dit.joint_attention(q, k, dev(v, "f16"), out, heads)
    vv = o.widen(v, "f16")
    mean = np.broadcast_to(vv.mean(axis=0), (n, d))
    check_attention(host(out), mean, np.broadcast_to(np.abs(vv).mean(axis=0), (n, d)), "f16", what="mean")


@pytest.mark.parametrize("scale", [0.0, -0.21, 0.35])
def test_joint_attention_softmax_scale(dit, scale):
    # zero scale (uniform weights), a negative scale (the row max of the scaled scores is the
    # min of the raw ones) and a non-default positive one
    say(f"joint_attention scale={scale}")
    n, heads = 200, 2
    d = 128 * heads
    qkv = di.draw((n, 3 * d), 1.0, "f16", 14, "q")
    t = dev(qkv, "f16")
    out = torch.empty(n, d, dtype=torch.float16, device="cuda")
    dit.joint_attention(t[:, :d], t[:, d:2 * d], t[:, 2 * d:], out, heads, softmax_scale=scale)
    x = o.widen(qkv, "f16")
    ref = o.joint_attention(x[:, :d], x[:, d:2 * d], x[:, 2 * d:], heads, 128, scale=scale)
    ref_abs = o.joint_attention(x[:, :d], x[:, d:2 * d], np.abs(x[:, 2 * d:]), heads, 128, scale=scale)
    check_attention(host(out), ref, ref_abs, "f16")


@pytest.mark.parametrize("direction", [1, -1])
def test_joint_attention_drifting_scores(dit, direction):
    # scores that rise (or fall) steadily along the keys, over ~100 in base-2 units: the
    # running max is raised again and again tile after tile (or never after the first)
    say(f"joint_attention drifting scores, direction {direction}")
    n, heads = 1000, 1
    rng = np.random.default_rng(15)
    b = np.linspace(-2.0, 4.0, n) * direction
    q = np.ones((n, 128)) + 0.3 * rng.standard_normal((n, 128))
    k = b[:, None] * np.ones((1, 128)) + 0.3 * rng.standard_normal((n, 128))
    v = rng.standard_normal((n, 128))
    qh, kh, vh = (np.asarray(a, np.float16) for a in (q, k, v))
    out = torch.empty(n, 128, dtype=torch.float16, device="cuda")
    dit.joint_attention(torch.from_numpy(qh).cuda(), torch.from_numpy(kh).cuda(), torch.from_numpy(vh).cuda(),
                        out, heads)
    x = [a.astype(np.float64) for a in (qh, kh, vh)]
    ref = o.joint_attention(x[0], x[1], x[2], heads, 128)
    ref_abs = o.joint_attention(x[0], x[1], np.abs(x[2]), heads, 128)
    check_attention(host(out), ref, ref_abs, "f16")


def test_empty_calls_launch_nothing(dit):
    before = dit.launch_count()
    q = torch.empty(0, 256, dtype=torch.float16, device="cuda")
    dit.joint_attention(q, q, q, torch.empty(0, 256, dtype=torch.float16, device="cuda"), 2)
    pos = torch.empty(0, 4, dtype=torch.int32, device="cuda")
    w = torch.ones(2, 2, 128, dtype=torch.bfloat16, device="cuda")
    dit.qk_rmsnorm_rope(q, torch.empty(0, 256, dtype=torch.float16, device="cuda"), 2, w, 0, pos)
    assert dit.launch_count() == before

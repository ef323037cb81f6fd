"""Per-entry-point parity of the HIP path against the fp64 oracle (GPU).

Each test draws seeded inputs, runs one C-ABI entry point through the binding, and
compares element by element with the oracle stage it implements.  Bars:
  * fp32 calls: max|gpu - oracle| / RMS(oracle) <= 1e-4;
  * bf16 calls: the same metric <= 2e-2, and every element within the rounding
    the output storage allows (the output is the oracle's value rounded once to
    bf16, up to fp32 arithmetic): |gpu - oracle| <= tol_ulp * ulp_bf16(oracle).
Every test also checks that the library really launched (dit_launch_count).
"""
import numpy as np
import pytest
import torch

import dit_inputs as di
from oracle import dit_oracle as o
from gpu_util import dev, host, metric, bf16_ulp, say, tdtype

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
    assert m <= 2e-2, f"{what}: max/RMS {m:.3e} > 2e-2"
    err = np.abs(gpu - ref)
    bound = tol_ulp * bf16_ulp(ref) + 1e-6 * np.sqrt(np.mean(ref ** 2))
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} elements beyond {tol_ulp} ulp, worst "
                           f"{np.max(err / bound):.2f}x at {np.unravel_index(np.argmax(err / bound), err.shape)}")
    return m


ROPE_CASES = [
    ("f32", 16, 8, 8, 2),       # the fp32 workload's shape
    ("bf16", 512, 64, 64, 24),  # 512 text + 64x64 image tokens, 24 heads
    ("bf16", 5, 3, 7, 3),       # ragged
    ("bf16", 1, 1, 1, 1),       # one text and one image token
    ("bf16", 0, 2, 3, 2),       # image only
]


@pytest.mark.parametrize("dtype,n_txt,gh,gw,heads", ROPE_CASES)
def test_qk_rmsnorm_rope(dit, dtype, n_txt, gh, gw, heads):
    say(f"qk_rmsnorm_rope {dtype} n_txt={n_txt} grid={gh}x{gw} heads={heads}")
    cfg = _cfg(dtype, n_txt, gh, gw, heads)
    n, d = cfg.n_tok, cfg.d
    qkv = di.draw((n, 3 * d), 1.5, dtype, 7, "q")
    w = np.stack([di._qk_norm_weights(cfg, 7, 0, "txt", "random"),
                  di._qk_norm_weights(cfg, 7, 0, "img", "random")])   # [2 sets][2][128]
    pos = di.positions(n_txt, gh, gw)
    t = dev(qkv, dtype)
    before = dit.launch_count()
    dit.qk_rmsnorm_rope(t[:, :d], t[:, d:2 * d], heads, dev(w, dtype), n_txt, dev(pos, "i32"), eps=1e-6)
    torch.cuda.synchronize()
    assert dit.launch_count() == before + 1
    out = host(t)
    x = o.widen(qkv, dtype)
    rq, rk = o.qk_rmsnorm_rope(x[:, :d], x[:, d:2 * d], heads, 128, o.widen(w, dtype), n_txt, 1e-6, pos, AXES, 1e4)
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
    ("f32", "f32", 256, 6, 80),
    ("bf16", "bf16", 3072, 6, 4608),
    ("bf16", "f32", 3072, 6, 600),     # fp32 input (the residual stream h)
    ("bf16", "bf16", 3072, 3, 37),     # single-stream block: 3 chunks, ragged rows
    ("bf16", "bf16", 264, 6, 5),       # d not a multiple of 512
]


@pytest.mark.parametrize("dtype,xdt,d,chunks,rows", ADALN_CASES)
def test_adaln_modulate(dit, dtype, xdt, d, chunks, rows):
    say(f"adaln_modulate {dtype} x={xdt} d={d} chunks={chunks} rows={rows}")
    cond = di.draw((d,), 1.0, dtype, 9, "cond")
    w = di.draw((chunks * d, d), 0.02, dtype, 9, "w_mod")
    x = di.draw((rows, d), 1.0, xdt, 9, "x")
    mod = torch.empty(chunks * d, dtype=torch.float32, device="cuda")
    xo = torch.empty(rows, d, dtype=tdtype(dtype), device="cuda")
    before = dit.launch_count()
    dit.adaln_modulate(dev(cond, dtype), dev(w, dtype), chunks, d, mod, x=dev(x, xdt), x_out=xo,
                       shift_chunk=chunks - 3, scale_chunk=chunks - 2, eps=1e-6)
    torch.cuda.synchronize()
    assert dit.launch_count() == before + 2
    m_ref, a_ref = o.adaln_modulate(o.widen(cond, dtype), o.widen(w, dtype), chunks, d, x=o.widen(x, xdt),
                                    shift_chunk=chunks - 3, scale_chunk=chunks - 2, eps=1e-6)
    m_gpu = host(mod).reshape(chunks, d)
    assert metric(m_gpu, m_ref) <= 1e-5
    # the bf16 output rounds the modulated value once; the fp32 vectors add < 1e-5 relative
    check(host(xo), a_ref, dtype, tol_ulp=0.75, what="x_out")


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


ATTN_CASES = [
    ("f32", 80, 2),
    ("f32", 333, 1),
    ("bf16", 80, 2),
    ("bf16", 1, 3),
    ("bf16", 77, 2),
    ("bf16", 1536, 24),
    ("bf16", 4608, 24),
]


@pytest.mark.parametrize("dtype,n,heads", ATTN_CASES)
def test_joint_attention(dit, dtype, n, heads):
    say(f"joint_attention {dtype} n={n} heads={heads}")
    d = 128 * heads
    # q, k with RMS ~1 per head after QK-norm in the block; draw N(0,1) and scale scores up
    # to the block's range by drawing q with std 1.5
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
    # bf16: P is rounded to bf16 before the PV product -> allow 1.5 ulp of the output
    check(got, ref, dtype, tol_ulp=1.5, what="O")


def test_joint_attention_strided_output_and_canary(dit):
    # output written into the first d columns of a wider buffer (the single-stream layout);
    # the columns beyond must stay untouched.
    say("joint_attention strided output")
    n, heads = 300, 4
    d = 128 * heads
    qkv = di.draw((n, 3 * d), 1.0, "bf16", 12, "q")
    t = dev(qkv, "bf16")
    buf = torch.full((n, d + 640), float("nan"), dtype=torch.bfloat16, device="cuda")
    dit.joint_attention(t[:, :d], t[:, d:2 * d], t[:, 2 * d:], buf[:, :d], heads)
    torch.cuda.synchronize()
    out = host(buf)
    assert np.isnan(out[:, d:]).all()
    x = o.widen(qkv, "bf16")
    ref = o.joint_attention(x[:, :d], x[:, d:2 * d], x[:, 2 * d:], heads, 128)
    check(out[:, :d], ref, "bf16", tol_ulp=1.5, what="O")


def test_joint_attention_constant_scores_mean(dit):
    # q = 0: every score equal -> each output row is the mean of v over all tokens
    say("joint_attention constant scores")
    n, heads = 1000, 2
    d = 128 * heads
    v = di.draw((n, d), 1.0, "bf16", 13, "v")
    q = torch.zeros(n, d, dtype=torch.bfloat16, device="cuda")
    k = dev(di.draw((n, d), 1.0, "bf16", 13, "k"), "bf16")
    out = torch.empty(n, d, dtype=torch.bfloat16, device="cuda")
    dit.joint_attention(q, k, dev(v, "bf16"), out, heads)
    mean = o.widen(v, "bf16").mean(axis=0)
    check(host(out), np.broadcast_to(mean, (n, d)), "bf16", tol_ulp=1.5, what="mean")


def test_empty_calls_launch_nothing(dit):
    before = dit.launch_count()
    q = torch.empty(0, 256, dtype=torch.bfloat16, device="cuda")
    dit.joint_attention(q, q, q, torch.empty(0, 256, dtype=torch.bfloat16, device="cuda"), 2)
    pos = torch.empty(0, 4, dtype=torch.int32, device="cuda")
    w = torch.ones(2, 2, 128, dtype=torch.bfloat16, device="cuda")
    dit.qk_rmsnorm_rope(q, torch.empty(0, 256, dtype=torch.bfloat16, device="cuda"), 2, w, 0, pos)
    assert dit.launch_count() == before

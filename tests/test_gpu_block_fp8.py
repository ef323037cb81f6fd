"""fp8 (OCP e4m3) double-stream block on the GPU against the oracle's fp8 block (GPU).

``dit_block_forward_fp8`` runs the block's four weight products on e4m3 codes: the weights are
quantised per output row by ``dit_quantize_fp8`` (from the same bf16 bits the oracle reads), the
activations per row inside the block.  The oracle's fp8 block (``double_block(fp8=True)``)
quantises the same four products' operands from its exact values.

Bars.  An e4m3 step is 2^-3 of a value, so any upstream difference between two correct fp8
implementations (the block carries a, qkv, O, b, f and the probabilities in fp16; the oracle is
exact) moves some operands to the neighbouring code, and each such flip moves the element by up to
2^-3 of itself: per element, two correct fp8 blocks need not agree beyond the fp8 error itself.
What is unique is the size of that error and how closely the GPU follows the fp8 definition:
* small shapes (d = 384, where the fp8 error is ~1e-3 RMS): max|gpu - oracle_fp8| / RMS <= 5e-2;
* the 3072-wide workloads (fp8 error ~6% RMS): the GPU's RMS distance to the exact block within 5%
  of the oracle fp8 block's, and its RMS distance to the oracle fp8 block at most 0.7 of the fp8
  error (measured 0.5: the two share the deterministic part of the rounding, the flips do not).
"""
import numpy as np
import pytest
import torch

import dit_inputs as di
from oracle import dit_oracle as o
from gpu_util import dev, host, metric, say, shape_of

pytestmark = pytest.mark.gpu

BAR_FP8 = 5e-2


@pytest.fixture(scope="module")
def dit():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import attention_dit_block_amd as m
    return m


def fp8_weights(dit, w: dict) -> dict:
    """Stream weights for dit_block_forward_fp8: the four product matrices quantised on the GPU."""
    out = {"w_mod": dev(w["w_mod"], "bf16"), "qk_norm_w": dev(w["qk_norm_w"], "bf16")}
    for name in ("qkv", "o", "ffn_in", "ffn_out"):
        wt = dev(w["w_" + name], "bf16")
        q = torch.empty(wt.shape, dtype=torch.uint8, device="cuda")
        s = torch.empty(wt.shape[0], dtype=torch.float32, device="cuda")
        dit.quantize_fp8(wt, q, s)
        out["w_" + name], out["s_" + name] = q, s
    return out


def run_fp8(dit, cfg, inp, y_dtype="f32"):
    sh = shape_of(cfg, dit, y_dtype=dit.DIT_BF16 if y_dtype == "bf16" else dit.DIT_F32)
    ws = torch.empty(dit.block_fp8_workspace_size(sh), dtype=torch.uint8, device="cuda")
    yt = torch.empty(cfg.n_txt, cfg.d, dtype=torch.float32 if y_dtype == "f32" else torch.bfloat16, device="cuda")
    yi = torch.empty(cfg.n_img, cfg.d, dtype=yt.dtype, device="cuda")
    wt, wi = fp8_weights(dit, inp["txt"]), fp8_weights(dit, inp["img"])
    before = dit.launch_count()
    dit.block_forward_fp8(sh, wt, wi, dev(inp["cond"], "bf16"), dev(inp["pos"], "i32"), dev(inp["x_txt"], "bf16"),
                          dev(inp["x_img"], "bf16"), yt, yi, ws)
    torch.cuda.synchronize()
    assert dit.launch_count() == before + 11
    return host(yt), host(yi)


def rms_rel(gpu, ref):
    return float(np.sqrt(np.mean((gpu - ref) ** 2) / np.mean(ref ** 2)))


def check(cfg, gpu, rows_txt=None, rows_img=None, bar=None, wide=False):
    inp = gpu["inp"]
    ref8 = o.double_block(cfg, inp, rows_txt=rows_txt, rows_img=rows_img, fp8=True)
    ref = o.double_block(cfg, inp, rows_txt=rows_txt, rows_img=rows_img)
    for s in ("txt", "img"):
        g = gpu["y_" + s]
        m8, m = metric(g, ref8["y_" + s]), metric(g, ref["y_" + s])
        say(f"  {cfg.name} y_{s}: fp8 oracle max {m8:.3e} rms {rms_rel(g, ref8['y_' + s]):.3e}; exact oracle max "
            f"{m:.3e} rms {rms_rel(g, ref['y_' + s]):.3e}; oracle fp8 vs exact max "
            f"{metric(ref8['y_' + s], ref['y_' + s]):.3e} rms {rms_rel(ref8['y_' + s], ref['y_' + s]):.3e}")
        if bar is not None:
            assert m8 <= bar, f"y_{s}: {m8:.3e} > {bar}"
        if wide:
            e8 = rms_rel(ref8["y_" + s], ref["y_" + s])        # the fp8 error of the definition
            assert rms_rel(g, ref["y_" + s]) <= 1.05 * e8
            assert rms_rel(g, ref8["y_" + s]) <= 0.7 * e8


@pytest.mark.parametrize("n_txt,grid", [(7, (5, 9)), (40, (16, 19))])
def test_fp8_block_small_ragged(dit, n_txt, grid):
    cfg = di.BlockConfig(f"fp8_ragged_t{n_txt}", "bf16", d=384, n_heads=3, ffn_inner=1152, n_txt=n_txt,
                         grid_h=grid[0], grid_w=grid[1])
    say(f"fp8 double block {cfg.name}")
    inp = di.double_block_inputs(cfg, seed=3)
    yt, yi = run_fp8(dit, cfg, inp)
    check(cfg, {"inp": inp, "y_txt": yt, "y_img": yi}, wide=True)


@pytest.mark.parametrize("qk", ["ones", "random"])
def test_fp8_block_c1(dit, qk):
    cfg = di.CONFIGS[1]
    say(f"fp8 double block {cfg.name} qk={qk}")
    inp = di.double_block_inputs(cfg, seed=0, qk_norm=qk)
    yt, yi = run_fp8(dit, cfg, inp)
    check(cfg, {"inp": inp, "y_txt": yt, "y_img": yi}, wide=True)


def test_fp8_block_c2_sampled_rows_bf16_out(dit):
    cfg = di.CONFIGS[2]
    say(f"fp8 double block {cfg.name} (sampled rows, bf16 output)")
    inp = di.double_block_inputs(cfg, seed=0)
    yt, yi = run_fp8(dit, cfg, inp, y_dtype="bf16")
    rng = np.random.default_rng(5)
    rt = np.unique(np.concatenate([[0, cfg.n_txt - 1], rng.choice(cfg.n_txt, 24, replace=False)]))
    ri = np.unique(np.concatenate([[0, cfg.n_img - 1], rng.choice(cfg.n_img, 40, replace=False)]))
    check(cfg, {"inp": inp, "y_txt": yt[rt], "y_img": yi[ri]}, rows_txt=rt, rows_img=ri, wide=True)


@pytest.mark.parametrize("n_txt,grid", [(0, (4, 5)), (9, (0, 0)), (1, (1, 1))],
                         ids=["image_only", "text_only", "one_each"])
def test_fp8_block_degenerate_streams(dit, n_txt, grid):
    cfg = di.BlockConfig(f"fp8_edge_{n_txt}_{grid[0]}x{grid[1]}", "bf16", d=256, n_heads=2, ffn_inner=768,
                         n_txt=n_txt, grid_h=grid[0], grid_w=grid[1])
    say(f"fp8 double block {cfg.name}")
    inp = di.double_block_inputs(cfg, seed=4)
    yt, yi = run_fp8(dit, cfg, inp)
    ref8 = o.double_block(cfg, inp, fp8=True)
    for s, g in (("txt", yt), ("img", yi)):
        r = ref8["y_" + s]
        if r.size:
            m = metric(g, r)
            say(f"  {cfg.name} y_{s}: fp8 oracle max {m:.3e}")
            assert m <= BAR_FP8
        else:
            assert g.size == 0


# ---- the single-stream block ---------------------------------------------------------------------

def run_single_fp8(dit, cfg, inp):
    sh = shape_of(cfg, dit)
    ws = torch.empty(dit.single_block_fp8_workspace_size(sh), dtype=torch.uint8, device="cuda")
    y = torch.empty(cfg.n_tok, cfg.d, dtype=torch.float32, device="cuda")
    w = inp["w"]
    wd = {"w_mod": dev(w["w_mod"], "bf16"), "qk_norm_w": dev(w["qk_norm_w"], "bf16")}
    for name, sname in (("w_1", "s_1"), ("w_2", "s_2")):
        wt = dev(w[name], "bf16")
        q = torch.empty(wt.shape, dtype=torch.uint8, device="cuda")
        s = torch.empty(wt.shape[0], dtype=torch.float32, device="cuda")
        dit.quantize_fp8(wt, q, s)
        wd[name], wd[sname] = q, s
    before = dit.launch_count()
    dit.single_block_forward_fp8(sh, wd, dev(inp["cond"], "bf16"), dev(inp["pos"], "i32"), dev(inp["x"], "bf16"), y,
                                 ws)
    torch.cuda.synchronize()
    assert dit.launch_count() == before + 8
    return host(y)


def check_single(cfg, inp, y, rows=None, bar=None, wide=False):
    ref8 = o.single_block(cfg, inp, rows=rows, fp8=True)["y"]
    ref = o.single_block(cfg, inp, rows=rows)["y"]
    m8, e8 = metric(y, ref8), rms_rel(ref8, ref)
    say(f"  {cfg.name} y: fp8 oracle max {m8:.3e} rms {rms_rel(y, ref8):.3e}; exact oracle rms {rms_rel(y, ref):.3e}; "
        f"oracle fp8 vs exact rms {e8:.3e}")
    if bar is not None:
        assert m8 <= bar
    if wide:
        assert rms_rel(y, ref) <= 1.05 * e8
        assert rms_rel(y, ref8) <= 0.7 * e8


@pytest.mark.parametrize("n_txt,grid", [(16, (8, 8)), (0, (4, 5)), (1, (1, 1))], ids=["small", "image_only", "one_each"])
def test_fp8_single_block_small(dit, n_txt, grid):
    cfg = di.BlockConfig(f"fp8_single_{n_txt}_{grid[0]}x{grid[1]}", "bf16", d=256, n_heads=2, ffn_inner=768,
                         n_txt=n_txt, grid_h=grid[0], grid_w=grid[1])
    say(f"fp8 single block {cfg.name}")
    inp = di.single_block_inputs(cfg, seed=7, qk_norm="random")
    check_single(cfg, inp, run_single_fp8(dit, cfg, inp), bar=BAR_FP8)


def test_fp8_single_block_c3_shape_sampled(dit):
    cfg = di.CONFIGS[3]
    say(f"fp8 single block at {cfg.name} shape (sampled rows)")
    inp = di.single_block_inputs(cfg, seed=0)
    y = run_single_fp8(dit, cfg, inp)
    rows = np.unique(np.concatenate([[0, cfg.n_tok - 1], np.random.default_rng(9).choice(cfg.n_tok, 64, replace=False)]))
    check_single(cfg, inp, y[rows], rows=rows, wide=True)


def test_fp8_block_c2_last_product_elementwise(dit):
    """Element-wise check of the full-width fp8 block (512 + 4096 tokens, d = 3072, F = 9216), every
    output tile: its last product y = h + gate2 (f W_down^T) on e4m3 codes, teacher-forced on the
    GPU's own fp32 residual h, AdaLN gates and e4m3 codes / row scales of f, read back from the
    workspace after the call.  Given those, the result is fixed up to fp32 rounding: the e4m3
    products are exact in fp32, a sum of K of them in any order is within (K - 1) 2^-24 sum|terms|
    (2^-23 with truncating adds), the two scale products add 2^-24 each, and the fused
    gate * acc + h rounds once more (2^-24 |y|).  Workspace layout: the range-flag word (256 bytes),
    the AdaLN vectors [2][6d] fp32, a, qkv, O (fp16), h (fp32), ...; the last two buffers are the
    current product's activation codes [n, max(d, F)] and row scales [n]."""
    cfg = di.CONFIGS[2]
    say(f"fp8 double block {cfg.name}: last product element-wise, teacher-forced")
    inp = di.double_block_inputs(cfg, seed=0)
    n, d, F = cfg.n_tok, cfg.d, cfg.ffn_inner
    sh = shape_of(cfg, dit)
    total = dit.block_fp8_workspace_size(sh)
    ws = torch.empty(total, dtype=torch.uint8, device="cuda")
    yt = torch.empty(cfg.n_txt, d, dtype=torch.float32, device="cuda")
    yi = torch.empty(cfg.n_img, d, dtype=torch.float32, device="cuda")
    wt, wi = fp8_weights(dit, inp["txt"]), fp8_weights(dit, inp["img"])
    dit.block_forward_fp8(sh, wt, wi, dev(inp["cond"], "bf16"), dev(inp["pos"], "i32"), dev(inp["x_txt"], "bf16"),
                          dev(inp["x_img"], "bf16"), yt, yi, ws)
    torch.cuda.synchronize()

    def up(x):
        return (x + 255) // 256 * 256
    wsh = ws.cpu().numpy()
    off_mod = 256
    off_h = off_mod + up(12 * d * 4) + up(n * d * 2) + up(n * 3 * d * 2) + up(n * d * 2)
    off_sq = total - up(n * 4)
    off_q8 = off_sq - up(n * max(d, F))
    mod = wsh[off_mod:off_mod + 12 * d * 4].view(np.float32).reshape(2, 6, d).astype(np.float64)
    h = wsh[off_h:off_h + n * d * 4].view(np.float32).reshape(n, d).astype(np.float64)
    fq = wsh[off_q8:off_q8 + n * F].reshape(n, F)
    sf = wsh[off_sq:off_sq + n * 4].view(np.float32)
    rng = np.random.default_rng(17)
    worst = 0.0
    for si, (s, y, w, rows0, nrows) in enumerate((("txt", yt, wt, 0, cfg.n_txt), ("img", yi, wi, cfg.n_txt, cfg.n_img))):
        # two rows of every 256-row tile of this stream's problem, and its first and last rows
        r = np.unique(np.concatenate([[0, nrows - 1]] + [t * 256 + rng.choice(min(256, nrows - t * 256), 2, replace=False)
                                                         for t in range((nrows + 255) // 256)]))
        wq, sw = w["w_ffn_out"].cpu().numpy(), w["s_ffn_out"].cpu().numpy()
        acc = o.linear_fp8(fq[rows0 + r], sf[rows0 + r], wq, sw)
        abs_sum = o.linear_fp8(fq[rows0 + r] & 0x7F, sf[rows0 + r], wq & 0x7F, sw)
        gate = mod[si, 5]
        ref = h[rows0 + r] + gate * acc
        bound = np.abs(gate) * (F * 2.0 ** -23 + 2.0 ** -22) * abs_sum + 2.0 ** -23 * np.abs(ref) + 1e-30
        err = np.abs(host(y)[r] - ref)
        worst = max(worst, float(np.max(err / bound)))
        say(f"  y_{s}: {len(r)} rows x {d}: max err / bound {np.max(err / bound):.3f}, max|gpu - ref|/RMS "
            f"{metric(host(y)[r], ref):.2e}")
        assert np.all(err <= bound), f"y_{s}: {np.sum(err > bound)} elements beyond the bound"
    assert worst > 0.0


_RAGGED_FP8ATTN = di.BlockConfig("ragged_fp8attn", "bf16", d=384, n_heads=3, ffn_inner=1152, n_txt=7, grid_h=5, grid_w=9)


@pytest.mark.parametrize("cfg, act", [(_RAGGED_FP8ATTN, "f16"), (_RAGGED_FP8ATTN, "bf16"), (di.CONFIGS[1], "f16")],
                         ids=["ragged", "ragged_bf16_act", "c1"])
def test_fp8_block_attention_operands_and_output(dit, cfg, act):
    """The fp8 block's attention, teacher-forced on the GPU's own values read back from the
    workspace: from its fp16 q, k, v (QKV product output), the oracle's QK-norm + RoPE (exact) and
    fp8_attention_operands give the codes and scales the e4m3 mode of the QK-norm + RoPE kernel must
    write -- k and v scales bit-identical (the same fp32 operations on the same values), v codes
    bit-identical, q and k codes equal or one e4m3 step apart (the GPU rotates in fp32; the oracle
    exactly), q scales within 1e-5.  The attention output O is then held to the fp8 attention bound
    (tests/test_gpu_attention_fp8.py) against the oracle's fp8 attention on the GPU's own codes.
    Workspace layout from the end: ... | attention codes [n, 3d] | scales sq [n, H], sk [H],
    sv [H], |v| maxima [H] | product codes [n, max(d, F)] | product scales [n]."""
    import test_gpu_attention_fp8 as ta
    say(f"fp8 double block {cfg.name}: attention operands and output, teacher-forced")
    inp = di.double_block_inputs(cfg, seed=4, qk_norm="random")
    n, d, F, H, D = cfg.n_tok, cfg.d, cfg.ffn_inner, cfg.n_heads, 128
    sh = shape_of(cfg, dit, act_dtype=dit.DIT_BF16 if act == "bf16" else None)
    total = dit.block_fp8_workspace_size(sh)
    ws = torch.empty(total, dtype=torch.uint8, device="cuda")
    yt = torch.empty(cfg.n_txt, d, dtype=torch.float32, device="cuda")
    yi = torch.empty(cfg.n_img, d, dtype=torch.float32, device="cuda")
    wt, wi = fp8_weights(dit, inp["txt"]), fp8_weights(dit, inp["img"])
    dit.block_forward_fp8(sh, wt, wi, dev(inp["cond"], "bf16"), dev(inp["pos"], "i32"), dev(inp["x_txt"], "bf16"),
                          dev(inp["x_img"], "bf16"), yt, yi, ws)
    torch.cuda.synchronize()

    def up(x):
        return (x + 255) // 256 * 256
    wsh = ws.cpu().numpy()
    off_qkv = 256 + up(12 * d * 4) + up(n * d * 2)
    off_o = off_qkv + up(n * 3 * d * 2)
    off_sq = total - up(n * 4)
    off_q8 = off_sq - up(n * max(d, F))
    off_a8s = off_q8 - up((n * H + 3 * H) * 4)
    off_a8 = off_a8s - up(n * 3 * d)
    def act16(buf, shape):
        if act == "bf16":
            return di.f32_from_bf16_bits(buf.view(np.uint16)).reshape(shape).astype(np.float64)
        return buf.view(np.float16).reshape(shape).astype(np.float64)
    qkv = act16(wsh[off_qkv:off_qkv + n * 3 * d * 2], (n, 3 * d))
    o_gpu = act16(wsh[off_o:off_o + n * d * 2], (n, d))
    a8 = wsh[off_a8:off_a8 + n * 3 * d].reshape(n, 3 * d)
    sc = wsh[off_a8s:off_a8s + (n * H + 3 * H) * 4].view(np.float32)
    sq, sk, sv = sc[:n * H].reshape(n, H), sc[n * H:n * H + H], sc[n * H + H:n * H + 2 * H]
    # the oracle's rotation of the GPU's q, k and its operands (k bound from both streams' k weights)
    qk_w = np.stack([o.widen(inp["txt"]["qk_norm_w"], "bf16").reshape(2, D),
                     o.widen(inp["img"]["qk_norm_w"], "bf16").reshape(2, D)])
    q, k = o.qk_rmsnorm_rope(qkv[:, :d], qkv[:, d:2 * d], H, D, qk_w, cfg.n_txt, cfg.eps_qk, inp["pos"],
                             cfg.axes_dim, cfg.theta)
    v = qkv[:, 2 * d:]
    q8r, sqr, k8r, skr, v8r, svr = o.fp8_attention_operands(q, k, v, H, D, float(np.max(np.abs(qk_w[:, 1]))))
    np.testing.assert_array_equal(sk, skr)
    np.testing.assert_array_equal(sv, svr)
    np.testing.assert_array_equal(a8[:, 2 * d:], v8r)
    np.testing.assert_allclose(sq, sqr, rtol=1e-5)

    def step_apart(got, ref):
        # e4m3 codes of one sign are ordered like their values: equal, or neighbours
        g, r = got.astype(np.int32), ref.astype(np.int32)
        same_sign = (g & 0x80) == (r & 0x80)
        near = same_sign & (np.abs((g & 0x7F) - (r & 0x7F)) <= 1)
        zero = ((g & 0x7F) <= 1) & ((r & 0x7F) <= 1)          # -0 / +0 / smallest subnormals
        return near | zero, float(np.mean(g == r))
    for name, got, ref in (("q", a8[:, :d], q8r), ("k", a8[:, d:2 * d], k8r)):
        ok, agree = step_apart(got, ref)
        say(f"  {name} codes: {agree:.4%} identical")
        assert np.all(ok), f"{name}: {np.sum(~ok)} codes more than one step from the oracle's"
        assert agree > 0.99
    # O against the oracle's fp8 attention on the GPU's own codes
    x = {"q8": a8[:, :d], "sq": sq, "k8": a8[:, d:2 * d], "sk": sk, "v8": a8[:, 2 * d:], "sv": sv}
    rows = np.arange(n) if n <= 256 else np.unique(np.concatenate(
        [[0, cfg.n_txt - 1, cfg.n_txt, n - 1], np.random.default_rng(3).choice(n, 60, replace=False)]))
    full = np.zeros((n, d))
    full[rows] = o_gpu[rows]
    ta._check(full, x, H, rows, act)


@pytest.mark.parametrize("cfg", [di.BlockConfig("attn_split_fp8", "bf16", d=256, n_heads=2, ffn_inner=768, n_txt=77,
                                                grid_h=64, grid_w=65), di.CONFIGS[2]], ids=["attn_split", "c2"])
@pytest.mark.parametrize("polls", [0, 1])
def test_fp8_block_split_owners_compute_missing_pieces(dit, cfg, polls):
    """The fp8 attention's key split on the block path (the 16-bit kernel's hand-over, attn_split.h):
    with a wait bound of 0 every owner computes all of its unit's pieces, with 1 poll some pieces are
    handed over and some claimed.  The block stays within the fp8 bars (small shape: 5e-2 max/RMS
    against the oracle's fp8 block; c2: within 1% RMS of the default run, whose pieces may round
    their probabilities against a different running max), and a later default run repeats the first
    bit for bit (no flag left behind)."""
    say(f"fp8 block split hand-over, wait bound {polls}: {cfg.name}")
    inp = di.double_block_inputs(cfg, seed=6)
    sh = shape_of(cfg, dit)
    ws = torch.empty(dit.block_fp8_workspace_size(sh), dtype=torch.uint8, device="cuda")
    yt = torch.empty(cfg.n_txt, cfg.d, dtype=torch.float32, device="cuda")
    yi = torch.empty(cfg.n_img, cfg.d, dtype=torch.float32, device="cuda")
    wt, wi = fp8_weights(dit, inp["txt"]), fp8_weights(dit, inp["img"])
    args = (dev(inp["cond"], "bf16"), dev(inp["pos"], "i32"), dev(inp["x_txt"], "bf16"), dev(inp["x_img"], "bf16"))

    def run():
        dit.block_forward_fp8(sh, wt, wi, *args, yt, yi, ws)
        torch.cuda.synchronize()
        return host(yt), host(yi)
    dit.set_split_wait_limit(-1)
    base = run()
    try:
        dit.set_split_wait_limit(polls)
        got = run()
    finally:
        dit.set_split_wait_limit(-1)
    after = run()
    ref8 = o.double_block(cfg, inp, fp8=True) if cfg.n_tok < 6000 else None
    for i, s in enumerate(("txt", "img")):
        assert np.all(np.isfinite(got[i]))
        np.testing.assert_array_equal(after[i], base[i])
        rel = rms_rel(got[i], base[i])
        say(f"  y_{s}: RMS distance to the default run {rel:.2e}")
        if cfg.n_tok < 6000 and cfg.d == 256:
            assert metric(got[i], ref8["y_" + s]) <= BAR_FP8
        else:
            assert rel <= 1e-2

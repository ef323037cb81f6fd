"""Guards of the block path (GPU): the split-work hand-over never drops a piece, and the fp16
activation range is watched.

Split work.  When a launch splits its last round of work units over a persistent grid, the owner
of a unit adds the partial results other workgroups publish for their pieces; if a partial does
not arrive within the wait bound, the owner computes that piece itself.  With the bound at 0 the
hand-over is off and every owner computes all of its unit's pieces (the path taken when the grid's
workgroups are not all resident); with a bound of 1 poll some pieces are handed over and some
claimed, racing the producers.  Either way the block must stay within the oracle bar, and the
launches after it (default bound) must be exactly the result of a run that never changed it: no
flag may be left behind.

Range.  With fp16 activations (act_dtype DIT_F16) every kernel that rounds an fp32 result to an
fp16 activation ORs DIT_RANGE_F16 into the call's flag word (workspace bytes 0-3) when a value is
NaN or above 65504 in magnitude; the block's first kernel resets the word."""
import numpy as np
import pytest
import torch

import dit_inputs as di
from oracle import dit_oracle as o
from gpu_util import dev, host, metric, say, shape_of, upload_stream_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dit():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import attention_dit_block_amd as m
    yield m
    m.set_split_wait_limit(-1)


def _block(dit, cfg, inp, f16w=True, act=None, ws=None):
    sh = shape_of(cfg, dit, act_dtype=act)
    if f16w:
        sh.gemm_w_dtype = dit.DIT_F16
    if ws is None:
        ws = torch.empty(dit.block_workspace_size(sh), dtype=torch.uint8, device="cuda")
    yt = torch.empty(cfg.n_txt, cfg.d, dtype=torch.float32, device="cuda")
    yi = torch.empty(cfg.n_img, cfg.d, dtype=torch.float32, device="cuda")
    wt, wi = upload_stream_weights(inp["txt"], "bf16", f16w), upload_stream_weights(inp["img"], "bf16", f16w)
    args = (dev(inp["cond"], "bf16"), dev(inp["pos"], "i32"), dev(inp["x_txt"], "bf16"), dev(inp["x_img"], "bf16"))

    def run():
        dit.block_forward(sh, wt, wi, *args, yt, yi, ws)
        torch.cuda.synchronize()
        return host(yt), host(yi), dit.workspace_flags(ws)
    return run


# c2 (FFN-in and attention split), c1 (the d-output GEMMs split every tile), and a small block whose
# attention splits every unit's key tiles about eight ways
SPLIT_CASES = [di.CONFIGS[2], di.CONFIGS[1],
               di.BlockConfig("attn_split", "bf16", d=256, n_heads=2, ffn_inner=768, n_txt=77, grid_h=64, grid_w=65)]


@pytest.mark.parametrize("cfg", SPLIT_CASES, ids=lambda c: c.name)
@pytest.mark.parametrize("polls", [0, 1])
def test_split_owners_compute_missing_pieces(dit, cfg, polls):
    say(f"split hand-over with a wait bound of {polls}: {cfg.name}")
    inp = di.double_block_inputs(cfg, seed=5)
    run = _block(dit, cfg, inp)
    dit.set_split_wait_limit(-1)
    base = run()
    try:
        dit.set_split_wait_limit(polls)
        got = run()
    finally:
        dit.set_split_wait_limit(-1)
    after = run()
    ref = o.double_block(cfg, inp)
    for i, s in enumerate(("txt", "img")):
        m = metric(got[i], ref["y_" + s])
        say(f"  y_{s}: max|gpu-oracle|/RMS = {m:.3e} (default bound {metric(base[i], ref['y_' + s]):.3e})")
        assert m <= 2e-2
        # a run with the default bound after it repeats the first one bit for bit (no stale flags)
        np.testing.assert_array_equal(after[i], base[i])
    assert got[2] == 0 and base[2] == 0 and after[2] == 0


SMALL = di.BlockConfig("range", "bf16", d=256, n_heads=2, ffn_inner=768, n_txt=5, grid_h=4, grid_w=4)


def test_fp16_range_flag_from_the_modulation(dit):
    # shift1 of the image stream = 4000 sum_k SiLU(c_k) ~ 2e5 (E SiLU(c) ~ 0.21 for c ~ N(0, 1), 256
    # terms): a = (1 + scale) RMSNorm(x) + shift leaves fp16's range
    inp = di.double_block_inputs(SMALL, seed=6)
    wm = o.widen(inp["img"]["w_mod"], "bf16").astype(np.float32)
    wm[:SMALL.d] = 4000.0
    inp["img"] = dict(inp["img"], w_mod=di.bf16_bits_from_f32(wm))
    yt, yi, flags = _block(dit, SMALL, inp, act=dit.DIT_F16)()
    say(f"  flags {flags:#x}")
    assert flags == dit.DIT_RANGE_F16
    # the same block with bf16 activations stays finite and raises nothing
    yt, yi, flags = _block(dit, SMALL, inp, f16w=False, act=dit.DIT_BF16)()
    assert flags == 0 and np.all(np.isfinite(yi))


def test_fp16_range_flag_from_a_gemm_epilogue_and_reset(dit):
    # W_in of the text stream scaled by 2^12: SiLU(g) u from the FFN-in epilogue reaches ~1e8
    inp = di.double_block_inputs(SMALL, seed=7)
    w = o.widen(inp["txt"]["w_ffn_in"], "bf16").astype(np.float32) * np.float32(4096.0)
    big = dict(inp, txt=dict(inp["txt"], w_ffn_in=di.bf16_bits_from_f32(w)))
    sh = shape_of(SMALL, dit, act_dtype=dit.DIT_F16)
    ws = torch.empty(dit.block_workspace_size(sh), dtype=torch.uint8, device="cuda")
    assert _block(dit, SMALL, big, f16w=False, act=dit.DIT_F16, ws=ws)()[2] == dit.DIT_RANGE_F16
    # a normal block on the same workspace resets the word in its first kernel
    yt, yi, flags = _block(dit, SMALL, inp, f16w=False, act=dit.DIT_F16, ws=ws)()
    assert flags == 0
    ref = o.double_block(SMALL, inp)
    assert metric(yt, ref["y_txt"]) <= 2e-2 and metric(yi, ref["y_img"]) <= 2e-2

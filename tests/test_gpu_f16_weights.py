"""fp16 copies of the matrix-product weights (gemm_w_dtype = DIT_F16) on the GPU.

The 16-bit block with fp16 activations converts each bf16 weight tile to fp16 while staging it;
with fp16 copies made once by dit_convert_bf16_to_f16 (the same round-to-nearest-even conversion)
the GEMMs stage them as they are.  The MFMA operands are then the same values, so the block output
must be bit-identical.  The conversion itself is checked against numpy's float32 -> float16 rounding
of the widened bf16 values (bf16 -> fp32 is exact).
"""
import numpy as np
import pytest
import torch

import dit_inputs as di
from gpu_util import dev, host, say, shape_of, upload_stream_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dit():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import attention_dit_block_amd as m
    return m


@pytest.mark.parametrize("n", [1, 7, 8, 4099, 1 << 20])
def test_convert_bf16_to_f16(dit, n):
    rng = np.random.default_rng(n)
    # magnitudes from fp16's subnormals (2^-24) to its largest finite value, both signs, zeros
    mag = np.exp2(rng.uniform(-26, 15.9, n)).astype(np.float32)
    x = (mag * rng.choice([-1.0, 1.0], n)).astype(np.float32)
    x[rng.integers(0, n, max(1, n // 100))] = 0.0
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)        # truncate to bf16 bits
    ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float16)
    src = dev(bits, "bf16")
    dst = torch.empty(n, dtype=torch.float16, device="cuda")
    dit.convert_bf16_to_f16(src, dst)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    np.testing.assert_array_equal(got.view(np.uint16), ref.view(np.uint16))


def _f16_weights(dit, w: dict, names) -> dict:
    out = upload_stream_weights(w, "bf16")
    for k in names:
        f = torch.empty(out[k].shape, dtype=torch.float16, device="cuda")
        dit.convert_bf16_to_f16(out[k], f)
        out[k] = f
    return out


@pytest.mark.parametrize("cfg", [di.BlockConfig("ragged_bf16_d384", "bf16", d=384, n_heads=3, ffn_inner=1152, n_txt=7,
                                                grid_h=5, grid_w=9), di.CONFIGS[1], di.CONFIGS[2]],
                         ids=["ragged", "c1", "c2"])
def test_double_block_f16_weights_bit_identical(dit, cfg):
    say(f"double block {cfg.name}: fp16 product weights")
    inp = di.double_block_inputs(cfg, seed=2, qk_norm="random")
    outs = []
    for wdt in (0, dit.DIT_F16):
        sh = shape_of(cfg, dit)
        sh.gemm_w_dtype = wdt
        ws = torch.empty(dit.block_workspace_size(sh), dtype=torch.uint8, device="cuda")
        yt = torch.empty(cfg.n_txt, cfg.d, dtype=torch.float32, device="cuda")
        yi = torch.empty(cfg.n_img, cfg.d, dtype=torch.float32, device="cuda")
        names = ("w_qkv", "w_o", "w_ffn_in", "w_ffn_out") if wdt else ()
        dit.block_forward(sh, _f16_weights(dit, inp["txt"], names), _f16_weights(dit, inp["img"], names),
                          dev(inp["cond"], "bf16"), dev(inp["pos"], "i32"), dev(inp["x_txt"], "bf16"),
                          dev(inp["x_img"], "bf16"), yt, yi, ws)
        torch.cuda.synchronize()
        outs.append((host(yt), host(yi)))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])


def test_single_block_f16_weights_bit_identical(dit):
    cfg = di.BlockConfig("single_small", "bf16", d=256, n_heads=2, ffn_inner=768, n_txt=16, grid_h=8, grid_w=8)
    say("single block: fp16 product weights")
    inp = di.single_block_inputs(cfg, seed=7, qk_norm="random")
    outs = []
    for wdt in (0, dit.DIT_F16):
        sh = shape_of(cfg, dit)
        sh.gemm_w_dtype = wdt
        ws = torch.empty(dit.block_workspace_size(sh, single_stream=True), dtype=torch.uint8, device="cuda")
        y = torch.empty(cfg.n_tok, cfg.d, dtype=torch.float32, device="cuda")
        w = _f16_weights(dit, inp["w"], ("w_1", "w_2") if wdt else ())
        dit.single_block_forward(sh, w, dev(inp["cond"], "bf16"), dev(inp["pos"], "i32"), dev(inp["x"], "bf16"), y, ws)
        torch.cuda.synchronize()
        outs.append(host(y))
    np.testing.assert_array_equal(outs[0], outs[1])

"""NHWC 2-D convolution (implicit GEMM on MFMA) against the oracle's direct definition.  The bound
per element: the bf16 products are exact in fp32 and a sum of K = kh*kw*Cin of them, in any order,
is within (K - 1) 2^-24 sum|terms| of the exact value (2^-23 allowing truncating adds); the bias add
one more rounding; a bf16 output adds half a bf16 ulp."""
import numpy as np
import pytest
import torch

import dit_inputs as di
from oracle import dit_oracle as o
from gpu_util import dev, host, metric, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dit():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import attention_dit_block_amd as m
    return m


def run(dit, B, H, W, cin, cout, k, bias, ydt, seed):
    x = di.draw((B, H, W, cin), 1.0, "bf16", seed, "x")
    w = di.draw((cout, k, k, cin), 0.05, "bf16", seed, "w_1")
    b = di.draw((cout,), 1.0, "f32", seed, "cond") if bias else None
    xt = dev(x, "bf16").view(B, H, W, cin)
    wt = dev(w, "bf16").view(cout, k, k, cin)
    bt = dev(b, "f32") if bias else None
    y = torch.empty(B, H, W, cout, dtype=ydt, device="cuda")
    before = dit.launch_count()
    dit.conv2d(xt, wt, y, bias=bt)
    torch.cuda.synchronize()
    assert dit.launch_count() == before + 1
    xf, wf = o.widen(x, "bf16"), o.widen(w, "bf16")
    ref = o.conv2d_nhwc(xf, wf, b)
    abs_sum = o.conv2d_nhwc(np.abs(xf), np.abs(wf), None if b is None else np.abs(b))
    K = k * k * cin
    bound = (K * 2.0 ** -23 + 2.0 ** -22) * abs_sum + 1e-30
    if ydt == torch.bfloat16:
        bound = bound + 0.5 * 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
    got = host(y)
    err = np.abs(got - ref)
    say(f"  conv {B}x{H}x{W}x{cin} -> {cout}, {k}x{k}, bias {bias}, {ydt}: max err/bound "
        f"{np.max(err / bound):.3f}, max|gpu-oracle|/RMS {metric(got, ref):.2e}")
    assert np.all(err <= bound), f"{np.sum(err > bound)} elements beyond the bound"
    return xf, got


def test_vae_like_3x3(dit):
    # a decoder layer at 832 x 480 / 8 latent resolution, 256 channels (6240 pixels: a ragged tile)
    run(dit, 1, 60, 104, 256, 256, 3, True, torch.float32, 61)


@pytest.mark.parametrize("B, H, W, cin, cout, k, bias, ydt", [
    (2, 13, 21, 64, 72, 3, True, torch.bfloat16),      # ragged everything, bf16 output
    (1, 32, 32, 128, 64, 1, False, torch.float32),      # 1x1 (a per-pixel linear layer)
    (1, 9, 11, 64, 16, 5, True, torch.float32),         # 5x5 with borders wider than the image rows
    (3, 1, 7, 64, 8, 3, False, torch.bfloat16),         # one-row images
    (1, 11, 13, 96, 96, 3, True, torch.bfloat16),      # 96 channels: each tap's second block half zeros
    (2, 7, 9, 24, 3, 3, True, torch.float32),          # fewer channels than one block, three outputs
    (1, 6, 10, 200, 5, 1, False, torch.bfloat16),      # 200 channels (3 blocks + 8), five outputs
])
def test_shapes(dit, B, H, W, cin, cout, k, bias, ydt):
    run(dit, B, H, W, cin, cout, k, bias, ydt, 62)


def test_identity_kernel_copies_input(dit):
    B, H, W, c = 1, 10, 12, 64
    x = di.draw((B, H, W, c), 1.0, "bf16", 63, "x")
    wgt = np.zeros((c, 3, 3, c), np.float32)
    wgt[:, 1, 1, :] = np.eye(c)
    xt = dev(x, "bf16").view(B, H, W, c)
    wt = dev(di.bf16_bits_from_f32(wgt), "bf16").view(c, 3, 3, c)
    y = torch.empty(B, H, W, c, dtype=torch.bfloat16, device="cuda")
    dit.conv2d(xt, wt, y)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(y), o.widen(x, "bf16"))


# ---- causal 3-D convolution over frames (same derived bound, K = kt*kh*kw*Cin) --------------------

def run3(dit, B, T, H, W, cin, cout, kt, k, bias, ydt, seed, sample=None):
    x = di.draw((B, T, H, W, cin), 1.0, "bf16", seed, "x")
    w = di.draw((cout, kt, k, k, cin), 0.05, "bf16", seed, "w_1")
    b = di.draw((cout,), 1.0, "f32", seed, "cond") if bias else None
    xt = dev(x, "bf16").view(B, T, H, W, cin)
    wt = dev(w, "bf16").view(cout, kt, k, k, cin)
    bt = dev(b, "f32") if bias else None
    y = torch.empty(B, T, H, W, cout, dtype=ydt, device="cuda")
    before = dit.launch_count()
    dit.conv3d_causal(xt, wt, y, bias=bt)
    torch.cuda.synchronize()
    assert dit.launch_count() == before + 1
    xf, wf = o.widen(x, "bf16"), o.widen(w, "bf16")
    got = host(y)
    if sample is not None:
        # frames t-kt+1 .. t of the sampled output frames only
        t0 = max(0, sample - kt + 1)
        xs = xf[:, t0:sample + 1]
        ref = o.conv3d_causal_nhwc(xs, wf, b)[:, -1]
        abs_sum = o.conv3d_causal_nhwc(np.abs(xs), np.abs(wf), None if b is None else np.abs(b))[:, -1]
        got = got[:, sample]
    else:
        ref = o.conv3d_causal_nhwc(xf, wf, b)
        abs_sum = o.conv3d_causal_nhwc(np.abs(xf), np.abs(wf), None if b is None else np.abs(b))
    K = kt * k * k * cin
    bound = (K * 2.0 ** -23 + 2.0 ** -22) * abs_sum + 1e-30
    if ydt == torch.bfloat16:
        bound = bound + 0.5 * 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
    err = np.abs(got - ref)
    say(f"  conv3d {B}x{T}x{H}x{W}x{cin} -> {cout}, {kt}x{k}x{k}, bias {bias}, {ydt}"
        f"{'' if sample is None else f', frame {sample}'}: max err/bound {np.max(err / bound):.3f}, "
        f"max|gpu-oracle|/RMS {metric(got, ref):.2e}")
    assert np.all(err <= bound), f"{np.sum(err > bound)} elements beyond the bound"
    return got


@pytest.mark.parametrize("B, T, H, W, cin, cout, kt, k, bias, ydt", [
    (2, 3, 5, 7, 64, 40, 3, 3, True, torch.float32),     # ragged, clips of 3 frames
    (1, 5, 9, 6, 128, 72, 2, 3, False, torch.bfloat16),  # kt = 2
    (1, 2, 4, 4, 64, 16, 3, 1, True, torch.float32),     # more taps than frames: the first reach before 0
    (1, 3, 8, 12, 96, 3, 3, 3, True, torch.float32),     # the decoder head's shape: 96 -> 3, 3x3x3
    (2, 2, 5, 6, 192, 192, 3, 3, False, torch.bfloat16),  # 192 channels (the 240 x 416 stage)
    (1, 3, 6, 7, 64, 16, 3, 5, True, torch.float32),     # narrow, but its 3x20x20-pixel window exceeds
                                                         # the direct kernel's LDS: 32-wide implicit GEMM
])
def test_conv3d_causal_shapes(dit, B, T, H, W, cin, cout, kt, k, bias, ydt):
    run3(dit, B, T, H, W, cin, cout, kt, k, bias, ydt, 64)


def test_conv3d_one_frame_tap_equals_conv2d(dit):
    # kt = 1: frames are independent images -- bit-identical to dit_conv2d on the frames as a batch
    B, T, H, W, c = 2, 3, 6, 10, 64
    x = dev(di.draw((B, T, H, W, c), 1.0, "bf16", 65, "x"), "bf16").view(B, T, H, W, c)
    w = dev(di.draw((c, 1, 3, 3, c), 0.05, "bf16", 65, "w_1"), "bf16").view(c, 1, 3, 3, c)
    y3 = torch.empty(B, T, H, W, c, dtype=torch.float32, device="cuda")
    y2 = torch.empty(B * T, H, W, c, dtype=torch.float32, device="cuda")
    dit.conv3d_causal(x, w, y3)
    dit.conv2d(x.view(B * T, H, W, c), w.view(c, 3, 3, c), y2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(y3).reshape(B * T, H, W, c), host(y2))


def test_conv3d_video_vae_layer_sampled_frames(dit):
    # a video-decoder layer at a quarter of 832 x 480 (120 x 208 pixels), 256 channels, 3x3x3
    # causal taps over 5 frames; frames 0 (taps before the clip) and 4 checked in full
    for t in (0, 4):
        run3(dit, 1, 5, 120, 208, 256, 256, 3, 3, True, torch.float32, 66, sample=t)


def test_conv3d_video_vae_head_sampled_frame(dit):
    # the decoder head, 96 -> 3 channels with 3x3x3 causal taps, at half of 832 x 480 (240 x 416
    # pixels): frame 1 of a 2-frame clip (its first tap reaches before the clip)
    run3(dit, 1, 2, 240, 416, 96, 3, 3, 3, True, torch.bfloat16, 67, sample=1)

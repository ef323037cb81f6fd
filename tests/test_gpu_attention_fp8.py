"""fp8 (e4m3) joint attention on the GPU against the oracle.

The kernel computes the scores from the e4m3 codes exactly up to fp32 accumulation, and its
softmax in fp32; its one deliberate approximation is that the probabilities enter the PV product
rounded to e4m3.  Relative to the row max, each probability w_j in (0, 1] then moves by at most
max(2^-4 w_j, 2^-10) (half a step of e4m3, normal or subnormal: the kernel rounds them relative to a
running max that is never above the row max, which only makes its steps finer), while the normaliser
stays the fp32 sum of the unrounded ones.  So, per output element,

    |O_gpu - O| <= sum_j max(2^-4 w_j, 2^-10) |V_j| / sum_j w_j  +  fp32 terms  +  output rounding,

with O the oracle's exact fp8 attention (``joint_attention_fp8``) and the fp32 terms bounded by
1e-4 sum_j w_j |V_j| / sum_j w_j (score accumulation and the per-query scale product, through
exp2, for scaled scores within +-40; sums over a few thousand keys).  That bound is element-wise
and worst-case; a second, statistical check holds the RMS error to at most 1.5x that of the
oracle's own model of the rounding (``round_p=True``, rounding relative to a max that lags the row
max by a random 0 .. 8 in log2 units, as the kernel's lazy running max does), which a dropped or
misplaced key tile, a wrong scale or a key permutation between P and V would exceed by orders of
magnitude.
"""
import numpy as np
import pytest
import torch

import dit_inputs as di
from oracle import dit_oracle as o
from gpu_util import host, say, tdtype, ulp

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module")
def dit():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import attention_dit_block_amd as m
    return m


def _to_gpu(x):
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in x.items()}
    return t


def _run(dit, x, n, H, out_dtype="f32", scale=None):
    t = _to_gpu(x)
    o_ = torch.full((n, H * D), float("nan"), dtype=tdtype(out_dtype), device="cuda")
    dit.joint_attention_fp8(t["q8"], t["sq"], t["k8"], t["sk"], t["v8"], t["sv"], o_, H, softmax_scale=scale)
    torch.cuda.synchronize()
    return host(o_)


def _bound(x, H, rows, scale=None):
    """Per-element worst-case bound (see the module docstring) for query rows `rows`."""
    if scale is None:
        scale = D ** -0.5
    q = o.e4m3_decode(x["q8"][rows]) * np.repeat(x["sq"][rows].astype(np.float64), D, axis=1)
    k = o.e4m3_decode(x["k8"]) * np.repeat(x["sk"].astype(np.float64), D)[None, :]
    v = o.e4m3_decode(x["v8"]) * np.repeat(x["sv"].astype(np.float64), D)[None, :]
    out = np.empty((len(rows), H * D))
    for h in range(H):
        c = slice(h * D, (h + 1) * D)
        s = q[:, c] @ k[:, c].T * scale
        w = np.exp(s - s.max(axis=1, keepdims=True))
        l = w.sum(axis=1, keepdims=True)
        av = np.abs(v[:, c])
        out[:, c] = (np.maximum(2.0 ** -4 * w, 2.0 ** -10) @ av + 1e-4 * (w @ av)) / l
    return out


def _check(got, x, H, rows, out_dtype, scale=None):
    exact = o.joint_attention_fp8(x["q8"], x["sq"], x["k8"], x["sk"], x["v8"], x["sv"], H, D, scale=scale,
                                  q_rows=rows)
    # the rounding model with the lag of the kernel's running max drawn per row (0 .. 8 in log2)
    lag = np.random.default_rng(len(rows)).uniform(0.0, 8.0, (len(rows), H))
    model = o.joint_attention_fp8(x["q8"], x["sq"], x["k8"], x["sk"], x["v8"], x["sv"], H, D, scale=scale,
                                  q_rows=rows, round_p=True, p_shift=lag)
    g = got[rows]
    assert np.all(np.isfinite(g))
    err = np.abs(g - exact)
    # plus the fp32 rounding of the final scaling (a few ulp of the result) and the storage rounding
    bound = (_bound(x, H, rows, scale) + 2.0 ** -21 * np.abs(exact) + 1e-30 +
             (ulp(exact, out_dtype) if out_dtype != "f32" else 0.0))
    worst = float(np.max(err / bound))
    rms_gpu = float(np.sqrt(np.mean((g - exact) ** 2)))
    rms_model = float(np.sqrt(np.mean((model - exact) ** 2)))
    rms_out = float(np.sqrt(np.mean(exact ** 2)))
    say(f"  max err/bound {worst:.3f}  rms err {rms_gpu:.3e} (model {rms_model:.3e}, output rms {rms_out:.3e})")
    assert worst <= 1.0
    assert rms_gpu <= 1.5 * rms_model + 1e-7 * rms_out


@pytest.mark.parametrize("n, H, out_dtype", [(1, 1, "f32"), (63, 2, "f32"), (64, 1, "bf16"), (300, 3, "f32"),
                                             (513, 2, "f16"), (1000, 2, "bf16")])
def test_fp8_attention_small(dit, n, H, out_dtype):
    say(f"fp8 attention n={n} H={H} out={out_dtype}")
    x = di.fp8_attention_inputs(n, H, seed=n)
    got = _run(dit, x, n, H, out_dtype)
    _check(got, x, H, np.arange(n), out_dtype)


def test_fp8_attention_negative_scale_and_strides(dit):
    # a negative softmax scale (the row max of the scaled scores is then the min of the raw ones)
    # and padded byte strides
    n, H = 200, 2
    say("fp8 attention: negative scale, strided operands")
    x = di.fp8_attention_inputs(n, H, seed=5)
    t = _to_gpu(x)
    pad = lambda a: torch.cat([a, torch.zeros(n, 48, dtype=a.dtype, device="cuda")], dim=1)[:, :H * D]
    q8, k8, v8 = pad(t["q8"]), pad(t["k8"]), pad(t["v8"])
    assert q8.stride(0) == H * D + 48
    o_ = torch.empty(n, H * D + 8, dtype=torch.float32, device="cuda")[:, :H * D]
    dit.joint_attention_fp8(q8, t["sq"], k8, t["sk"], v8, t["sv"], o_, H, softmax_scale=-0.07)
    torch.cuda.synchronize()
    _check(host(o_), x, H, np.arange(n), "f32", scale=-0.07)


def test_fp8_attention_equal_keys_give_mean_of_v(dit):
    # every key the same: each probability is exactly 1 up to the exp2 of a rounding residue, so
    # the output is the mean of V to fp32 accuracy, whatever the query
    n, H = 777, 2
    say("fp8 attention: equal keys")
    x = di.fp8_attention_inputs(n, H, seed=9)
    x["k8"] = np.repeat(x["k8"][:1], n, axis=0)
    got = _run(dit, x, n, H)
    v = o.e4m3_decode(x["v8"]) * np.repeat(x["sv"].astype(np.float64), D)[None, :]
    np.testing.assert_allclose(got, np.broadcast_to(v.mean(axis=0), got.shape), rtol=1e-5, atol=1e-6)


def test_fp8_attention_full_size_sampled_rows(dit):
    # the benchmarked shape: 512 text + 4096 image tokens, 24 heads; sampled query rows
    n, H = 4608, 24
    say(f"fp8 attention n={n} H={H}: sampled rows")
    x = di.fp8_attention_inputs(n, H, seed=24)
    got = _run(dit, x, n, H, "bf16")
    rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(505, 520), np.arange(2300, 2310),
                                     np.arange(n - 12, n), np.random.default_rng(0).integers(0, n, 20)]))
    _check(got, x, H, rows, "bf16")


def test_fp8_attention_16896_tokens_sampled_rows(dit):
    # 512 text + 16384 image tokens (the largest single-GPU block workload), sampled query rows
    n, H = 16896, 24
    say(f"fp8 attention n={n} H={H}: sampled rows")
    x = di.fp8_attention_inputs(n, H, seed=31)
    got = _run(dit, x, n, H, "f16")
    rows = np.unique(np.concatenate([[0, 511, 512, n - 1], np.random.default_rng(1).integers(0, n, 28)]))
    _check(got, x, H, rows, "f16")


def test_fp8_attention_rejects_bad_arguments(dit):
    n, H = 64, 1
    x = _to_gpu(di.fp8_attention_inputs(n, H, seed=1))
    o_ = torch.empty(n, H * D, dtype=torch.float32, device="cuda")
    with pytest.raises(Exception):
        dit.joint_attention_fp8(x["q8"], x["sq"], x["k8"], x["sk"], x["v8"], x["sv"], o_, H, head_dim=64)
    buf = torch.zeros(n, 4 * H * D, dtype=torch.uint8, device="cuda")
    buf[:, :H * D] = x["q8"]
    with pytest.raises(Exception, match="overlaps"):      # o (fp32) over the bytes of q
        dit.joint_attention_fp8(buf[:, :H * D], x["sq"], x["k8"], x["sk"], x["v8"], x["sv"], buf.view(torch.float32),
                                H)
    # zero tokens: nothing is read or written
    e = torch.empty(0, H * D, dtype=torch.uint8, device="cuda")
    dit.joint_attention_fp8(e, x["sq"][:0], e, x["sk"], e, x["sv"], o_[:0], H)

"""fp8 (OCP e4m3) quantisation and GEMM on the GPU against the oracle.  Quantised codes and scales
must match bit for bit (the kernel's float32 decisions, taken the same way by the oracle); the
GEMM on given codes must match the exact product within the bound of fp32 accumulation of exact
e4m3 products (its own tolerance, derived per element below); the distance of the fp8 product
from the unquantised one is reported, not held to a bar."""
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


@pytest.mark.parametrize("dtype, rows, cols", [("bf16", 64, 3072), ("f16", 37, 200), ("f32", 10, 9216),
                                               # rows kept in registers: the FFN-down input, the single
                                               # block's linear2 input (d + F), one-chunk rows
                                               ("f16", 20, 9216), ("bf16", 9, 12288), ("f16", 3, 8),
                                               # longer 16-bit rows and ragged fp32 rows: two passes
                                               ("bf16", 7, 13320), ("f32", 7, 1000)])
def test_quantize_matches_oracle_bit_for_bit(dit, dtype, rows, cols):
    x = di.draw((rows, cols), 1.0, dtype, 51, "x")
    xf = o.widen(x, dtype).astype(np.float32)
    # rows of very different magnitude, a zero row, one huge element
    if dtype != "f16":
        xs = xf * np.float32(2.0) ** np.arange(-6, rows - 6, dtype=np.float32)[:, None].clip(-6, 6)
        xs[3] = 0.0
        xs[4, 7] = np.float32(3.0e4)
        x = di.bf16_bits_from_f32(xs) if dtype == "bf16" else xs
        xf = o.widen(x, dtype).astype(np.float32)
    t = dev(x, dtype).view(rows, cols)
    ldq = (cols + 15) // 16 * 16          # byte rows padded to 16 (a strided view when cols is not)
    q = torch.empty(rows, ldq, dtype=torch.uint8, device="cuda")[:, :cols]
    s = torch.empty(rows, dtype=torch.float32, device="cuda")
    dit.quantize_fp8(t, q, s)
    torch.cuda.synchronize()
    wq, ws = o.quantize_fp8_rows(xf)
    np.testing.assert_array_equal(host(s).astype(np.float32), ws)
    got = q.cpu().numpy()
    bad = got != wq
    if bad.any():
        for r, c in np.argwhere(bad)[:8]:
            y = np.float32(xf[r, c]) / ws[r]
            say(f"  row {r} col {c}: x {xf[r, c]!r} x/s {y!r} gpu {got[r, c]:#04x} ({o.e4m3_decode(got[r, c])}) "
                f"oracle {wq[r, c]:#04x} ({o.e4m3_decode(wq[r, c])})")
    assert not bad.any(), f"{bad.sum()} codes differ, first at {np.argwhere(bad)[0]}"


@pytest.mark.parametrize("case", ["ffn_in_sampled", "ragged", "bf16_out"])
def test_linear_fp8(dit, case):
    if case == "ffn_in_sampled":
        m, n, k = 4608, 18432, 3072           # the block's FFN-in product (both halves)
        ydt = torch.float32
    elif case == "ragged":
        m, n, k = 300, 72, 256
        ydt = torch.float32
    else:
        m, n, k = 513, 256, 384
        ydt = torch.bfloat16
    x = o.widen(di.draw((m, k), 1.0, "bf16", 52, "x"), "bf16").astype(np.float32)
    w = o.widen(di.draw((n, k), 0.02, "bf16", 52, "w_1"), "bf16").astype(np.float32)
    xq, sx = o.quantize_fp8_rows(x)
    wq, sw = o.quantize_fp8_rows(w)
    y = torch.empty(m, n, dtype=ydt, device="cuda")
    dit.linear_fp8(torch.from_numpy(xq).cuda(), torch.from_numpy(sx).cuda(), torch.from_numpy(wq).cuda(),
                   torch.from_numpy(sw).cuda(), y)
    torch.cuda.synchronize()
    rows = None if m * n <= 1 << 22 else np.unique(np.concatenate([[0, m - 1], np.random.default_rng(3).choice(m, 200, replace=False)]))
    r = slice(None) if rows is None else rows
    ref = o.linear_fp8(xq[r], sx[r], wq, sw)
    got = host(y)[r]
    # Bound per element: the e4m3 products are exact in fp32; a sum of k of them in any order is
    # within (k - 1) 2^-24 sum|terms| of the exact sum (2^-23 allowing truncating adds), the two
    # scale products add 2^-24 each, and a bf16 output half a bf16 ulp.
    abs_sum = o.linear_fp8(xq[r] & 0x7F, sx[r], wq & 0x7F, sw)
    bound = (k * 2.0 ** -23 + 2.0 ** -22) * abs_sum + 1e-30
    if ydt == torch.bfloat16:
        bound = bound + 0.5 * 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
    err = np.abs(got - ref)
    exact = o.linear(x[r], w)
    say(f"  fp8 linear {case} [{m}x{k}] x [{n}x{k}]^T: max err/bound {np.max(err / bound):.3f}, "
        f"max|gpu - e4m3 product|/RMS {metric(got, ref):.2e}; fp8 product vs unquantised {metric(ref, exact):.2e}")
    assert np.all(err <= bound), f"{np.sum(err > bound)} elements beyond the bound"

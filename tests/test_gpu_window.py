"""Windowed (neighborhood) attention on the GPU against the fp64 oracle, with the per-element
bound of the joint-attention tests: the exact output rounded once to the storage type, plus the
probabilities' rounding (fp16 2^-11, bf16 two-term 2^-16) times the attention of |v|.  fp32:
max|gpu - oracle| / RMS <= 1e-4."""
import numpy as np
import pytest
import torch

import dit_inputs as di
from oracle import dit_oracle as o
from gpu_util import dev, host, metric, say, tdtype
from test_gpu_kernels import check, check_attention

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dit():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import attention_dit_block_amd as m
    return m


def _rows(grid, k, seed):
    """All rows for small grids; else the corners of every frame, the first and last rows and
    columns, and k random rows."""
    T, H, W = grid
    n = T * H * W
    if n <= 4096:
        return None
    rng = np.random.default_rng(seed)
    edge = []
    for t in (0, T // 2, T - 1):
        for h in (0, 1, H // 2, H - 2, H - 1):
            for w in (0, 1, W // 2, W - 2, W - 1):
                edge.append((t * H + h) * W + w)
    return np.unique(np.concatenate([edge, rng.choice(n, k, replace=False)]))


def run_case(dit, dtype, grid, kernel, heads, seed, strided=False):
    T, H, W = grid
    n, d = T * H * W, 128 * heads
    say(f"window attention {dtype} grid {grid} kernel {kernel} heads {heads}")
    qkv = di.draw((n, 3 * d), 1.0, dtype, seed, "q")
    t = dev(qkv, dtype)
    if strided:
        q, k, v = t[:, :d], t[:, d:2 * d], t[:, 2 * d:]
    else:
        q, k, v = (t[:, i * d:(i + 1) * d].contiguous() for i in range(3))
    out = torch.empty(n, d, dtype=tdtype(dtype), device="cuda")
    before = dit.launch_count()
    dit.neighborhood_attention(q, k, v, out, grid, kernel, heads)
    torch.cuda.synchronize()
    assert dit.launch_count() == before + 1
    x = o.widen(qkv, dtype)
    rows = _rows(grid, 300, seed)
    ref = o.neighborhood_attention(x[:, :d], x[:, d:2 * d], x[:, 2 * d:], grid, kernel, heads, 128, q_rows=rows)
    got = host(out) if rows is None else host(out)[rows]
    if dtype == "f32":
        check(got, ref, dtype, what="O")
    else:
        ref_abs = o.neighborhood_attention(x[:, :d], x[:, d:2 * d], np.abs(x[:, 2 * d:]), grid, kernel, heads, 128,
                                           q_rows=rows)
        check_attention(got, ref, ref_abs, dtype)
    return x, host(out)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_page_shape_9x64x64_window_11(dit, dtype):
    # the page's repro shape: a 9-frame grid of 64 x 64 with an [11, 11, 11] window (T clamps to 9)
    run_case(dit, dtype, (9, 64, 64), (11, 11, 11), 2, 41)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_page_edge_case_every_axis_clamps(dit, dtype):
    # grid [1, 4, 4], kernel [3, 7, 7]: every axis narrower than the window -> full attention
    x, got = run_case(dit, dtype, (1, 4, 4), (3, 7, 7), 2, 42)
    d = 256
    full = o.joint_attention(x[:, :d], x[:, d:2 * d], x[:, 2 * d:], 2, 128)
    if dtype == "f32":
        check(got, full, dtype, what="O vs full attention")
    else:
        ref_abs = o.joint_attention(x[:, :d], x[:, d:2 * d], np.abs(x[:, 2 * d:]), 2, 128)
        check_attention(got, full, ref_abs, dtype, what="O vs full attention")


@pytest.mark.parametrize("dtype, grid, kernel", [
    ("f16", (2, 13, 21), (3, 5, 7)),          # ragged patches at both edges
    ("bf16", (3, 17, 16), (5, 9, 1)),          # one column per window
    ("bf16", (1, 20, 70), (1, 3, 41)),         # wide window: 64-key box rows
    ("f16", (4, 6, 5), (9, 3, 3)),             # T narrower than the window
])
def test_ragged_and_wide_windows(dit, dtype, grid, kernel):
    run_case(dit, dtype, grid, kernel, 3, 43, strided=True)


def test_fp32(dit):
    run_case(dit, "f32", (2, 9, 10), (3, 3, 5), 2, 44)


def test_single_key_window_copies_v(dit):
    grid = (2, 5, 7)
    n, d = 70, 128
    qkv = di.draw((n, 3 * d), 1.0, "bf16", 45, "q")
    t = dev(qkv, "bf16")
    out = torch.empty(n, d, dtype=torch.bfloat16, device="cuda")
    dit.neighborhood_attention(t[:, :d], t[:, d:2 * d], t[:, 2 * d:], out, grid, (1, 1, 1), 1)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out), o.widen(qkv, "bf16")[:, 2 * d:])

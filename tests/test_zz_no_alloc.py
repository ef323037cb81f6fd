"""The allocation-free timestep embedding (dit_timestep_embedding_noalloc, scratch in the
library's static per-GPU array) against the workspace entry point dit_timestep_embedding (GPU).

Both run the same kernels on the same inputs, so the conditioning vectors must be bit-identical;
two calls in a row, the second with a smaller problem, show that the shared scratch left by one
call does not leak into the next.  Also checked against the fp64 oracle within the bf16 bar."""
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


def _weights(cfg, seed):
    e = di.edge_inputs(cfg, seed=seed)
    t = cfg.dtype
    return e, {k: dev(e[k], t).view(e[k].shape[0], -1) for k in ("w_t_in", "w_t_out", "w_g_in", "w_g_out")}


def test_noalloc_matches_workspace_entry_point(dit):
    big = di.CONFIGS[2]                      # d = 3072 (bf16), freq_dim 256
    small = di.BlockConfig("temb_small", "bf16", d=384, n_heads=3, ffn_inner=1152, n_txt=7, grid_h=5, grid_w=9)
    tt = torch.tensor([0.731], dtype=torch.float32, device="cuda")
    gt = torch.tensor([0.35], dtype=torch.float32, device="cuda")
    for i, (cfg, guided) in enumerate(((big, True), (small, False))):
        say(f"call {i + 1}: d = {cfg.d}, guidance {guided}")
        e, w = _weights(cfg, seed=3 + i)
        d = cfg.d
        kw = dict(g=gt, w_g_in=w["w_g_in"], w_g_out=w["w_g_out"]) if guided else {}
        ws = torch.empty(dit.timestep_embedding_workspace_size(256, d), dtype=torch.uint8, device="cuda")
        ref_c = torch.empty(d, dtype=torch.bfloat16, device="cuda")
        dit.timestep_embedding(tt, w["w_t_in"], w["w_t_out"], ref_c, ws, **kw)
        got = torch.full((d,), float("nan"), dtype=torch.bfloat16, device="cuda")
        before = dit.launch_count()
        dit.timestep_embedding_noalloc(tt, w["w_t_in"], w["w_t_out"], got, **kw)
        torch.cuda.synchronize()
        assert dit.launch_count() == before + (7 if guided else 4), "the HIP path did not run"
        np.testing.assert_array_equal(got.view(torch.int16).cpu().numpy(), ref_c.view(torch.int16).cpu().numpy())
        wid = lambda k: o.widen(e[k], "bf16")
        ref = o.conditioning_vector(0.731, wid("w_t_in"), wid("w_t_out"), 256, g=0.35 if guided else None,
                                    w_g_in=wid("w_g_in"), w_g_out=wid("w_g_out"))
        m = metric(host(got), ref)
        say(f"  max|gpu-oracle|/RMS = {m:.3e}")
        assert m <= 2e-2


def test_noalloc_rejects_sizes_beyond_the_static_scratch(dit):
    d = 8192                                 # 256 + 2 x 8192 fp32 values: more than 64 KiB
    w_in = torch.zeros(d, 256, dtype=torch.bfloat16, device="cuda")
    w_out = torch.zeros(d, d, dtype=torch.bfloat16, device="cuda")
    cond = torch.empty(d, dtype=torch.bfloat16, device="cuda")
    tt = torch.tensor([0.5], dtype=torch.float32, device="cuda")
    before = dit.launch_count()
    with pytest.raises(dit.DitError) as ex:
        dit.timestep_embedding_noalloc(tt, w_in, w_out, cond)
    assert ex.value.status == "DIT_ERR_UNSUPPORTED" and "static scratch" in str(ex.value)
    assert dit.launch_count() == before

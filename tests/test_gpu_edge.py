"""Parity of the layers either side of the block stack (timestep embedding, linear / patch
embedding, final layer) and of the shared-modulation step, against the fp64 oracle (GPU).

Bars as for the block: max|gpu - oracle| / RMS(oracle) <= 2e-2 on the bf16 workloads and
<= 1e-4 on fp32 ones."""
import numpy as np
import pytest
import torch

import dit_inputs as di
from oracle import dit_oracle as o
from gpu_util import dev, host, metric, say, shape_of, upload_stream_weights

pytestmark = pytest.mark.gpu

BAR = {"bf16": 2e-2, "f32": 1e-4}


@pytest.fixture(scope="module")
def dit():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import attention_dit_block_amd as m
    return m


def report(name, gpu, ref, bar):
    m = metric(gpu, ref)
    say(f"  {name}: max|gpu-oracle|/RMS = {m:.3e} (bar {bar:g})")
    assert m <= bar, f"{name}: {m:.3e} > {bar}"


SMALL_F32 = di.BlockConfig("edge_f32", "f32", d=256, n_heads=2, ffn_inner=768, n_txt=8, grid_h=8, grid_w=8)
SMALL_BF16 = di.BlockConfig("edge_bf16", "bf16", d=384, n_heads=3, ffn_inner=1152, n_txt=7, grid_h=5, grid_w=9)


@pytest.mark.parametrize("cfg", [di.CONFIGS[2], SMALL_F32], ids=lambda c: c.name)
def test_timestep_embedding(dit, cfg):
    t = cfg.dtype
    e = di.edge_inputs(cfg, seed=3)
    d = cfg.d
    ws = torch.empty(dit.timestep_embedding_workspace_size(256, d), dtype=torch.uint8, device="cuda")
    cond = torch.empty(d, dtype=torch.bfloat16 if t == "bf16" else torch.float32, device="cuda")
    w = {k: dev(e[k], t).view(e[k].shape[0], -1) for k in ("w_t_in", "w_t_out", "w_g_in", "w_g_out")}
    tv, gv = np.float32(0.731), np.float32(0.35)
    tt = torch.tensor([tv], dtype=torch.float32, device="cuda")
    gt = torch.tensor([gv], dtype=torch.float32, device="cuda")
    wid = lambda k: o.widen(e[k], t)
    for guided in (False, True):
        before = dit.launch_count()
        if guided:
            dit.timestep_embedding(tt, w["w_t_in"], w["w_t_out"], cond, ws, g=gt, w_g_in=w["w_g_in"],
                                   w_g_out=w["w_g_out"])
        else:
            dit.timestep_embedding(tt, w["w_t_in"], w["w_t_out"], cond, ws)
        torch.cuda.synchronize()
        assert dit.launch_count() == before + (7 if guided else 4)
        ref = o.conditioning_vector(float(tv), wid("w_t_in"), wid("w_t_out"), 256,
                                    g=float(gv) if guided else None, w_g_in=wid("w_g_in"), w_g_out=wid("w_g_out"))
        report(f"{cfg.name} cond (guidance {guided})", host(cond), ref, BAR[t])


def test_timestep_embedding_graph_replay_reads_t(dit):
    """t lives on the device: a captured graph replayed after t changes embeds the new value."""
    cfg = SMALL_BF16
    e = di.edge_inputs(cfg, seed=4)
    d = cfg.d
    ws = torch.empty(dit.timestep_embedding_workspace_size(256, d), dtype=torch.uint8, device="cuda")
    cond = torch.empty(d, dtype=torch.bfloat16, device="cuda")
    wi, wo = dev(e["w_t_in"], "bf16").view(d, 256), dev(e["w_t_out"], "bf16").view(d, d)
    tt = torch.tensor([0.9], dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dit.timestep_embedding(tt, wi, wo, cond, ws, stream=s)     # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dit.timestep_embedding(tt, wi, wo, cond, ws, stream=s)
    for tv in (0.25, 0.6, 0.05):
        tt.fill_(tv)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = o.conditioning_vector(float(np.float32(tv)), o.widen(e["w_t_in"], "bf16"),
                                    o.widen(e["w_t_out"], "bf16"), 256)
        report(f"graph replay t={tv}", host(cond), ref, BAR["bf16"])


@pytest.mark.parametrize("case", ["patch_c2", "ragged_f16", "bf16_out", "f32"])
def test_linear(dit, case):
    rng_seed = {"patch_c2": 5, "ragged_f16": 6, "bf16_out": 7, "f32": 8}[case]
    if case == "patch_c2":
        cfg = di.CONFIGS[2]
        e = di.edge_inputs(cfg, seed=rng_seed)
        x_np, w_np, t, xdt = e["latent"], e["w_patch"], "bf16", "bf16"
        m, k, n = cfg.n_img, 64, cfg.d
        ydt = torch.float32
    elif case == "ragged_f16":
        m, n, k = 77, 72, 128
        x_np = di.draw((m, k), 1.0, "f16", rng_seed, "latent")
        w_np = di.draw((n, k), 0.02, "bf16", rng_seed, "w_patch")
        t, xdt, ydt = "bf16", "f16", torch.float32
    elif case == "bf16_out":
        m, n, k = 300, 256, 192
        x_np = di.draw((m, k), 1.0, "bf16", rng_seed, "latent")
        w_np = di.draw((n, k), 0.02, "bf16", rng_seed, "w_patch")
        t, xdt, ydt = "bf16", "bf16", torch.bfloat16
    else:
        m, n, k = 50, 40, 48
        x_np = di.draw((m, k), 1.0, "f32", rng_seed, "latent")
        w_np = di.draw((n, k), 0.02, "f32", rng_seed, "w_patch")
        t, xdt, ydt = "f32", "f32", torch.float32
    x = dev(x_np, xdt).view(m, k)
    w = dev(w_np, t).view(n, k)
    y = torch.empty(m, n, dtype=ydt, device="cuda")
    dit.linear(x, w, y)
    torch.cuda.synchronize()
    ref = o.linear(o.widen(x_np, xdt), o.widen(w_np, t))
    report(f"linear {case} [{m}x{k}] x [{n}x{k}]^T", host(y), ref, BAR[t])


@pytest.mark.parametrize("cfg", [di.CONFIGS[2], SMALL_F32], ids=lambda c: c.name)
def test_final_layer(dit, cfg):
    t = cfg.dtype
    e = di.edge_inputs(cfg, seed=9)
    d, n = cfg.d, cfg.n_img
    x_np = di.draw((n, d), 1.0, "f32", 9, "x_img")
    x = dev(x_np, "f32").view(n, d)
    act = dit.DIT_F16 if t == "bf16" else dit.DIT_F32
    ws = torch.empty(dit.final_layer_workspace_size(n, d, act), dtype=torch.uint8, device="cuda")
    y = torch.empty(n, 64, dtype=torch.float32, device="cuda")
    cond = dev(e["cond"], t)
    wm = dev(e["w_final_mod"], t).view(2 * d, cfg.dc)
    wo = dev(e["w_final_out"], t).view(64, d)
    before = dit.launch_count()
    dit.final_layer(x, cond, wm, wo, y, ws, act_dtype=act)
    torch.cuda.synchronize()
    assert dit.launch_count() == before + 3
    ref = o.final_layer(x_np.astype(np.float64), o.widen(e["cond"], t), o.widen(e["w_final_mod"], t),
                        o.widen(e["w_final_out"], t))
    report(f"{cfg.name} final layer [{n}x{d}] -> [{n}x64]", host(y), ref, BAR[t])


def test_step_shared_mod(dit):
    """Shared modulation: equal to dit_step_forward when every block carries the shared w_mod
    (bit for bit), one GEMV launch per block kind, and the oracle chain with the shared AdaLN
    vectors within the block bar."""
    from test_gpu_block import _step_weights
    cfg = SMALL_BF16
    nd, ns = 2, 2
    say(f"shared-modulation step {nd} double + {ns} single, {cfg.name}")
    dbl, sgl, (wt, wi, ws_) = _step_weights(cfg, nd, ns, seed=31)
    shared = di.shared_mod_weights(cfg, seed=31)
    t = cfg.dtype
    mt, mi, msg = (dev(shared[k], t) for k in ("txt", "img", "single"))
    act = dbl[0]
    cond, pos = dev(act["cond"], t), dev(act["pos"], "i32")
    xt, xi = dev(act["x_txt"], t), dev(act["x_img"], t)
    sh = shape_of(cfg, dit)
    ws = torch.empty(dit.step_shared_mod_workspace_size(sh, nd, ns), dtype=torch.uint8, device="cuda")
    y = torch.empty(cfg.n_tok, cfg.d, dtype=torch.float32, device="cuda")
    no_mod = lambda ws_list: [{k: v for k, v in w.items() if k != "w_mod"} for w in ws_list]
    before = dit.launch_count()
    dit.step_forward_shared_mod(sh, no_mod(wt), no_mod(wi), no_mod(ws_), mt, mi, msg, cond, pos, xt, xi, y, ws)
    torch.cuda.synchronize()
    assert dit.launch_count() == before + 8 * nd + 5 * ns + 2
    # the plain step with every block's w_mod set to the shared matrices
    z = torch.empty_like(y)
    wt2 = [dict(w, w_mod=mt) for w in wt]
    wi2 = [dict(w, w_mod=mi) for w in wi]
    ws2 = [dict(w, w_mod=msg) for w in ws_]
    wsp = torch.empty(dit.step_workspace_size(sh, nd, ns), dtype=torch.uint8, device="cuda")
    dit.step_forward(sh, wt2, wi2, ws2, cond, pos, xt, xi, z, wsp)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(y), host(z))
    # oracle chain with the shared AdaLN vectors
    c = o.widen(act["cond"], t)
    m_d = {s: o.adaln_modulation(o.widen(shared[s], t), c).reshape(6, cfg.d) for s in ("txt", "img")}
    m_s = o.adaln_modulation(o.widen(shared["single"], t), c).reshape(3, cfg.d)
    st = None
    for b in range(nd):
        inp = dict(dbl[b])
        if st is not None:
            inp.update(x_txt=st[:cfg.n_txt], x_img=st[cfg.n_txt:], x_dtype="f64")
        r = o.double_block(cfg, inp, mods=m_d)
        st = np.concatenate([r["y_txt"], r["y_img"]])
    for b in range(ns):
        st = o.single_block(cfg, {"cond": act["cond"], "pos": act["pos"], "w": sgl[b], "x": st, "x_dtype": "f64"},
                            mods=m_s)["y"]
    report(f"{cfg.name} shared-modulation stack output", host(y), st, BAR[t])

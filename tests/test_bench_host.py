"""Host-side checks of bench.py: the algorithmic work model behind its TFLOP/s and
roofline figures, and the refusal of more than one GPU.  No GPU is touched."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import dit_inputs as di  # noqa: E402


def _closed_form_flops(cfg):
    # Per block, with the SwiGLU inner width F = 3d: the double-stream block's QKV (3d), output
    # projection (d), FFN-in (2F) and FFN-down products, or the single-stream block's fused
    # linear1 (3d + 2F) and linear2 (d + F) products, both come to 26 N d^2 multiply-add pairs
    # counted as 2 flop; attention's QK^T and PV add 2 N^2 d each.
    n, d = cfg.n_tok, cfg.d
    return (cfg.n_double + cfg.n_single) * (26.0 * n * d * d + 4.0 * n * n * d)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_step_flops_match_closed_form(name):
    cfg = di.config_by_name(name)
    assert cfg.ffn_inner == 3 * cfg.d
    work = bench.step_work(cfg)
    total = sum(f for f, _, _, _ in work.values())
    assert total == pytest.approx(_closed_form_flops(cfg), rel=1e-12)


def test_step_launch_counts_and_bounds():
    cfg = di.config_by_name("c3")          # 5 double-stream then 20 single-stream blocks
    work = bench.step_work(cfg)
    blocks = cfg.n_double + cfg.n_single
    for name in ("modulate_x", "joint_attention", "adaln_gemv"):
        assert work[name][3] == blocks
    # double blocks: QK RMSNorm + RoPE in the QKV product's epilogue (the angle table comes with the
    # modulation), single blocks: the separate pass
    assert work["qk_rmsnorm_rope"][3] == cfg.n_single
    for name in ("gemm_qkv", "gemm_out_proj", "modulate_h", "gemm_ffn_in_swiglu", "gemm_ffn_down"):
        assert work[name][3] == cfg.n_double
    for name in ("gemm_linear1", "gemm_linear2"):
        assert work[name][3] == cfg.n_single
    assert bench.step_work(cfg, shared_mod=True)["adaln_gemv"][3] == 2
    for name, (f, b, bound, _) in work.items():
        assert (bound == "hbm") == (f == 0.0 and b > 0.0), name


def test_adaln_gemv_bytes_are_the_weight_matrix():
    # The GEMV streams its weight matrix once: 12 d x d_c entries for the double-stream block
    # (six modulation vectors per stream), 3 d x d_c for the single-stream block.
    cfg = di.config_by_name("c2")
    f, b, bound = bench.kernel_work(cfg, "adaln_gemv")
    assert f is None and bound == "hbm"
    assert b == 12 * cfg.d * cfg.dc * 2
    assert bench.kernel_work(cfg, "no_such_kernel") == (None, None, "?")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _fake_counter_csv(path, counter, rows):
    import csv
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for d, name, v in rows:
            # two instances per dispatch: the reader sums them
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v / 2})
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v / 2})
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": "OTHER", "Counter_Value": 1e9})


def test_counter_bytes_per_launch_site(tmp_path):
    # a counter pass: a fill, 3 calibration copies (counted at half their bytes), setup conversions,
    # then 3 steps of 3 library launches; the bytes of launch site i come from its dispatches in the
    # last two steps, scaled by the copies
    kib = bench.CALIB_BYTES / 1024
    rows = [(1, "at::fill", kib), (2, "at::copy", kib / 2), (3, "at::copy", kib / 2), (4, "at::copy", kib / 2),
            (5, "dit::bf16_to_f16_kernel(unsigned short const*, unsigned short*, unsigned long)", 7.0)]
    sites = ["void dit::gemv()", "void dit::gemm<0>()", "void dit::attn()"]
    d = 6
    for stepi in range(3):
        for i, name in enumerate(sites):
            rows.append((d, name, 100.0 * (i + 1) + (50.0 if stepi == 0 else 0.0)))   # the first step is cold
            d += 1
    p = tmp_path / "c_counter_collection.csv"
    _fake_counter_csv(p, "FETCH_SIZE", rows)
    parsed = bench._read_counter_csv(str(p), "FETCH_SIZE")
    assert [r[0] for r in parsed] == list(range(1, d)) and parsed[5][2] == 150.0
    c = bench.counters_from_csv(str(p), "FETCH_SIZE")
    # the median of the three largest dispatches before the library's: a copy (the fill, counted
    # differently here, is outvoted)
    assert c["scale"] == 2.0
    assert c["symbols"] == sites * 3 and c["values"][1] == 250.0 * 1024 * 2.0 and c["values"][4] == 200.0 * 1024 * 2.0
    counters = {"FETCH_SIZE": c}
    order = ["adaln_gemv", "gemm_qkv", "joint_attention"]
    tr = bench.traffic_of(counters, order, "gemm_qkv")
    assert tr["bytes"] == int(200.0 * 1024 * 2.0) and tr["fetch_size_scale"] == 2.0
    assert bench.traffic_of(counters, order, "joint_attention")["bytes"] == int(300.0 * 1024 * 2.0)
    # a step whose launches do not line up with the site order gives no figure
    assert bench.traffic_of(counters, order + ["modulate_h"], "gemm_qkv") is None
    assert bench.traffic_of(counters, order, "not_a_site") is None
    assert bench.traffic_of(None, order, "gemm_qkv") is None

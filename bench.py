"""Benchmark: forward pass of one FLUX-style double-stream DiT block on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2|c1|c4|c3] [--no-cpu-baseline]

A step is one dit_block_forward call (all 9 kernels of the block) over the
workload's synthetic inputs, already resident in HBM (c3: the whole denoising
step, 5 double-stream then 20 single-stream blocks).  Prints ONE JSON line.
Throughput (``value``) is algorithmic TFLOP/s: 26 N d^2 (GEMMs) + 4 N^2 d
(attention QK^T and PV) per block, 2 flop per multiply-add.  The bf16 workloads
run with fp16 activations and, by default, the matrix-product weights as fp16
copies of the bf16 weights made once at setup (outputs bit-identical to the bf16
weights; ``--gemm-weights bf16`` times the weights as given).

``roofline`` covers the kernel with the largest total time, timed with HIP
events the library records on the launch stream around each of its launches
(dit_timing_*).  Its ``traffic`` is measured in this run: before the bench
touches the GPU it runs its own step twice more as child processes under
``rocprofv3 --pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE``, each after three plain
device copies of a known size that scale the counters to bytes (``--no-traffic``
skips this).  ``calibration`` holds the launch floor, a measured MFMA-loop peak
and streaming read / copy bandwidth, and ``cold_hbm`` the AdaLN GEMV, modulation and QK-norm +
RoPE kernels on buffers rotated over more than 512 MB (every launch reads HBM).
``cpu_baseline`` times the fp64 oracle on one block of the same workload on the
host cores.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import signal
import tempfile
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DiT block fwd ms & TFLOP/s (bf16, 4096 img+512 txt tok), % of MFMA peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="c2", choices=["c0", "c1", "c2", "c3", "c4"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true", help="skip timing the step replayed from a captured graph")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--fp8-gemm", action="store_true",
                   help="time the fp8 (e4m3) GEMM on the block's four products at the workload's token count "
                        "(one JSON line of its own)")
    p.add_argument("--fp8-block", action="store_true",
                   help="time the fp8 double-stream block (its four weight products on e4m3 codes) at the "
                        "workload's size (one JSON line of its own)")
    p.add_argument("--fp8-attention", action="store_true",
                   help="time dit_joint_attention_fp8 (e4m3 q, k, v) at the workload's joint sequence and heads, "
                        "next to the fp16 kernel on the same shape")
    p.add_argument("--conv", action="store_true",
                   help="time the causal 3-D convolution on the video decoder's stage shapes at 832 x 480 "
                        "(one JSON line of its own)")
    p.add_argument("--shared-mod", action="store_true",
                   help="multi-block workloads: one AdaLN weight set per block kind, computed once per step")
    p.add_argument("--gemm-weights", default="f16", choices=["bf16", "f16"],
                   help="f16 (default): the matrix-product weights as fp16 copies of the bf16 weights, converted "
                        "once at setup by dit_convert_bf16_to_f16 (the conversion the fp16-activation GEMMs "
                        "otherwise apply to every staged weight tile; block outputs are bit-identical); "
                        "bf16: the bf16 weights as given")
    p.add_argument("--act", default="f16", choices=["f16", "bf16"],
                   help="storage of the activations between the block's steps (bf16 workloads)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                   help="first run a plain device-to-device copy of BYTES (3 times), to scale HBM "
                        "byte counters against a kernel of known traffic")
    p.add_argument("--no-traffic", action="store_true",
                   help="skip the two rocprofv3 counter passes that measure the kernels' HBM bytes")
    p.add_argument("--no-calibration", action="store_true",
                   help="skip the launch-floor, MFMA-loop, copy and cold-buffer measurements")
    p.add_argument("--traffic-child", action="store_true", help=argparse.SUPPRESS)
    return p.parse_args()


def step_work(cfg, shared_mod=False):
    """Algorithmic work of one step per launch site: {name: (flops, bytes, bound, launches)}.
    A step is the workload's blocks: n_double double-stream blocks (the first reads the bf16 input,
    later ones the fp32 residual stream), then n_single single-stream blocks (fp32 stream).
    shared_mod: the AdaLN GEMV runs once per block kind instead of once per block."""
    n, d, F, dc = cfg.n_tok, cfg.d, cfg.ffn_inner, cfg.dc
    es = 2 if cfg.dtype == "bf16" else 4            # weights and inter-step activations
    work = {}

    def add(name, flops=0.0, nbytes=0.0, bound="mfma"):
        f, b_, _, c = work.get(name, (0.0, 0.0, bound, 0))
        work[name] = (f + flops, b_ + nbytes, bound, c + 1)

    for blk in range(cfg.n_double + cfg.n_single):
        double = blk < cfg.n_double
        ex = es if blk == 0 else 4                   # block input: workload type, then fp32 stream
        if not shared_mod or blk in (0, cfg.n_double):
            add("adaln_gemv", nbytes=(12 if double else 3) * d * dc * es, bound="hbm")
        if double and cfg.dtype == "bf16" and d % 256 == 0:
            # QK RMSNorm + RoPE in the QKV product's epilogue, from a table of the angles' (cos, sin)
            # that the modulation writes as well (positions read, 64 pairs of fp32 written per token)
            add("modulate_x", nbytes=n * d * (ex + es) + n * 64 * 8.0 + 16.0 * n, bound="hbm")
        else:
            add("modulate_x", nbytes=n * d * (ex + es), bound="hbm")
            add("qk_rmsnorm_rope", nbytes=4.0 * n * d * es + 16.0 * n, bound="hbm")
        add("joint_attention", flops=4.0 * n * n * d)
        if double:
            add("gemm_qkv", flops=2.0 * n * d * 3 * d)
            add("gemm_out_proj", flops=2.0 * n * d * d)
            add("modulate_h", nbytes=n * d * (4 + es), bound="hbm")
            add("gemm_ffn_in_swiglu", flops=2.0 * n * d * 2 * F)
            add("gemm_ffn_down", flops=2.0 * n * F * d)
        else:
            add("gemm_linear1", flops=2.0 * n * d * (3 * d + 2 * F))
            add("gemm_linear2", flops=2.0 * n * (d + F) * d)
    return work


def kernel_work(cfg, name, shared_mod=False):
    """Algorithmic work of one launch of a launch site, averaged over the step: (flops, bytes, bound)."""
    w = step_work(cfg, shared_mod).get(name)
    if w is None:
        return None, None, "?"
    f, b, bound, cnt = w
    return (f / cnt if f else None), (b / cnt if b else None), bound


CALIB_BYTES = 1 << 28            # plain copy that scales the byte counters
TRAFFIC_COUNTERS = ("FETCH_SIZE", "WRITE_SIZE")


def provenance():
    """Where the numbers come from (no GPU use): git revision and dirty flag when the tree is a git
    checkout, a hash of the sources the library is built from, the ROCm version."""
    info = {"git_rev": None, "git_dirty": None}
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=20)
        if r.returncode == 0:
            info["git_rev"] = r.stdout.strip()
            st = subprocess.run(["git", "-C", ROOT, "status", "--porcelain", "--untracked-files=no"],
                                capture_output=True, text=True, timeout=20)
            info["git_dirty"] = bool(st.stdout.strip()) if st.returncode == 0 else None
    except Exception:
        pass
    h = hashlib.sha256()
    srcs = sorted(glob.glob(os.path.join(ROOT, "attention_dit_block_amd", "csrc", "*")) +
                  [os.path.join(ROOT, "include", "dit.h")])
    for path in srcs:
        h.update(os.path.relpath(path, ROOT).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    info["source_sha256"] = h.hexdigest()[:16]
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        info["rocm"] = None
    return info


def _run_child(cmd, timeout_s):
    """Run cmd in its own process group; kill the whole group if it outlives timeout_s."""
    proc = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                            start_new_session=True)
    try:
        out, _ = proc.communicate(timeout=timeout_s)
    except subprocess.TimeoutExpired:
        os.killpg(proc.pid, signal.SIGKILL)
        out, _ = proc.communicate()
        return -9, out
    return proc.returncode, out


def _read_counter_csv(path, counter):
    """[(dispatch id, kernel name, counter value summed over its instances)] in dispatch order."""
    vals, names = {}, {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") != counter:
                continue
            d = int(r["Dispatch_Id"])
            vals[d] = vals.get(d, 0.0) + float(r["Counter_Value"])
            names[d] = r["Kernel_Name"]
    return [(d, names[d], vals[d]) for d in sorted(vals)]


def counters_from_csv(path, counter):
    """One counter pass -> {"scale": bytes per counted byte, "values": bytes of each library launch
    after setup, in order, "symbols": their kernels}, or a reason string.  The scale is the median
    over the three largest non-library dispatches before the first library launch (the calibration
    copies of CALIB_BYTES each way); the library's setup conversions (bf16 -> fp16 weight copies) are
    skipped."""
    rows = _read_counter_csv(path, counter)
    lib = [i for i, (_, n, _) in enumerate(rows) if "dit::" in n and "bf16_to_f16" not in n]
    if not lib:
        return f"{counter}: no library dispatches"
    copies = sorted((v for _, n, v in rows[:lib[0]] if "dit::" not in n), reverse=True)[:3]
    if len(copies) < 3 or min(copies) <= 0:
        return f"{counter}: calibration copies not found"
    scale = CALIB_BYTES / (sorted(copies)[1] * 1024.0)
    return {"scale": scale, "values": [rows[i][2] * 1024.0 * scale for i in lib], "symbols": [rows[i][1] for i in lib]}


def counter_passes(args):
    """The step's HBM bytes per launch, measured: the bench runs its own step (3 steps, after three
    plain copies of CALIB_BYTES) as a child process under rocprofv3 --pmc FETCH_SIZE, then under
    --pmc WRITE_SIZE.  Both counters are in KiB per dispatch; each is scaled by what it reads for
    the copies (the copy moves CALIB_BYTES each way).  Runs before this process uses the GPU.
    Returns ({counter: {"scale": bytes per counted byte, "per_step": [bytes of launch i of a step],
    "symbols": [...]}}, command) or (None, reason)."""
    child = [sys.executable, os.path.abspath(__file__), "--traffic-child", "--workload", args.workload,
             "--steps", "3", "--warmup", "0", "--seed", str(args.seed), "--act", args.act,
             "--gemm-weights", args.gemm_weights, "--copy-calibration", str(CALIB_BYTES)]
    res = {}
    with tempfile.TemporaryDirectory(prefix="dit_counters_") as tmp:
        for ctr in TRAFFIC_COUNTERS:
            d = os.path.join(tmp, ctr)
            cmd = ["rocprofv3", "--pmc", ctr, "--output-format", "csv", "-d", d, "-o", "c", "--"] + child
            print(f"traffic: rocprofv3 --pmc {ctr} pass", file=sys.stderr, flush=True)
            try:
                rc, out = _run_child(cmd, 400)
            except OSError as e:
                return None, f"rocprofv3 not runnable: {e}"
            files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
            if rc != 0 or not files:
                return None, f"{ctr} pass failed (rc {rc}): {out[-300:]}"
            res[ctr] = counters_from_csv(files[0], ctr)
            if isinstance(res[ctr], str):
                return None, res[ctr]
    cmd_text = "rocprofv3 --pmc <FETCH_SIZE|WRITE_SIZE> --output-format csv -d <dir> -o c -- " + " ".join(
        ["python3", "bench.py"] + child[2:])
    return res, cmd_text


def traffic_of(counters, order, name):
    """Bytes per launch of launch site `name` (position order.index(name) in a step of len(order)
    launches), averaged over the child's last two steps; None if the dispatches do not line up."""
    if not counters or name not in order:
        return None
    L, p = len(order), order.index(name)
    total, detail = 0.0, {}
    for ctr, c in counters.items():
        v, sym = c["values"], c["symbols"]
        if len(v) % L or len(v) < 2 * L:
            return None
        idx = [len(v) - 2 * L + p, len(v) - L + p]
        if sym[idx[0]] != sym[idx[1]]:
            return None
        b = sum(v[i] for i in idx) / 2
        detail[ctr.lower() + "_bytes"] = int(b)
        detail[ctr.lower() + "_scale"] = round(c["scale"], 4)
        total += b
    detail["bytes"] = int(total)
    return detail


def calibration(dit, torch, dev):
    """Launch floor (the library's smallest launch, back to back), measured MFMA-loop rate and
    device copy bandwidth: the ceilings this box reaches, next to the published peaks."""
    s = torch.cuda.current_stream()

    def ev_ms(fn, reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        for _ in range(reps):
            fn()
        b.record(s)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    out = {}
    src = torch.zeros(8, dtype=torch.bfloat16, device=dev)
    dst = torch.empty(8, dtype=torch.float16, device=dev)
    ev_ms(lambda: dit.convert_bf16_to_f16(src, dst), 200)
    out["launch_floor_us"] = round(min(ev_ms(lambda: dit.convert_bf16_to_f16(src, dst), 2000) for _ in range(3))
                                   / 2000 * 1e3, 2)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wg, iters = 8 * cus, 4000
    buf = torch.empty(wg * 256, dtype=torch.float32, device=dev)
    ev_ms(lambda: dit.mfma_loop(wg, iters, buf), 3)
    best = min(ev_ms(lambda: dit.mfma_loop(wg, iters, buf), 5) / 5 for _ in range(3))
    out["mfma_loop_f16_tflops"] = round(wg * 4 * iters * 4 * 32768.0 / (best * 1e-3) / 1e12, 1)
    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    ev_ms(lambda: b.copy_(a), 2)
    best = min(ev_ms(lambda: b.copy_(a), 10) / 10 for _ in range(3))
    out["copy_gbs"] = round(2.0 * n * 4 / (best * 1e-3) / 1e9, 1)      # the runtime's device copy
    out["copy_bytes"] = 2 * n * 4
    # the library's own streaming probe (16-byte nontemporal accesses, 8 workgroups per CU)
    sink = torch.empty(8 * cus * 256, dtype=torch.float32, device=dev)
    for mode, key, moved in ((0, "stream_read_gbs", n * 4), (1, "stream_copy_gbs", 2 * n * 4)):
        fn = (lambda: dit.stream_probe(0, a, sink=sink, workgroups=8 * cus)) if mode == 0 else \
             (lambda: dit.stream_probe(1, a, dst=b, workgroups=8 * cus))
        ev_ms(fn, 2)
        best = min(ev_ms(fn, 10) / 10 for _ in range(3))
        out[key] = round(moved / (best * 1e-3) / 1e9, 1)
    # the GEMM's k-loop and the attention step with their operands in LDS (one workgroup per CU): what
    # the instruction schedules reach without the kernels' global loads and epilogues
    res = torch.empty(cus * 512, dtype=torch.float32, device=dev)
    win = torch.full((2 << 20,), 0.015625, dtype=torch.float16, device=dev)        # 4 MiB of 2^-6
    # random-valued operands as well: constant ones let the device hold a higher clock
    win_r = (torch.rand(2 << 20, device=dev) * 0.25 - 0.125).to(torch.float16)
    ks, tiles = 2000, 2000
    for mode, key in ((0, "interleaved"), (1, "pingpong"), (2, "interleaved_l2_loads"), (3, "pingpong_l2_loads"),
                      (8, "registers"), (12, "registers_random"), (4, "interleaved_random"), (5, "pingpong_random"),
                      (6, "interleaved_l2_loads_random"), (7, "pingpong_l2_loads_random")):
        fn = lambda: dit.gemm_kloop_probe(mode, cus, ks, res, window=win_r if mode & 4 else win)
        ev_ms(fn, 2)
        best = min(ev_ms(fn, 5) / 5 for _ in range(3))
        out.setdefault("gemm_kloop_lds_tflops", {})[key] = round(2.0 * 256 * 256 * 64 * ks * cus / (best * 1e-3) / 1e12, 1)
    for mode, key in ((0, "kernel_order"), (1, "pingpong"), (2, "kernel_order_random")):
        fn = lambda: dit.attention_step_probe(mode, cus, tiles, res, c2=0.18 if mode & 2 else 0.0)
        ev_ms(fn, 2)
        best = min(ev_ms(fn, 5) / 5 for _ in range(3))
        out.setdefault("attention_step_lds_tflops", {})[key] = round(4.0 * 256 * 64 * 128 * tiles * cus / (best * 1e-3) / 1e12, 1)
    return out


def cold_hbm(cfg, dit, torch, dev):
    """The HBM-bound kernels of the block, one standalone launch after another on inputs rotated
    over more than 512 MB (more than the MI355X's 8 x 4 MB L2 and 256 MB MALL), so every launch
    reads HBM: the AdaLN GEMV (both streams' 12 d x d_cond weights), the modulation of x (bf16 in)
    and of h (fp32 in) to fp16, and QK-norm + RoPE in place on fp16 q and k of a [n, 3d] buffer.
    Algorithmic bytes per launch: weights + vectors (GEMV), n d (in + out) (modulation), 4 n d 2 +
    16 n (QK-norm + RoPE: q and k read and written, positions)."""
    n, d, dc, H = cfg.n_tok, cfg.d, cfg.dc, cfg.n_heads
    rot = 600 << 20
    out = {}

    def measure(site, make, call, nbytes):
        sets = [make() for _ in range(max(2, -(-rot // nbytes)))]
        for st in sets:
            call(st)
        torch.cuda.synchronize()
        reps = 3
        dit.timing_begin(8 * reps * len(sets))
        for _ in range(reps):
            for st in sets:
                call(st)
        dit.timing_end()
        torch.cuda.synchronize()
        cnt, tot = dit.timing_read()[site]
        us = tot / cnt * 1e3
        out[site if site != "modulate" else make.__name__] = {
            "us": round(us, 2), "bytes": int(nbytes), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4), "rotated_sets": len(sets)}
        del sets
        torch.cuda.empty_cache()

    cond = torch.randn(dc, device=dev).to(torch.bfloat16)
    mod = torch.empty(12 * d, dtype=torch.float32, device=dev)

    def gemv_set():
        return torch.randn(12 * d, dc, device=dev).mul_(0.02).to(torch.bfloat16)
    measure("adaln_gemv", gemv_set, lambda w: dit.adaln_modulate(cond, w, 12, d, mod), 12 * d * dc * 2 + dc * 2 + 12 * d * 4)

    w2 = torch.randn(2 * d, dc, device=dev).mul_(0.02).to(torch.bfloat16)
    mod2 = torch.empty(2 * d, dtype=torch.float32, device=dev)

    def modulate_x():
        return (torch.randn(n, d, device=dev).to(torch.bfloat16), torch.empty(n, d, dtype=torch.float16, device=dev))

    def modulate_h():
        return (torch.randn(n, d, device=dev), torch.empty(n, d, dtype=torch.float16, device=dev))
    for mk, es in ((modulate_x, 2), (modulate_h, 4)):
        measure("modulate", mk, lambda xs: dit.adaln_modulate(cond, w2, 2, d, mod2, x=xs[0], x_out=xs[1]),
                n * d * (es + 2))

    import dit_inputs as di
    pos = torch.from_numpy(di.positions(cfg.n_txt, cfg.grid_h, cfg.grid_w)).to(dev)
    qk_w = torch.ones(2, 2, 128, dtype=torch.bfloat16, device=dev)

    def qkv_set():
        return torch.randn(n, 3 * d, device=dev).to(torch.float16)
    measure("qk_rmsnorm_rope", qkv_set,
            lambda b: dit.qk_rmsnorm_rope(b[:, :d], b[:, d:2 * d], H, qk_w, cfg.n_txt, pos), 4 * n * d * 2 + 16 * n)
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the block is not sharded across GPUs "
              f"in this build", file=sys.stderr)
        sys.exit(2)

    import torch
    import dit_inputs as di
    import attention_dit_block_amd as dit

    cfg = di.config_by_name(args.workload)
    # everything that starts another program runs here, before this process uses the GPU
    prov = provenance() if not args.traffic_child else None
    counters, counters_cmd = None, None
    single_block = cfg.n_double == 1 and cfg.n_single == 0
    if not (args.traffic_child or args.no_traffic or args.fp8_gemm or args.conv or args.fp8_block or
            args.fp8_attention) and single_block:
        counters, counters_cmd = counter_passes(args)
        if counters is None:
            print(f"traffic: not measured ({counters_cmd})", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    if args.fp8_gemm:
        return fp8_gemm_bench(args, cfg, dit, torch)
    if args.conv:
        return conv_bench(args, dit, torch)
    if args.fp8_block:
        return fp8_block_bench(args, cfg, dit, torch)
    if args.fp8_attention:
        return fp8_attention_bench(args, cfg, dit, torch)
    t = cfg.dtype
    if args.copy_calibration:
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copy calibration: 3 copies of {n * 4} bytes", file=sys.stderr, flush=True)
        del src, dst

    def up(a, dt):
        a = np.ascontiguousarray(a)
        if dt == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        if dt == "i32":
            return torch.from_numpy(a).to(dev)
        return torch.from_numpy(a).to(dev)

    tdt = dit.DIT_BF16 if t == "bf16" else dit.DIT_F32
    step_blocks = []            # callables, one per block of the step
    t0 = time.time()
    inp = di.double_block_inputs(cfg, seed=args.seed)
    cond, pos = up(inp["cond"], t), up(inp["pos"], "i32")
    x_txt, x_img = up(inp["x_txt"], t), up(inp["x_img"], t)
    act = None if t != "bf16" else (dit.DIT_F16 if args.act == "f16" else dit.DIT_BF16)
    f16w = t == "bf16" and args.act == "f16" and args.gemm_weights == "f16"
    shape = dit.Shape(dtype=tdt, d=cfg.d, n_heads=cfg.n_heads, ffn_inner=cfg.ffn_inner, n_txt=cfg.n_txt,
                      n_img=cfg.n_img, d_cond=cfg.dc, x_dtype=tdt, y_dtype=dit.DIT_F32, act_dtype=act,
                      gemm_w_dtype=dit.DIT_F16 if f16w else 0)
    product_weights = ("w_qkv", "w_o", "w_ffn_in", "w_ffn_out", "w_1", "w_2")

    def upw(a, dt, name):
        """Upload one weight tensor; with fp16 product weights, convert those once on the GPU."""
        g = up(a, dt)
        if f16w and name in product_weights:
            h = torch.empty(g.shape, dtype=torch.float16, device=dev)
            dit.convert_bf16_to_f16(g, h)
            torch.cuda.synchronize()
            del g
            return h
        return g
    ws = torch.empty(max(dit.block_workspace_size(shape), dit.block_workspace_size(shape, True)),
                     dtype=torch.uint8, device=dev)
    y_txt = torch.empty(cfg.n_txt, cfg.d, dtype=torch.float32, device=dev)
    y_img = torch.empty(cfg.n_img, cfg.d, dtype=torch.float32, device=dev)
    if cfg.n_double == 1 and cfg.n_single == 0:
        wt = {k: upw(v, t, k) for k, v in inp["txt"].items()}
        wi = {k: upw(v, t, k) for k, v in inp["img"].items()}
        step_blocks.append(lambda: dit.block_forward(shape, wt, wi, cond, pos, x_txt, x_img, y_txt, y_img, ws))
    else:
        # the full step through dit_step_forward: n_double double-stream blocks, then n_single
        # single-stream blocks over [txt; img], one fp32 residual stream
        wts, wis, sws = [], [], []
        for b in range(cfg.n_double):
            print(f"setup: double block {b + 1}/{cfg.n_double}", file=sys.stderr, flush=True)
            bi = di.double_block_inputs(cfg, seed=args.seed, block=b)
            wts.append({k: upw(v, t, k) for k, v in bi["txt"].items()})
            wis.append({k: upw(v, t, k) for k, v in bi["img"].items()})
        for b in range(cfg.n_single):
            print(f"setup: single block {b + 1}/{cfg.n_single}", file=sys.stderr, flush=True)
            sws.append({k: upw(v, t, k) for k, v in di.single_weights(cfg, args.seed, cfg.n_double + b).items()})
        state = torch.empty(cfg.n_tok, cfg.d, dtype=torch.float32, device=dev)
        if args.shared_mod:
            sm = {k: up(v, t) for k, v in di.shared_mod_weights(cfg, seed=args.seed).items()}
            ws = torch.empty(dit.step_shared_mod_workspace_size(shape, cfg.n_double, cfg.n_single),
                             dtype=torch.uint8, device=dev)
            step_blocks.append(lambda: dit.step_forward_shared_mod(shape, wts, wis, sws, sm["txt"], sm["img"],
                                                                   sm["single"], cond, pos, x_txt, x_img, state, ws))
        else:
            ws = torch.empty(dit.step_workspace_size(shape, cfg.n_double, cfg.n_single), dtype=torch.uint8,
                             device=dev)
            step_blocks.append(lambda: dit.step_forward(shape, wts, wis, sws, cond, pos, x_txt, x_img, state, ws))
    setup_s = time.time() - t0
    shared = bool(args.shared_mod) and (cfg.n_double + cfg.n_single) > 1

    def step():
        for f in step_blocks:
            f()

    if args.traffic_child:
        # a counter pass: the steps only (the parent reads the counters of their launches)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        return
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t_start = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps
    ev_ms = evs[0].elapsed_time(evs[-1]) / args.steps
    step_ms = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    flops = cfg.flops_step()
    tflops = flops / (ms_per_step * 1e-3) / 1e12

    # the same step replayed from a captured graph (one launch per step from the host)
    ms_graph = None
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        ms_graph = g0.elapsed_time(g1) / args.steps
        del graph

    # per-kernel durations: HIP events around every launch of the library, same stream
    dit.timing_begin(args.steps * 16 * (cfg.n_double + cfg.n_single))     # >= the launches of every step
    for _ in range(args.steps):
        step()
    dit.timing_end()
    torch.cuda.synchronize()
    kt = dit.timing_read()
    # launch sites in the order of a step (first appearance), when each runs once per step
    order = list(kt) if all(c == args.steps for c, _ in kt.values()) else []
    kernels = {}
    for name, (cnt, tot) in kt.items():
        avg = tot / cnt
        fl, by, bound = kernel_work(cfg, name, shared)
        e = {"launches_per_step": cnt / args.steps, "avg_ms": round(avg, 5),
             "share": round(tot / sum(v[1] for v in kt.values()), 4), "bound": bound}
        tr = traffic_of(counters, order, name)
        if tr:
            e["traffic_bytes"] = tr["bytes"]
        if fl:
            e["tflops"] = round(fl / (avg * 1e-3) / 1e12, 1)
            e["frac_mfma"] = round(e["tflops"] / PEAK_BF16_TFLOPS, 4)
        if by:
            e["gbs"] = round(by / (avg * 1e-3) / 1e9, 1)
            e["frac_hbm"] = round(e["gbs"] / PEAK_HBM_GBS, 4)
        kernels[name] = e
    dom = max(kt.items(), key=lambda kv: kv[1][1])[0]
    fl, by, bound = kernel_work(cfg, dom, shared)
    avg = kt[dom][1] / kt[dom][0]
    if fl:
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(fl / (avg * 1e-3) / 1e12, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(by / (avg * 1e-3) / 1e9, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["avg_us"] = round(avg * 1e3, 2)
    roof["algorithmic"] = {"flops": fl} if fl else {"bytes": by}
    tr = traffic_of(counters, order, dom)
    roof["traffic"] = tr["bytes"] if tr else None
    if tr:
        roof["traffic_detail"] = tr
        roof["traffic_source"] = counters_cmd
    else:
        roof["traffic_note"] = ("counter passes skipped (--no-traffic)" if args.no_traffic else
                                counters_cmd if counters is None else
                                "the counter passes' launches did not line up with the step's launch sites")
    calib = None if args.no_calibration else calibration(dit, torch, dev)
    cold = None if args.no_calibration or t != "bf16" else cold_hbm(cfg, dit, torch, dev)

    # the arithmetic type of the matrix products: fp16 operands when the activations are fp16 (bf16
    # weights converted to fp16 copies, or while they are staged), bf16 operands otherwise
    if t != "bf16":
        mfma_dtype, arithmetic = "f32", "fp32 storage and FMA arithmetic"
    elif args.act == "f16":
        mfma_dtype = "f16"
        arithmetic = ("fp16-operand MFMA with fp32 accumulation (bf16 model weights, fp16 activations), fp32 "
                      "residual stream, softmax and norms")
    else:
        mfma_dtype, arithmetic = "bf16", "bf16-operand MFMA with fp32 accumulation, fp32 residual stream"
    out = {
        "metric": METRIC, "value": round(tflops, 1), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": mfma_dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "model_dtype": t, "activations": args.act if t == "bf16" else "f32",
                   "product_weights": ("f16 copies of the bf16 weights, converted once at setup (round to nearest "
                                       "even; |w| < 2^-14 become fp16 subnormals)") if f16w else t,
                   "arithmetic": arithmetic,
                   "blocks": cfg.n_double + cfg.n_single, "d": cfg.d, "heads": cfg.n_heads,
                   "ffn_inner": cfg.ffn_inner, "n_txt": cfg.n_txt, "n_img": cfg.n_img, "tokens": cfg.n_tok,
                   "gflop_per_step": round(flops / 1e9, 1),
                   "modulation": "shared" if shared else "per_block"},
        "frac_mfma_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "ms_per_step_hip_events": round(ev_ms, 4),
        "ms_per_step_median": round(step_ms[len(step_ms) // 2], 4),
        "ms_per_step_min": round(step_ms[0], 4),
        "ms_per_step_graph_replay": None if ms_graph is None else round(ms_graph, 4),
        "roofline": roof,
        "kernels": kernels,
        "calibration": calib,
        "cold_hbm": cold,
        "provenance": prov,
        "setup_s": round(setup_s, 1),
    }

    if not args.no_cpu_baseline and cfg.n_single == 0:
        out["cpu_baseline"] = cpu_baseline(cfg, inp)
    print(json.dumps(out), flush=True)


def fp8_block_bench(args, cfg, dit, torch):
    """The workload's blocks with their weight products on e4m3 codes (dit_block_forward_fp8,
    dit_single_block_forward_fp8): the weight matrices quantised once to e4m3 before timing (a
    weight format, like the bf16 storage of the others), the activations quantised inside every
    step.  One double block for the one-block workloads; the whole step (double blocks on the text
    and image streams, then single blocks over [text; image], one fp32 residual stream) otherwise.
    Times K steps like the main bench and every launch with the library's HIP events."""
    if cfg.dtype != "bf16":
        print("--fp8-block needs a bf16 workload", file=sys.stderr)
        sys.exit(2)
    import dit_inputs as di
    dev = torch.device("cuda:0")

    def up(a, dt):
        a = np.ascontiguousarray(a)
        if dt == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    def quantised(w, names):
        out = {"w_mod": up(w["w_mod"], "bf16"), "qk_norm_w": up(w["qk_norm_w"], "bf16")}
        for name, sname in names:
            wt = up(w[name], "bf16")
            q = torch.empty(wt.shape, dtype=torch.uint8, device=dev)
            sc = torch.empty(wt.shape[0], dtype=torch.float32, device=dev)
            dit.quantize_fp8(wt, q, sc)
            out[name], out[sname] = q, sc
            del wt
        torch.cuda.synchronize()
        return out

    dnames = [("w_qkv", "s_qkv"), ("w_o", "s_o"), ("w_ffn_in", "s_ffn_in"), ("w_ffn_out", "s_ffn_out")]
    inp = di.double_block_inputs(cfg, seed=args.seed)
    cond, pos = up(inp["cond"], "bf16"), up(inp["pos"], "i32")
    x_txt, x_img = up(inp["x_txt"], "bf16"), up(inp["x_img"], "bf16")
    kw = dict(d=cfg.d, n_heads=cfg.n_heads, ffn_inner=cfg.ffn_inner, n_txt=cfg.n_txt, n_img=cfg.n_img,
              d_cond=cfg.dc, y_dtype=dit.DIT_F32, act_dtype=dit.DIT_F16)
    sh_in = dit.Shape(dtype=dit.DIT_BF16, x_dtype=dit.DIT_BF16, **kw)       # first block: bf16 input
    sh_st = dit.Shape(dtype=dit.DIT_BF16, x_dtype=dit.DIT_F32, **kw)        # later blocks: fp32 stream
    ws = torch.empty(max(dit.block_fp8_workspace_size(sh_in), dit.single_block_fp8_workspace_size(sh_st)),
                     dtype=torch.uint8, device=dev)
    state = torch.empty(cfg.n_tok, cfg.d, dtype=torch.float32, device=dev)
    st_txt, st_img = state[:cfg.n_txt], state[cfg.n_txt:]
    calls = []
    for b in range(cfg.n_double):
        print(f"setup: fp8 double block {b + 1}/{cfg.n_double}", file=sys.stderr, flush=True)
        bi = inp if b == 0 else di.double_block_inputs(cfg, seed=args.seed, block=b)
        wt, wi = quantised(bi["txt"], dnames), quantised(bi["img"], dnames)
        if b == 0:
            calls.append(lambda wt=wt, wi=wi: dit.block_forward_fp8(sh_in, wt, wi, cond, pos, x_txt, x_img, st_txt,
                                                                     st_img, ws))
        else:
            calls.append(lambda wt=wt, wi=wi: dit.block_forward_fp8(sh_st, wt, wi, cond, pos, st_txt, st_img, st_txt,
                                                                     st_img, ws))
    for b in range(cfg.n_single):
        print(f"setup: fp8 single block {b + 1}/{cfg.n_single}", file=sys.stderr, flush=True)
        w = quantised(di.single_weights(cfg, args.seed, cfg.n_double + b), [("w_1", "s_1"), ("w_2", "s_2")])
        calls.append(lambda w=w: dit.single_block_forward_fp8(sh_st, w, cond, pos, state, state, ws))

    def step():
        for f in calls:
            f()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    dit.timing_begin(args.steps * 16 * len(calls))
    for _ in range(args.steps):
        step()
    dit.timing_end()
    torch.cuda.synchronize()
    kt = dit.timing_read()
    n, d, F = cfg.n_tok, cfg.d, cfg.ffn_inner
    gemm = {"gemm_fp8_qkv": 6.0 * n * d * d, "gemm_fp8_out_proj": 2.0 * n * d * d,
            "gemm_fp8_ffn_in_swiglu": 4.0 * n * d * F, "gemm_fp8_ffn_down": 2.0 * n * F * d,
            "gemm_fp8_linear1_qkv": 6.0 * n * d * d, "gemm_fp8_linear1_gu": 4.0 * n * d * F,
            "gemm_fp8_linear2": 2.0 * n * (d + F) * d}
    quant = {"quantize_o": n * d * 3.0, "quantize_f": n * F * 3.0, "quantize_of": n * (d + F) * 3.0,
             "modulate_h_fp8": n * d * 5.0,              # 16-bit / fp32 read + code written
             "qk_rmsnorm_rope_fp8": n * 3 * d * 3.0}     # q, k, v read (16-bit), their codes written
    gemm["joint_attention_fp8"] = 4.0 * n * n * d
    kernels = {}
    for name, (cnt, tot) in kt.items():
        avg = tot / cnt
        e = {"launches_per_step": cnt / args.steps, "avg_ms": round(avg, 5),
             "share": round(tot / sum(v[1] for v in kt.values()), 4)}
        if name in gemm:
            e["tflops"] = round(gemm[name] / (avg * 1e-3) / 1e12, 1)
            e["frac_fp8_peak"] = round(e["tflops"] / 5000.0, 4)
        elif name in quant:
            e["gbs"] = round(quant[name] / (avg * 1e-3) / 1e9, 1)
            e["frac_hbm"] = round(e["gbs"] / PEAK_HBM_GBS, 4)
        kernels[name] = e
    flops = cfg.flops_step()
    out = {"metric": "fp8 (e4m3 products) DiT block fwd ms & TFLOP/s", "value": round(flops / (ms * 1e-3) / 1e12, 1),
           "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3+f16",
           "data": "synthetic",
           "config": {"workload": cfg.name, "blocks": cfg.n_double + cfg.n_single, "tokens": cfg.n_tok,
                      "gflop_per_step": round(flops / 1e9, 1),
                      "products": "e4m3 weights (per-row scales, quantised once) x e4m3 activations (per row, "
                                  "every step)"},
           "kernels": kernels}
    print(json.dumps(out), flush=True)


def fp8_attention_bench(args, cfg, dit, torch):
    """dit_joint_attention_fp8 over the workload's joint sequence (n_txt + n_img tokens, its heads)
    on seeded e4m3 codes and scales (dit_inputs.fp8_attention_inputs), and dit_joint_attention on
    fp16 q, k, v of the same shape; both one workgroup per (head, 256 queries), timed with HIP
    events around K launches after W warm-up launches.  Flop: 4 N^2 d (QK^T and PV)."""
    import dit_inputs as di
    n, H = cfg.n_tok, cfg.n_heads
    x = di.fp8_attention_inputs(n, H, seed=args.seed)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in x.items()}
    o8 = torch.empty(n, H * 128, dtype=torch.float16, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(args.seed)
    q16, k16, v16 = (torch.randn(n, H * 128, device="cuda", generator=g).half() for _ in range(3))
    o16 = torch.empty_like(q16)
    s = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        for _ in range(args.steps):
            fn()
        b.record(s)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps
    ms8 = timed(lambda: dit.joint_attention_fp8(t["q8"], t["sq"], t["k8"], t["sk"], t["v8"], t["sv"], o8, H))
    ms16 = timed(lambda: dit.joint_attention(q16, k16, v16, o16, H))
    flops = 4.0 * n * n * H * 128
    tf8, tf16 = flops / (ms8 * 1e-3) / 1e12, flops / (ms16 * 1e-3) / 1e12
    out = {"metric": "fp8 joint attention ms & TFLOP/s (e4m3 q, k, v; scores and PV on fp8 MFMA)",
           "value": round(tf8, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms8, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "fp8_e4m3", "data": "synthetic",
           "config": {"workload": cfg.name, "tokens": n, "heads": H, "head_dim": 128,
                      "inputs": "e4m3 codes drawn directly (dit_inputs.fp8_attention_inputs), per token-and-head q "
                                "scales, per-head k and v scales"},
           "roofline": {"bound": "mfma", "achieved": round(tf8, 1), "peak": 5000.0, "unit": "TFLOP/s",
                        "frac": round(tf8 / 5000.0, 4), "frac_of_bf16_peak": round(tf8 / PEAK_BF16_TFLOPS, 4)},
           "fp16_same_shape": {"ms": round(ms16, 4), "tflops": round(tf16, 1),
                               "frac_bf16_peak": round(tf16 / PEAK_BF16_TFLOPS, 4)},
           "speedup_over_fp16": round(ms16 / ms8, 3)}
    print(json.dumps(out), flush=True)


# Causal 3-D convolutions at the video decoder's stage resolutions for an 832 x 480 output (the
# decoder page's measurement size): latent 104 x 60 doubled three times, 384 channels at the two
# coarsest stages, then 192 and 96, and the 96 -> 3 head; 3 x 3 x 3 taps over 3-frame clips.
CONV_LAYERS = [
    ("384ch_60x104", 60, 104, 384, 384), ("384ch_120x208", 120, 208, 384, 384),
    ("192ch_240x416", 240, 416, 192, 192), ("96ch_480x832", 480, 832, 96, 96), ("head_96to3_480x832", 480, 832, 96, 3),
]


def conv_bench(args, dit, torch):
    """dit_conv3d_causal on the layer shapes above (one clip of 3 frames each, bf16 in and out, fp32
    bias), timed with HIP events on the launch stream.  Flop: 2 x outputs x Cout x taps x Cin
    (no padded work counted)."""
    import dit_inputs as di
    T, KT, K = 3, 3, 3
    s = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(args.steps):
            fn()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps
    per, tot, flops = {}, 0.0, 0.0
    for name, H, W, cin, cout in CONV_LAYERS:
        x = torch.from_numpy(di.draw((T * H * W * cin,), 1.0, "bf16", args.seed, "x").view("int16")).view(
            torch.bfloat16).to("cuda").view(1, T, H, W, cin)
        w = torch.from_numpy(di.draw((cout * KT * K * K * cin,), 0.02, "bf16", args.seed, "w_1").view("int16")).view(
            torch.bfloat16).to("cuda").view(cout, KT, K, K, cin)
        b = torch.zeros(cout, dtype=torch.float32, device="cuda")
        y = torch.empty(1, T, H, W, cout, dtype=torch.bfloat16, device="cuda")
        t = timed(lambda: dit.conv3d_causal(x, w, y, bias=b))
        f = 2.0 * T * H * W * cout * KT * K * K * cin
        per[name] = {"us_per_clip": round(t * 1e3, 1), "us_per_frame": round(t * 1e3 / T, 1),
                     "tflops": round(f / t / 1e9, 1)}
        tot, flops = tot + t, flops + f
        del x, w, b, y
    out = {"metric": "causal 3-D convolution TFLOP/s on the video decoder's stage shapes", "value": round(flops / tot / 1e9, 1),
           "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(tot, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "video_decoder_conv3d_832x480", "frames_per_clip": T, "taps": [KT, K, K]},
           "frac_mfma_peak": round(flops / tot / 1e9 / 2500.0, 4), "layers": per}
    print(json.dumps(out), flush=True)


def fp8_gemm_bench(args, cfg, dit, torch):
    """The block's four products (QKV, out-proj, FFN-in, FFN-down over all n_txt + n_img tokens) as
    fp8 e4m3 GEMMs on quantised seeded inputs, timed with HIP events on the launch stream; the
    bf16 kernel on the same shapes beside it.  The activation quantisation is timed separately."""
    import dit_inputs as di
    n, d, F = cfg.n_tok, cfg.d, cfg.ffn_inner
    shapes = {"qkv": (3 * d, d), "out_proj": (d, d), "ffn_in": (2 * F, d), "ffn_down": (d, F)}
    s = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(args.steps):
            fn()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps
    per, tot8, tot16, totq, flops = {}, 0.0, 0.0, 0.0, 0.0
    for name, (nout, k) in shapes.items():
        x = torch.from_numpy(di.draw((n, k), 1.0, "bf16", args.seed, "x").view("int16")).view(torch.bfloat16).to("cuda")
        w = torch.from_numpy(di.draw((nout, k), 0.02, "bf16", args.seed, "w_1").view("int16")).view(torch.bfloat16).to("cuda")
        xq = torch.empty(n, k, dtype=torch.uint8, device="cuda")
        sx = torch.empty(n, dtype=torch.float32, device="cuda")
        wq = torch.empty(nout, k, dtype=torch.uint8, device="cuda")
        sw = torch.empty(nout, dtype=torch.float32, device="cuda")
        y = torch.empty(n, nout, dtype=torch.bfloat16, device="cuda")
        dit.quantize_fp8(w, wq, sw)
        tq = timed(lambda: dit.quantize_fp8(x, xq, sx))
        t8 = timed(lambda: dit.linear_fp8(xq, sx, wq, sw, y))
        t16 = timed(lambda: dit.linear(x, w, y))
        f = 2.0 * n * nout * k
        per[name] = {"fp8_us": round(t8 * 1e3, 1), "fp8_tflops": round(f / t8 / 1e9, 1),
                     "quantize_x_us": round(tq * 1e3, 1), "bf16_us": round(t16 * 1e3, 1),
                     "bf16_tflops": round(f / t16 / 1e9, 1)}
        tot8, tot16, totq, flops = tot8 + t8, tot16 + t16, totq + tq, flops + f
    out = {"metric": "fp8 (e4m3) GEMM TFLOP/s on the block's four products", "value": round(flops / tot8 / 1e9, 1),
           "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(tot8, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "fp8_e4m3", "data": "synthetic",
           "config": {"workload": cfg.name + "_gemms", "tokens": n, "d": d, "ffn_inner": F},
           "frac_fp8_peak": round(flops / tot8 / 1e9 / 5000.0, 4),
           "ms_quantize_activations": round(totq, 4), "ms_bf16_same_products": round(tot16, 4),
           "products": per}
    print(json.dumps(out), flush=True)


def cpu_baseline(cfg, inp):
    """The fp64 oracle, as it stands, on one full block of the same workload."""
    from oracle import dit_oracle as o
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        threads = os.cpu_count()
    t0 = time.perf_counter()
    o.double_block(cfg, inp)
    dt = time.perf_counter() - t0
    return {"value": round(cfg.flops_double() / dt / 1e12, 4), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "sample": f"one full double block of {cfg.name} in float64 (numpy, {dt:.1f} s)",
            "seconds": round(dt, 2)}


if __name__ == "__main__":
    main()

"""The calibration kernels bench.py reads its ceilings from: the streaming copy must copy, the read
must visit every element (its xor-fold changes when one word does), the MFMA loop must run and
write its per-thread values."""
import pytest
import torch

from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dit():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import attention_dit_block_amd as m
    return m


def test_stream_probe_copies_and_reads_everything(dit):
    say("stream probe: copy and read of 4 MiB")
    n = 1 << 20                                    # 4 MiB of int32
    a = torch.randint(-2**31, 2**31 - 1, (n,), dtype=torch.int32, device="cuda")
    b = torch.zeros_like(a)
    dit.stream_probe(1, a, dst=b, workgroups=37)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    sink = torch.empty(64 * 256, dtype=torch.float32, device="cuda")

    def fold():
        dit.stream_probe(0, a, sink=sink, workgroups=64)
        torch.cuda.synchronize()
        return sink.view(torch.int32).clone()
    f0 = fold()
    for idx in (0, n // 3, n - 1):                  # first, middle and last word each reach the fold
        a[idx] ^= 1 << 7
        assert not torch.equal(fold(), f0)
        a[idx] ^= 1 << 7
    with pytest.raises(Exception):
        dit.stream_probe(1, a[:1000], dst=b[:1000])  # not a multiple of 16 KiB


def test_mfma_loop_runs(dit):
    out = torch.full((4 * 256,), float("nan"), dtype=torch.float32, device="cuda")
    dit.mfma_loop(4, 10, out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("mode", [0, 1, 2, 3, 8, 9])
def test_gemm_kloop_probe_closed_form(dit, mode):
    """Every staged element is 2^-6, so a k-step adds 64 * 2^-12 to each of a thread's 128
    accumulators: the per-thread sum after k steps is 2 k, exactly, in every schedule."""
    say(f"GEMM k-loop probe, mode {mode}")
    wg, ks = 5, 37
    out = torch.full((wg * 512,), float("nan"), dtype=torch.float32, device="cuda")
    win = torch.full((2 << 20,), 0.015625, dtype=torch.float16, device="cuda")
    dit.gemm_kloop_probe(mode, wg, ks, out, window=win)
    torch.cuda.synchronize()
    assert torch.equal(out, torch.full_like(out, 2.0 * ks))


@pytest.mark.parametrize("mode", [0, 1])
def test_attention_step_probe_closed_form(dit, mode):
    """With c2 = 0 every probability is 2^-1: a tile adds 32 * 2^-1 to the row sum and 64 * 2^-6 * 2^-1
    to each of a thread's 64 output accumulators, 48 per tile in all (mode 1 runs one more softmax)."""
    say(f"attention step probe, mode {mode}")
    wg, tiles = 3, 41
    out = torch.full((wg * 512,), float("nan"), dtype=torch.float32, device="cuda")
    dit.attention_step_probe(mode, wg, tiles, out)
    torch.cuda.synchronize()
    assert torch.equal(out, torch.full_like(out, 48.0 * tiles + (16.0 if mode == 1 else 0.0)))


def test_probes_random_operands_deterministic(dit):
    """With random operands (mode bit 2 / bit 1) the probes give finite sums, the same on every run."""
    say("probes with random operands")
    out = torch.empty(4 * 512, dtype=torch.float32, device="cuda")
    win = (torch.rand(2 << 20, device="cuda") * 0.25 - 0.125).to(torch.float16)
    for run in (lambda: dit.gemm_kloop_probe(6, 4, 9, out, window=win), lambda: dit.gemm_kloop_probe(4, 4, 9, out),
                lambda: dit.attention_step_probe(2, 4, 7, out, c2=0.18)):
        run()
        torch.cuda.synchronize()
        first = out.clone()
        assert torch.isfinite(first).all()
        run()
        torch.cuda.synchronize()
        assert torch.equal(out, first)


def test_probe_arguments_rejected(dit):
    out = torch.empty(512, dtype=torch.float32, device="cuda")
    small = torch.zeros(1024, dtype=torch.float16, device="cuda")
    with pytest.raises(Exception):
        dit.gemm_kloop_probe(2, 1, 1, out, window=small)       # window under 4 MiB
    with pytest.raises(Exception):
        dit.attention_step_probe(4, 1, 1, out)                  # no such mode
    with pytest.raises(Exception):
        dit.gemm_kloop_probe(10, 1, 1, out, window=small)       # registers only with global loads

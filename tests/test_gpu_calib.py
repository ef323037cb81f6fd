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

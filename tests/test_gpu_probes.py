"""The measurement probes on the GPU: the MFMA probe's accumulators reach the value its
all-ones operands fix exactly, and the copy probe copies every byte."""
import pytest

from gated_deltanet_recurrence_rule_amd import binding as G

pytestmark = pytest.mark.gpu


def test_mfma_probe_result_is_exact():
    import torch
    nwg, iters = 300, 64
    sink = torch.full((nwg * 256,), -1.0, dtype=torch.float32, device="cuda:0")
    flops = G.gdn_probe_mfma(nwg, iters, sink)
    torch.cuda.synchronize()
    assert flops == nwg * 4 * iters * 4 * 32768
    # each of a thread's 64 accumulator elements gains 16 (a dot product of 16 ones) per product
    assert torch.equal(sink.cpu(), torch.full((nwg * 256,), 64.0 * 16 * iters))


def test_copy_probe_copies_every_byte():
    import torch
    n = 3 * 32768
    g = torch.Generator(device="cuda:0")
    g.manual_seed(11)
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda:0", generator=g)
    dst = torch.zeros_like(src)
    G.gdn_probe_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src.cpu(), dst.cpu())

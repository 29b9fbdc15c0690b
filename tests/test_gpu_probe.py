"""The fp8 MFMA throughput probe and the logits-core probe (measurement helpers of the roofline
report): each runs, writes one finite value per thread and reports the flops of its launch."""

import pytest
import torch

import fp8_mqa_logits_amd as F

pytestmark = pytest.mark.gpu


def test_mfma_probe_runs_and_counts_flops():
    blocks, iters = 8, 16
    out, flops = F.fp8idx_probe_mfma_fp8(blocks, iters)
    torch.cuda.synchronize()
    assert flops == blocks * 4 * iters * 4 * 65536
    v = out.cpu()
    assert v.numel() == blocks * 256
    assert torch.isfinite(v).all() and (v > 0).all()
    # the same launch again gives the same values (register-only arithmetic)
    out2, _ = F.fp8idx_probe_mfma_fp8(blocks, iters)
    torch.cuda.synchronize()
    assert torch.equal(out2.cpu(), v)


def test_logits_core_probe_runs_and_counts_flops():
    blocks, iters = 6, 40
    out, flops = F.fp8idx_probe_logits_core(blocks, iters)
    torch.cuda.synchronize()
    assert flops == blocks * 4 * iters * 8 * 65536
    v = out.cpu()
    assert v.numel() == blocks * 256
    assert torch.isfinite(v).all() and (v != 0).any()
    out2, _ = F.fp8idx_probe_logits_core(blocks, iters)
    torch.cuda.synchronize()
    assert torch.equal(out2.cpu(), v)

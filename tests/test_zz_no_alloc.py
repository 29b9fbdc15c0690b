"""The allocation-free ragged logits entry (indexer_logits_ragged_noalloc) against the entry it
varies (indexer_logits_ragged with a caller workspace): identical bytes on consecutive calls on one
device, the second and third smaller than the first, so each call has to clear what the one before
it left in the shared static counters; plus sampled rows against the oracle."""

import numpy as np
import pytest
import torch

import fp8_mqa_logits_amd as F
from oracle import mqa_logits
from tests.parity import assert_logits_close, to_dev
from workloads.generate import ragged_inputs

pytestmark = pytest.mark.gpu


def _dev(inp):
    return [to_dev(a) for a in (inp.q, inp.kv, inp.kv_scale, inp.weights, inp.ks, inp.ke)]


def test_noalloc_matches_workspace_entry_on_consecutive_calls():
    # 600 x 12000 and 400 x 10000 both hand items out through the counters (more items than
    # resident workgroups); 40 x 3000 is covered by the fixed first items and touches no counter
    shapes = [(600, 12000, 71), (400, 10000, 72), (40, 3000, 73), (600, 12000, 74)]
    for clean in (True, False):
        for m, n, seed in shapes:
            inp = ragged_inputs(m, n, 8, seed=seed)
            d = _dev(inp)
            print(f"noalloc m={m} n={n} clean={clean}", flush=True)
            ref = torch.full((m, n + 4), 5.0, dtype=torch.float32, device="cuda")
            got = torch.full((m, n + 4), 5.0, dtype=torch.float32, device="cuda")
            F.indexer_logits_ragged(*d, clean=clean, logits=ref)
            F.indexer_logits_ragged_noalloc(*d, clean=clean, logits=got)
            torch.cuda.synchronize()
            assert torch.equal(got, ref), f"m={m} n={n} clean={clean}"
            if clean:
                rows = np.array([0, m // 3, m - 1])
                o = mqa_logits(inp.q[rows], inp.kv, inp.kv_scale, inp.weights[rows], inp.ks[rows], inp.ke[rows])
                g = got[torch.as_tensor(rows, device="cuda"), :n].cpu().numpy()
                assert_logits_close(g, o, inp.ks[rows], inp.ke[rows], clean=True, what=f"noalloc m={m}")


def test_noalloc_back_to_back_on_one_stream():
    """Calls queued one after another without a host wait: each call's clear runs after the previous
    call's kernel on the same stream."""
    a, b = ragged_inputs(600, 12000, 8, seed=75), ragged_inputs(400, 10000, 8, seed=76)
    da, db = _dev(a), _dev(b)
    ref_a = F.indexer_logits_ragged(*da, clean=True)
    ref_b = F.indexer_logits_ragged(*db, clean=True)
    outs = [torch.empty_like(ref_a if i % 2 == 0 else ref_b) for i in range(6)]
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        F.indexer_logits_ragged_noalloc(*(da if i % 2 == 0 else db), clean=True, logits=o)
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        assert torch.equal(o, ref_a if i % 2 == 0 else ref_b), f"call {i}"

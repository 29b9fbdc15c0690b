"""Parity of the HIP sparse MLA attention (the consumer of the top-k slots) with the float64 oracle.

Tolerance, from the arithmetic: the scores are exact bf16 x fp8 products summed in fp32 (the
kernel's two-part e4m3 split of q is exact for every value above 2^-10 of its 32-value block
maximum and off by at most 2^-17 of that maximum below it, far under this bound); the
probabilities enter the value product rounded to bf16 (relative error <= 2^-9 each), so
|o_gpu - o| <= 2^-9 * max |v| over the token's selected values; the test allows twice that.
lse sees only fp32 accumulation and exp / log rounding: 1e-4 + 1e-5 |lse|.
"""

import numpy as np
import pytest
import torch

import fp8_mqa_logits_amd as F
from oracle import sparse_mla
from oracle.indexer_oracle import decode_e4m3fn, paged_topk_mapped
from tests.parity import to_dev
from workloads.generate import paged_inputs, sparse_mla_inputs

pytestmark = pytest.mark.gpu


def _run(inp, want_lse=True):
    q = torch.from_numpy(inp.q_bits.view(np.int16)).cuda()
    kv = to_dev(inp.kv_codes)
    sc = to_dev(inp.kv_scale)
    idx = to_dev(inp.indices)
    out, lse = F.indexer_sparse_mla(q, kv, sc, idx, inp.sm_scale, want_lse=want_lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (lse.cpu().numpy() if lse is not None else None)


def _check(inp, o_gpu, lse_gpu, tokens, what):
    o_ref, lse_ref = sparse_mla(inp.q_bits, inp.kv_codes, inp.kv_scale, inp.indices, inp.sm_scale, tokens=tokens)
    S = inp.kv_codes.shape[0]
    for n, t in enumerate(tokens):
        idx = inp.indices[t]
        sel = idx[(idx >= 0) & (idx < S)]
        vmax = float(np.abs(decode_e4m3fn(inp.kv_codes[sel, :512]) * inp.kv_scale[sel, None]).max()) if sel.size else 0.0
        tol = 2.0 * 2.0 ** -9 * vmax + 1e-6
        d = np.abs(o_gpu[t] - o_ref[n])
        assert d.max() <= tol, f"{what} token {t}: max |do| {d.max():.3e} > {tol:.3e}"
        if lse_gpu is not None:
            lr, lg = lse_ref[n], lse_gpu[t]
            fin = np.isfinite(lr)
            assert np.array_equal(fin, np.isfinite(lg)), f"{what} token {t}: lse finiteness"
            assert np.all(lg[~fin] == -np.inf)
            dl = np.abs(lg[fin] - lr[fin])
            assert np.all(dl <= 1e-4 + 1e-5 * np.abs(lr[fin])), f"{what} token {t}: lse {dl.max():.3e}"


@pytest.mark.parametrize("T,H,S,topk,inval,dup", [
    (1, 16, 300, 64, 0, 0),        # one step, one head tile, split into nothing
    (3, 64, 500, 100, 7, 3),       # ragged top-k (two steps, the second partial), padding, repeats
    (2, 32, 1000, 256, 0, 0),      # two head tiles of a block
    (5, 128, 2000, 512, 40, 5),    # two head blocks
    (4, 48, 3000, 2048, 300, 0),   # many splits (few tokens): the combine kernel
    (1, 64, 200, 2048, 0, 0),      # topk > S: slots repeat
])
def test_sparse_mla_vs_oracle(T, H, S, topk, inval, dup):
    inp = sparse_mla_inputs(T, H, S, topk, seed=T * 100 + H + topk, invalid_tail=inval, duplicates=dup)
    o, lse = _run(inp)
    _check(inp, o, lse, list(range(T)), f"T{T} H{H} S{S} k{topk}")


def test_no_valid_slot_and_single_slot():
    inp = sparse_mla_inputs(3, 16, 400, 192, seed=7)
    inp.indices[0, :] = -1                      # nothing valid: o = 0, lse = -inf
    inp.indices[1, :] = np.where(np.arange(192) == 77, 5, -1)   # exactly one slot
    inp.indices[2, 100:] = 400 + np.arange(92)  # past the pool: skipped
    o, lse = _run(inp)
    assert np.all(o[0] == 0.0) and np.all(lse[0] == -np.inf)
    _check(inp, o, lse, [0, 1, 2], "edge slots")


def test_zero_scales_count_in_the_softmax():
    inp = sparse_mla_inputs(2, 32, 600, 128, seed=9)
    inp.kv_scale[inp.indices[0, :40]] = 0.0     # valid slots with a zero scale: score 0, value 0
    o, lse = _run(inp)
    _check(inp, o, lse, [0, 1], "zero scales")


def test_lse_is_optional_and_bytes_match():
    inp = sparse_mla_inputs(2, 64, 800, 320, seed=11, invalid_tail=20)
    o1, lse1 = _run(inp)
    o2, none = _run(inp, want_lse=False)
    assert none is None
    assert np.array_equal(o1, o2)               # deterministic, and lse does not change o


def test_full_decode_shape_sampled():
    """256 tokens (64 requests x 4 rows) x 64 heads over 2048 slots each: one workgroup per token,
    no split.  Sampled tokens against the oracle."""
    inp = sparse_mla_inputs(256, 64, 300000, 2048, seed=12, invalid_tail=0)
    o, lse = _run(inp)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    _check(inp, o, lse, [0, 1, 77, 128, 200, 255], "decode 256x64x2048")


def test_chained_after_the_oracle_top_k():
    """The indexer's top-k physical slots (computed by the oracle on a paged decode input) select the
    MLA rows: the pool holds one MLA row per physical slot of the indexer's pages."""
    pin = paged_inputs(3, 4, 300, 900, 128, seed=13, page_size=64)
    width = pin.max_pages * 64
    _, _, slots = paged_topk_mapped(pin, width=width)       # [rows, k] physical slot ids, -1 padded
    S = pin.kv_pool.shape[0] * 64
    mla = sparse_mla_inputs(slots.shape[0], 64, S, slots.shape[1], seed=14)
    mla.indices[:] = slots.astype(np.int32)
    o, lse = _run(mla)
    _check(mla, o, lse, list(range(slots.shape[0])), "chained")


def test_q_blocks_of_very_different_magnitudes():
    """q scaled by 2^-u per 16-value group (u in 0..16, exact in bf16): the per-block exponents of
    the fp8 score path differ from block to block and between the two halves of a block, which
    pins the block-to-scale-lane layout of the scaled MFMA."""
    import dataclasses
    inp = sparse_mla_inputs(3, 64, 700, 256, seed=11)
    rng = np.random.default_rng(11)
    qf = (inp.q_bits.astype(np.uint32) << 16).view(np.float32)
    T, H, D = qf.shape
    u = rng.integers(0, 17, size=(T, H, D // 16))
    qf = qf * np.repeat(np.exp2(-u.astype(np.float64)), 16, axis=2).astype(np.float32)
    q_bits = np.ascontiguousarray((qf.view(np.uint32) >> 16).astype(np.uint16))
    assert np.array_equal((q_bits.astype(np.uint32) << 16).view(np.float32), qf)   # exact in bf16
    inp = dataclasses.replace(inp, q_bits=q_bits)
    o, lse = _run(inp)
    _check(inp, o, lse, [0, 1, 2], "q block magnitudes")


def test_more_splits_than_one_combine_chunk():
    """540000 slots for one token: 2048-slot splits give 264 of them, more than the 256 split
    weights the combine holds in LDS at once, so the combine runs in two chunks."""
    inp = sparse_mla_inputs(1, 16, 500, 540000, seed=21)
    assert F.fp8idx_sparse_mla_workspace_bytes(1, 16, 540000) == 264 * 16 * 513 * 4 + 256
    o, lse = _run(inp)
    _check(inp, o, lse, [0], "264 splits")

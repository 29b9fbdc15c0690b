"""Full-size parity that reaches every work item.

The ragged logits kernel hands its (16-row block, key slice) items out from device-side
queues that steal from each other, so a dropped or doubled item would leave some rows
wrong while most stay right.  These tests therefore look at every row block:

* one row of every 16-row block (its offset inside the block cycling through 0..15) of
  the full-size launches, compared element by element with the float64 oracle, with
  both top-k checks (tolerant against the oracle, exact on the device's own logits);
* a sentinel fill that proves, on the device and for every row, that each in-window
  logit was written and nothing outside the window was (clean = 0 writes only the
  window);
* the 256 paged decode rows, all of them, against the oracle;
* the overlapped chunk loop against the oracle.
"""

import numpy as np
import pytest
import torch

import fp8_mqa_logits_amd as F
from oracle import map_block_table, mqa_logits, paged_topk_mapped, topk_indices
from tests.parity import assert_logits_close, assert_topk_exact, assert_topk_tolerant, to_dev
from workloads.generate import config_inputs, ragged_inputs

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FBADBAD   # a NaN bit pattern no kernel computes


def _dev(inp):
    return [to_dev(a) for a in (inp.q, inp.kv, inp.kv_scale, inp.weights, inp.ks, inp.ke)]


def _block_rows(m, block=16):
    """One row of each block of 16 rows; the offset inside the block cycles through 0..15."""
    nb = (m + block - 1) // block
    return np.array([min(m - 1, b * block + (b % block)) for b in range(nb)], dtype=np.int64)


def _gather_rows(t, rows):
    return t[torch.as_tensor(rows, device=t.device)].cpu().numpy()


def _check_ragged_rows(inp, rows, g_logits, sel, what):
    o = mqa_logits(inp.q[rows], inp.kv, inp.kv_scale, inp.weights[rows], inp.ks[rows], inp.ke[rows])
    assert_logits_close(g_logits, o, inp.ks[rows], inp.ke[rows], clean=True, what=what)
    assert_topk_tolerant(sel, o, inp.ks[rows], inp.ke[rows], inp.k, what=what)
    exact = topk_indices(g_logits.astype(np.float64), inp.ks[rows], inp.ke[rows], inp.k)
    assert_topk_exact(sel, exact, what=what)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["prefill_64k", "prefill_35k"])
def test_full_prefill_every_row_block(name):
    """One launch at the full shape; 512 rows (one per 16-row block) element by element; the
    fused one-shot top-k of the same rows."""
    inp = config_inputs(name)
    d = _dev(inp)
    rows = _block_rows(inp.m)
    print(f"{name}: logits launch {inp.m} x {inp.n}, {rows.size} rows checked", flush=True)
    g = F.indexer_logits_ragged(*d, clean=True)
    torch.cuda.synchronize()
    got = _gather_rows(g, rows)
    del g
    torch.cuda.empty_cache()
    out = F.indexer_logits_topk_ragged(*d, inp.k)
    torch.cuda.synchronize()
    _check_ragged_rows(inp, rows, got, out.cpu().numpy()[rows], what=f"{name} full launch")


@pytest.mark.timeout(900)
def test_long_prefix_fused_every_row_block():
    """The 7500 x 210000 long prefix through the fused entry under the 2e9-byte cap (4 chunks) and
    through the overlapped entry: one row per 16-row block of every chunk's logits launch, element
    by element, and both top-k checks on the fused output."""
    inp = config_inputs("long_prefix_210k")
    d = _dev(inp)
    cap = inp.cap_bytes
    rpc = F.fp8idx_rows_per_chunk(cap, inp.n, inp.m)
    assert rpc == 2380
    print(f"long prefix: fused {inp.m} x {inp.n} in chunks of {rpc}", flush=True)
    out = F.indexer_logits_topk_ragged(*d, inp.k, logits_cap_bytes=cap)
    side = torch.cuda.Stream()
    over = F.indexer_logits_topk_ragged_overlap(*d, inp.k, side_stream=side, logits_cap_bytes=cap)
    torch.cuda.synchronize()
    assert torch.equal(out, over), "overlapped loop differs from the serial loop"
    # the chunk launches the fused entry makes, one at a time, to read their logits
    rows = _block_rows(inp.m)
    ld = (inp.n + 3) // 4 * 4
    buf = torch.empty((rpc, ld), dtype=torch.float32, device="cuda")
    got = np.empty((rows.size, inp.n), dtype=np.float32)
    q, kv, sc, w, ks, ke = d
    for s0 in range(0, inp.m, rpc):
        e0 = min(inp.m, s0 + rpc)
        F.indexer_logits_ragged(q[s0:e0], kv, sc, w[s0:e0], ks[s0:e0], ke[s0:e0], clean=True, logits=buf[:e0 - s0])
        torch.cuda.synchronize()
        pick = np.nonzero((rows >= s0) & (rows < e0))[0]
        got[pick] = _gather_rows(buf, rows[pick] - s0)[:, :inp.n]
    del buf
    torch.cuda.empty_cache()
    _check_ragged_rows(inp, rows, got, out.cpu().numpy()[rows], what="long prefix fused")


def _sentinel_check_ragged(inp, d, r0, r1):
    """Logits of rows [r0, r1) into a sentinel-filled buffer with clean = 0: every in-window
    element changed (and finite), every other element still the sentinel."""
    q, kv, sc, w, ks, ke = d
    m = r1 - r0
    ld = (inp.n + 3) // 4 * 4 + 4          # a wider row stride: columns past n must stay untouched too
    lg = torch.empty((m, ld), dtype=torch.float32, device="cuda")
    lg.view(torch.int32).fill_(SENTINEL)
    F.indexer_logits_ragged(q[r0:r1], kv, sc, w[r0:r1], ks[r0:r1], ke[r0:r1], clean=False, logits=lg)
    torch.cuda.synchronize()
    cols = torch.arange(ld, device="cuda", dtype=torch.int32)
    ks_d, ke_d = ks[r0:r1], ke[r0:r1]
    missing = untouched_bad = 0
    for a in range(0, m, 256):
        b = min(m, a + 256)
        blk = lg[a:b]
        inside = (cols[None, :] >= ks_d[a:b, None]) & (cols[None, :] < ke_d[a:b, None])
        is_sent = blk.view(torch.int32) == SENTINEL
        missing += int((inside & (is_sent | ~torch.isfinite(blk))).sum())
        untouched_bad += int((~inside & ~is_sent).sum())
    del lg
    torch.cuda.empty_cache()
    assert missing == 0, f"rows [{r0}, {r1}): {missing} in-window logits not written"
    assert untouched_bad == 0, f"rows [{r0}, {r1}): {untouched_bad} logits written outside the window"


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,r0,r1", [("prefill_64k", 0, 8192), ("prefill_35k", 0, 8192),
                                        ("long_prefix_210k", 0, 2380), ("long_prefix_210k", 2380, 4760),
                                        ("long_prefix_210k", 7140, 7500), ("tiny", 0, 64)])
def test_every_window_logit_written_exactly(name, r0, r1):
    inp = config_inputs(name)
    print(f"{name} rows [{r0}, {r1}): sentinel fill, clean = 0", flush=True)
    _sentinel_check_ragged(inp, _dev(inp), r0, r1)


def test_sentinel_ragged_windows_of_every_shape():
    """The same completeness check on random windows (empty, one key, full, ragged starts) over
    shapes with a ragged key tail and a partial last row block, several launches in a row."""
    rng = np.random.default_rng(17)
    for m, n in ((1, 17), (37, 1000), (300, 5000), (1000, 2100), (513, 20001)):
        ks = rng.integers(0, n, m)
        ke = np.minimum(n, ks + rng.integers(0, n + 1, m))
        ks[0], ke[0] = 0, n
        if m > 2:
            ks[1], ke[1] = 5 % n, 5 % n
            ks[2], ke[2] = n - 1, n
        inp = ragged_inputs(m, n, 8, seed=m + n, ks=ks.astype(np.int32), ke=ke.astype(np.int32))
        _sentinel_check_ragged(inp, _dev(inp), 0, m)


@pytest.mark.timeout(600)
def test_paged_decode_every_row():
    """All 256 decode rows: logits element by element, top-k (tolerant and exact), physical slots;
    and a sentinel fill showing clean = 0 writes exactly each row's window."""
    inp = config_inputs("paged_decode")
    width = inp.max_pages * 64
    args = [to_dev(a) for a in (inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len, inp.block_table)]
    slots = F.indexer_logits_topk_paged(*args, inp.k, width=width)
    raw = F.indexer_logits_topk_paged(*args, inp.k, width=width, map_to_slots=False)
    logits = F.indexer_logits_paged(*args, width=width, clean=True)
    lg = torch.empty((inp.rows, width), dtype=torch.float32, device="cuda")
    lg.view(torch.int32).fill_(SENTINEL)
    F.indexer_logits_paged(*args, width=width, clean=False, logits=lg)
    torch.cuda.synchronize()
    cols = torch.arange(width, device="cuda", dtype=torch.int32)
    inside = cols[None, :] < args[4][:, None]
    is_sent = lg.view(torch.int32) == SENTINEL
    assert int((inside & is_sent).sum()) == 0, "paged: in-window logits not written"
    assert int((~inside & ~is_sent).sum()) == 0, "paged: logits written outside the window"
    del lg, is_sent, inside
    rows = list(range(inp.rows))
    print(f"paged decode: oracle over all {inp.rows} rows", flush=True)
    L, _, _ = paged_topk_mapped(inp, width=width)
    g = logits.cpu().numpy().astype(np.float64)
    zeros = np.zeros(inp.rows, np.int64)
    assert_logits_close(g, L, zeros, inp.row_len, clean=True, what="paged all rows")
    r = raw.cpu().numpy()
    assert_topk_tolerant(r, L, zeros, inp.row_len, inp.k, what="paged all rows")
    exact = topk_indices(g, zeros, inp.row_len, inp.k)
    assert_topk_exact(r, exact, what="paged all rows")
    want = map_block_table(exact, rows, inp.next_n, inp.block_table, 64, inp.kv_pool.shape[0])
    got = slots.cpu().numpy()
    for i in rows:
        assert set(got[i].tolist()) == set(want[i].tolist()), f"paged slots row {i}"


@pytest.mark.parametrize("cap_rows", [1, 37, 100, 700])
def test_overlap_against_oracle(cap_rows):
    """The overlapped loop (top-k of chunk N - 1 on a side stream during chunk N's logits) against
    the oracle directly, over 700 causal rows of 30000 keys, from 700 chunks down to one."""
    inp = ragged_inputs(700, 30000, 2048, seed=61)
    d = _dev(inp)
    ld = (inp.n + 3) // 4 * 4
    side = torch.cuda.Stream()
    got = F.indexer_logits_topk_ragged_overlap(*d, inp.k, side_stream=side, logits_cap_bytes=cap_rows * ld * 4)
    g_logits = F.indexer_logits_ragged(*d, clean=True)
    torch.cuda.synchronize()
    rows = np.arange(inp.m) if cap_rows == 100 else _block_rows(inp.m, 7)
    g = _gather_rows(g_logits, rows)
    _check_ragged_rows(inp, rows, g, got.cpu().numpy()[rows], what=f"overlap cap {cap_rows} rows")

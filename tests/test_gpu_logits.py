"""Parity of the HIP logits kernels (ragged prefill and paged decode) with the float64 oracle."""

import numpy as np
import pytest
import torch

import fp8_mqa_logits_amd as F
from oracle import mqa_logits, paged_mqa_logits
from tests.parity import assert_logits_close, cancellation_tol, to_dev
from workloads.generate import H, D, config_inputs, ragged_inputs, multi_request_ragged, paged_inputs

pytestmark = pytest.mark.gpu


def _ragged_dev(inp):
    return [to_dev(a) for a in (inp.q, inp.kv, inp.kv_scale, inp.weights, inp.ks, inp.ke)]


def _run_ragged(inp, clean=True, ld=None):
    q, kv, sc, w, ks, ke = _ragged_dev(inp)
    out = None
    if ld is not None:
        out = torch.full((inp.m, ld), 12345.0, dtype=torch.float32, device="cuda")
    g = F.indexer_logits_ragged(q, kv, sc, w, ks, ke, clean=clean, logits=out)
    torch.cuda.synchronize()
    return g.cpu().numpy()


def test_tiny_config_all_rows():
    inp = ragged_inputs(64, 4096, 512, seed=1)
    g = _run_ragged(inp)
    o = mqa_logits(inp.q, inp.kv, inp.kv_scale, inp.weights, inp.ks, inp.ke)
    assert_logits_close(g, o, inp.ks, inp.ke, clean=True, what="tiny m64 n4096")


def _random_windows(rng, m, n):
    ks = rng.integers(0, n, m)
    ke = np.minimum(n, ks + rng.integers(0, n, m))
    # a few special windows: empty, full, single key, last key
    ks[0], ke[0] = 0, n
    if m > 1:
        ks[1], ke[1] = 3 % n, 3 % n
    if m > 2:
        ks[2], ke[2] = n - 1, n
    if m > 3:
        ks[3], ke[3] = 0, 1
    return ks.astype(np.int32), ke.astype(np.int32)


def test_ragged_repeats_streams_and_graph_replays():
    """Workgroups claim items from a per-stream device work queue that each launch resets when it ends:
    back-to-back launches, launches on two streams at once and graph replays between eager launches
    must all give the same bytes."""
    rng = np.random.default_rng(77)
    ks1, ke1 = _random_windows(rng, 300, 5000)
    a = ragged_inputs(300, 5000, 8, seed=78, ks=ks1, ke=ke1)
    b = ragged_inputs(1000, 2100, 8, seed=79)
    da, db = _ragged_dev(a), _ragged_dev(b)
    ref_a = F.indexer_logits_ragged(*da, clean=True)
    ref_b = F.indexer_logits_ragged(*db, clean=True)
    torch.cuda.synchronize()
    assert_logits_close(ref_a.cpu().numpy(), mqa_logits(a.q, a.kv, a.kv_scale, a.weights, a.ks, a.ke),
                        a.ks, a.ke, clean=True, what="queue a")
    assert_logits_close(ref_b.cpu().numpy(), mqa_logits(b.q, b.kv, b.kv_scale, b.weights, b.ks, b.ke),
                        b.ks, b.ke, clean=True, what="queue b")
    for rep in range(3):
        out = F.indexer_logits_ragged(*da, clean=True)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_a), f"repeat {rep}"
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    torch.cuda.synchronize()
    for rep in range(3):
        with torch.cuda.stream(s1):
            oa = F.indexer_logits_ragged(*da, clean=True)
        with torch.cuda.stream(s2):
            ob = F.indexer_logits_ragged(*db, clean=True)
        outs.append((oa, ob))
    torch.cuda.synchronize()
    for rep, (oa, ob) in enumerate(outs):
        assert torch.equal(oa, ref_a) and torch.equal(ob, ref_b), f"two streams, round {rep}"
    sg = torch.cuda.Stream()
    static_out = torch.empty_like(ref_a)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=sg):
        F.indexer_logits_ragged(*da, clean=True, logits=static_out)
    for rep in range(3):
        static_out.fill_(7.0)
        g.replay()
        eager = F.indexer_logits_ragged(*db, clean=True)
        torch.cuda.synchronize()
        assert torch.equal(static_out, ref_a), f"graph replay {rep}"
        assert torch.equal(eager, ref_b), f"eager launch after replay {rep}"


@pytest.mark.parametrize("name", ["prefill_64k", "prefill_35k"])
def test_full_size_ragged_logits_sampled_rows(name):
    """One launch at the full prefill shape (every workgroup resident, work handed out by the device
    queues, queues stealing from each other at the end): sampled rows of its output, element by element,
    against the oracle, with clean set so the -inf outside each window is checked too."""
    inp = config_inputs(name)
    d = _ragged_dev(inp)
    g = F.indexer_logits_ragged(*d, clean=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    # first and last rows, both rows of every 16-row block edge sampled, and random rows
    rows = sorted({0, 1, 15, 16, 4095, 4096, inp.m - 17, inp.m - 16, inp.m - 1} |
                  set(rng.integers(0, inp.m, 5).tolist()))
    ridx = np.array(rows)
    got = g[torch.as_tensor(ridx, device=g.device)].cpu().numpy()
    del g
    o = mqa_logits(inp.q[ridx], inp.kv, inp.kv_scale, inp.weights[ridx], inp.ks[ridx], inp.ke[ridx])
    assert_logits_close(got, o, inp.ks[ridx], inp.ke[ridx], clean=True, what=f"{name} full launch")


@pytest.mark.parametrize("m,n", [(1, 17), (5, 64), (16, 65), (37, 1000), (50, 3000), (33, 4133)])
@pytest.mark.parametrize("clean", [True, False])
def test_ragged_shapes_and_windows(m, n, clean):
    rng = np.random.default_rng(m * 1000 + n)
    ks, ke = _random_windows(rng, m, n)
    inp = ragged_inputs(m, n, 8, seed=m + n, ks=ks, ke=ke)
    g = _run_ragged(inp, clean=clean)
    o = mqa_logits(inp.q, inp.kv, inp.kv_scale, inp.weights, inp.ks, inp.ke)
    assert_logits_close(g, o, inp.ks, inp.ke, clean=clean, what=f"m{m} n{n} clean{clean}")


def test_ld_wider_than_n_leaves_tail_untouched():
    inp = ragged_inputs(20, 700, 8, seed=3)
    g = _run_ragged(inp, clean=True, ld=720)
    o = mqa_logits(inp.q, inp.kv, inp.kv_scale, inp.weights, inp.ks, inp.ke)
    assert_logits_close(g[:, :700], o, inp.ks, inp.ke, clean=True, what="ld 720")
    assert np.all(g[:, 700:] == 12345.0)


def test_multi_request_rows():
    inp = multi_request_ragged([(300, 7), (1200, 20), (65, 3), (2048, 33)], k=16, seed=5)
    g = _run_ragged(inp)
    o = mqa_logits(inp.q, inp.kv, inp.kv_scale, inp.weights, inp.ks, inp.ke)
    assert_logits_close(g, o, inp.ks, inp.ke, clean=True, what="multi-request")


def test_signed_weights():
    inp = ragged_inputs(24, 900, 8, seed=6, weight_mode="signed")
    g = _run_ragged(inp)
    o = mqa_logits(inp.q, inp.kv, inp.kv_scale, inp.weights, inp.ks, inp.ke)
    extra = cancellation_tol(inp.q, inp.kv, inp.kv_scale, inp.weights, np.arange(24), 0, 900)
    assert_logits_close(g, o, inp.ks, inp.ke, clean=True, extra_tol=extra, what="signed weights")


@pytest.mark.parametrize("mode", ["zero_scale", "zero_weights"])
def test_zero_scale_or_weights(mode):
    kw = {"scale_mode": "zero"} if mode == "zero_scale" else {"weight_mode": "zero"}
    inp = ragged_inputs(18, 300, 8, seed=7, **kw)
    g = _run_ragged(inp)
    inside = np.isfinite(mqa_logits(inp.q, inp.kv, inp.kv_scale, inp.weights, inp.ks, inp.ke))
    assert np.all(g[inside] == 0.0)


def test_extreme_codes_no_overflow():
    # largest e4m3fn magnitudes: dot = 448*448*128 ~ 2.6e7 per head, well inside fp32
    inp = ragged_inputs(4, 128, 8, seed=8)
    inp.q[:] = 0x7E
    inp.kv[:, :] = 0x7E
    inp.kv[::2, ::2] = 0xFE
    g = _run_ragged(inp)
    o = mqa_logits(inp.q, inp.kv, inp.kv_scale, inp.weights, inp.ks, inp.ke)
    assert_logits_close(g, o, inp.ks, inp.ke, clean=True, what="extreme codes")


def test_rows_independent_of_batching():
    # the value of (i, j) must not depend on which rows share a workgroup or key split
    inp = ragged_inputs(40, 5000, 8, seed=9)
    full = _run_ragged(inp)
    rows = np.array([3, 17, 39])
    q, kv, sc, w, ks, ke = _ragged_dev(inp)
    sub = F.indexer_logits_ragged(q[rows], kv, sc, w[rows], ks[rows], ke[rows], clean=True)
    torch.cuda.synchronize()
    assert np.array_equal(sub.cpu().numpy(), full[rows])


# ---------------------------------------------------------------------------
# paged decode
# ---------------------------------------------------------------------------

def _run_paged(inp, width, clean=True, block_table=None):
    bt = inp.block_table if block_table is None else block_table
    args = [to_dev(a) for a in (inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len, bt)]
    g = F.indexer_logits_paged(*args, width=width, clean=clean)
    torch.cuda.synchronize()
    return g.cpu().numpy()


@pytest.mark.parametrize("B,next_n", [(3, 4), (2, 1), (2, 2), (3, 5), (1, 8)])
def test_paged_vs_oracle(B, next_n):
    inp = paged_inputs(B, next_n, 70, 2600, 16, seed=B * 10 + next_n, page_size=64)
    width = int(inp.row_len.max())
    g = _run_paged(inp, width)
    o = paged_mqa_logits(inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len,
                         inp.block_table, inp.page_size, width=width)
    assert_logits_close(g, o, np.zeros(inp.rows, np.int64), inp.row_len, clean=True,
                        what=f"paged B{B} next_n{next_n}")


def test_paged_width_past_lengths_is_neg_inf():
    inp = paged_inputs(2, 4, 500, 900, 16, seed=31, page_size=64)
    width = inp.max_pages * 64
    g = _run_paged(inp, width)
    o = paged_mqa_logits(inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len,
                         inp.block_table, inp.page_size, width=width)
    assert_logits_close(g, o, np.zeros(inp.rows, np.int64), inp.row_len, clean=True, what="paged wide")


def test_paged_invalid_page_ids_are_masked():
    inp = paged_inputs(2, 4, 600, 700, 16, seed=32, page_size=64)
    bt = inp.block_table.copy()
    bt[0, 2] = -5                   # negative id
    bt[1, 1] = inp.kv_pool.shape[0] + 3   # past the pool
    width = int(inp.row_len.max())
    g = _run_paged(inp, width, block_table=bt)
    o = paged_mqa_logits(inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len,
                         inp.block_table, inp.page_size, width=width)
    for r in range(inp.rows):
        b = r // 4
        bad_page = 2 if b == 0 else 1
        cols = np.arange(width)
        masked = (cols // 64 == bad_page)
        assert np.all(g[r, masked] == -np.inf)
        keep = ~masked & (cols < inp.row_len[r])
        d = np.abs(g[r, keep] - o[r, keep])
        assert np.all(d <= 1e-3 + 2e-3 * np.abs(o[r, keep]))


@pytest.mark.parametrize("B,next_n", [(150, 1), (70, 3), (40, 6)])
def test_paged_many_units_and_empty_rows(B, next_n):
    """More (request, 4-row group) units than one wave-wide scan covers, with empty and one-key
    contexts mixed in, so the persistent grid's page ranges start and end inside units and skip
    units that own no pages."""
    rng = np.random.default_rng(B * 7 + next_n)
    ctx = rng.integers(0, 700, B)
    ctx[rng.random(B) < 0.2] = 0
    ctx[::17] = 1
    ctx[0] = 700
    inp = paged_inputs(B, next_n, 0, 700, 16, seed=40 + B, page_size=64, ctx=ctx)
    width = inp.max_pages * 64
    g = _run_paged(inp, width)
    o = paged_mqa_logits(inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len,
                         inp.block_table, inp.page_size, width=width)
    assert_logits_close(g, o, np.zeros(inp.rows, np.int64), inp.row_len, clean=True,
                        what=f"paged many units B{B} next_n{next_n}")


def test_paged_clean_false_writes_only_inside_width():
    """clean=0: [0, row_len) matches the oracle, [row_len, width) holds -inf or the old value,
    and nothing at or past the width is touched."""
    inp = paged_inputs(6, 4, 100, 1500, 16, seed=41, page_size=64)
    width = inp.max_pages * 64
    ld = width + 36
    args = [to_dev(a) for a in (inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len, inp.block_table)]
    out = torch.full((inp.rows, ld), 12345.0, dtype=torch.float32, device="cuda")
    F.indexer_logits_paged(*args, width=width, clean=False, logits=out)
    torch.cuda.synchronize()
    g = out.cpu().numpy()
    o = paged_mqa_logits(inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len,
                         inp.block_table, inp.page_size, width=width)
    for r in range(inp.rows):
        n = int(inp.row_len[r])
        d = np.abs(g[r, :n] - o[r, :n])
        assert np.all(d <= 1e-3 + 2e-3 * np.abs(o[r, :n])), r
        tail = g[r, n:width]
        assert np.all((tail == 12345.0) | (tail == -np.inf)), r
        assert np.all(g[r, width:] == 12345.0), r


def test_paged_long_contexts_many_pages_per_wave():
    """Contexts of 120K-131K keys for 96 requests: every wave of the persistent grid takes far
    more than 64 pages, so page ids are read in several segments.  Pages are drawn with
    repetition from a small pool (the kernel does not need distinct pages); sampled rows are
    checked against the oracle over the full width."""
    import dataclasses
    B, nn = 96, 2
    base = paged_inputs(B, nn, 4096, 4096, 16, seed=42, page_size=64)
    rng = np.random.default_rng(42)
    ctx = rng.integers(120000, 131073, B)
    max_pages = 2048
    P = base.kv_pool.shape[0]
    bt = rng.integers(0, P, (B, max_pages)).astype(np.int32)
    pages = (ctx + 63) // 64
    for b in range(B):
        bt[b, pages[b]:] = -1
    row_len = np.array([ctx[b] - nn + r + 1 for b in range(B) for r in range(nn)], np.int32)
    inp = dataclasses.replace(base, ctx=ctx.astype(np.int32), row_len=row_len, block_table=bt)
    width = max_pages * 64
    args = [to_dev(a) for a in (inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len, inp.block_table)]
    g = F.indexer_logits_paged(*args, width=width, clean=True)
    torch.cuda.synchronize()
    rows = [0, 1, 77, 150, 190, 191]
    L = paged_mqa_logits(inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len,
                         inp.block_table, inp.page_size, width=width, rows=rows)
    gs = g.cpu().numpy()[np.array(rows)]
    assert_logits_close(gs, L, np.zeros(len(rows), np.int64), row_len[np.array(rows)], clean=True,
                        what="paged long contexts")


def test_paged_equals_ragged_on_gathered_kv():
    inp = paged_inputs(2, 4, 900, 1500, 16, seed=33, page_size=64)
    width = int(inp.row_len.max())
    g = _run_paged(inp, width)
    for b in range(inp.B):
        n_b = int(inp.ctx[b])
        pages = (n_b + 63) // 64
        kv = inp.kv_pool[inp.block_table[b, :pages]].reshape(-1, D)[:n_b]
        sc = inp.scale_pool[inp.block_table[b, :pages]].reshape(-1)[:n_b]
        rows = slice(b * 4, b * 4 + 4)
        q = inp.q[b]
        gr = F.indexer_logits_ragged(to_dev(q), to_dev(kv), to_dev(sc), to_dev(inp.weights[rows]),
                                     to_dev(np.zeros(4, np.int32)), to_dev(inp.row_len[rows]), clean=True)
        torch.cuda.synchronize()
        # same per-(row, key) arithmetic, so the two forms agree bit for bit
        assert np.array_equal(gr.cpu().numpy(), g[rows, :n_b])


@pytest.mark.parametrize("clean", [False, True])
def test_paged_store_paths_agree(clean):
    """The paged kernel stores a page's logits 16 bytes per lane when the rows are 16-byte aligned
    and one key at a time otherwise.  Aligned rows, an odd row stride and a base 4 bytes past
    alignment must give the same bits inside every window and the same contract outside it
    (clean=0: nothing at or past row_len written; clean=1: -inf up to the width, nothing past it)."""
    inp = paged_inputs(5, 4, 100, 1500, 16, seed=43, page_size=64)
    width = inp.max_pages * 64 - 20        # not a whole number of pages
    args = [to_dev(a) for a in (inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len, inp.block_table)]
    o = paged_mqa_logits(inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len,
                         inp.block_table, inp.page_size, width=width)
    got = []
    for ld, shift in ((width + 36, 0), (width + 33, 0), (width + 36, 1)):
        flat = torch.full((inp.rows * ld + 4,), 12345.0, dtype=torch.float32, device="cuda")
        out = flat[shift:shift + inp.rows * ld].view(inp.rows, ld)
        F.indexer_logits_paged(*args, width=width, clean=clean, logits=out)
        torch.cuda.synchronize()
        g = out.cpu().numpy()
        for r in range(inp.rows):
            n = min(int(inp.row_len[r]), width)
            d = np.abs(g[r, :n] - o[r, :n])
            assert np.all(d <= 1e-3 + 2e-3 * np.abs(o[r, :n])), (ld, shift, r)
            tail = g[r, n:width]
            if clean:
                assert np.all(tail == -np.inf), (ld, shift, r)
            else:
                assert np.all((tail == 12345.0) | (tail == -np.inf)), (ld, shift, r)
            assert np.all(g[r, width:] == 12345.0), (ld, shift, r)
        got.append([g[r, :min(int(inp.row_len[r]), width)].copy() for r in range(inp.rows)])
    for other in got[1:]:
        for a, b in zip(got[0], other):
            assert np.array_equal(a, b)


@pytest.mark.parametrize("clean", [False, True])
def test_paged_large_chunk_path(clean):
    """Block tables that can name at least 131072 pages in total take 16-page chunks; smaller ones
    take 4-page chunks.  128 one-row requests with a 1024-page table and a 65536-key width take the
    large chunks (aligned rows and an odd stride, so both store forms); the same rows over a
    narrower table take the small chunks.  Every row against the oracle, and the in-window bits of
    all forms equal."""
    B = 128
    inp = paged_inputs(B, 1, 100, 3000, 16, seed=44, page_size=64)
    bt = np.full((B, 1024), -1, dtype=np.int32)
    bt[:, :inp.block_table.shape[1]] = inp.block_table
    width = 1024 * 64
    args = [to_dev(a) for a in (inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len, bt)]
    o = paged_mqa_logits(inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len,
                         inp.block_table, inp.page_size, width=int(inp.row_len.max()))
    got = []
    for ld in (width, width + 33):
        out = torch.full((inp.rows, ld), 12345.0, dtype=torch.float32, device="cuda")
        F.indexer_logits_paged(*args, width=width, clean=clean, logits=out)
        torch.cuda.synchronize()
        g = out.cpu().numpy()
        for r in range(inp.rows):
            n = int(inp.row_len[r])
            d = np.abs(g[r, :n] - o[r, :n])
            assert np.all(d <= 1e-3 + 2e-3 * np.abs(o[r, :n])), (ld, r)
            tail = g[r, n:width]
            if clean:
                assert np.all(tail == -np.inf), (ld, r)
            else:
                assert np.all((tail == 12345.0) | (tail == -np.inf)), (ld, r)
            assert np.all(g[r, width:] == 12345.0), (ld, r)
        got.append(g)
    # the narrow table (the requests' own pages only) runs the 4-page chunks
    narrow = inp.block_table.shape[1] * 64
    small = F.indexer_logits_paged(*[to_dev(a) for a in (inp.q, inp.kv_pool, inp.scale_pool, inp.weights,
                                                        inp.row_len, inp.block_table)], width=narrow, clean=clean)
    torch.cuda.synchronize()
    s = small.cpu().numpy()
    for r in range(inp.rows):
        n = int(inp.row_len[r])
        assert np.array_equal(got[0][r, :n], got[1][r, :n]), r
        assert np.array_equal(got[0][r, :n], s[r, :n]), r


@pytest.mark.parametrize("clean", [False, True])
def test_paged_large_chunk_path_many_units_and_empty_rows(clean):
    """The 16-page chunks with several units per request (next_n 6: a 4-row unit and a 2-row unit)
    and empty and one-key contexts mixed in; every row against the oracle."""
    B, nn = 70, 6
    rng = np.random.default_rng(45)
    ctx = rng.integers(0, 900, B)
    ctx[rng.random(B) < 0.2] = 0
    ctx[::13] = 1
    ctx[0] = 900
    inp = paged_inputs(B, nn, 0, 900, 16, seed=46, page_size=64, ctx=ctx)
    bt = np.full((B, 1024), -1, dtype=np.int32)
    bt[:, :inp.block_table.shape[1]] = inp.block_table
    width = 1024 * 64   # 70 requests x 2 units x 1024 table pages >= 131072: 16-page chunks
    args = [to_dev(a) for a in (inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len, bt)]
    out = torch.full((inp.rows, width), 12345.0, dtype=torch.float32, device="cuda")
    F.indexer_logits_paged(*args, width=width, clean=clean, logits=out)
    torch.cuda.synchronize()
    g = out.cpu().numpy()
    o = paged_mqa_logits(inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len,
                         inp.block_table, inp.page_size, width=max(1, int(inp.row_len.max())))
    for r in range(inp.rows):
        n = int(inp.row_len[r])
        d = np.abs(g[r, :n] - o[r, :n])
        assert np.all(d <= 1e-3 + 2e-3 * np.abs(o[r, :n])), r
        tail = g[r, n:]
        if clean:
            assert np.all(tail == -np.inf), r
        else:
            assert np.all((tail == 12345.0) | (tail == -np.inf)), r

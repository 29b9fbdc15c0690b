"""The boundary under concurrency, and keys on page ids outside the pool.

The library keeps no state between calls: the ragged logits kernel's work-queue counters
come from the caller's workspace (cleared by each call on its stream), and the overlapped
loop orders its streams with events it creates for the call.  So calls that run at the same
time, on any streams, from any threads, or as replays of graphs captured on one stream,
give the same bytes as eager calls.  Keys whose page id lies outside the kv pool hold no kv:
their logits are -inf whatever the clean flag says, so the fused paged top-k never reads a
stale workspace value, and a selected one maps to -1.
"""

import threading

import numpy as np
import pytest
import torch

import fp8_mqa_logits_amd as F
from oracle import map_block_table, mqa_logits, paged_mqa_logits, topk_indices
from tests.parity import ATOL, RTOL, assert_logits_close, assert_topk_exact, assert_topk_tolerant, to_dev
from workloads.generate import paged_inputs, ragged_inputs

pytestmark = pytest.mark.gpu


def _dev(inp):
    return [to_dev(a) for a in (inp.q, inp.kv, inp.kv_scale, inp.weights, inp.ks, inp.ke)]


def _ws():
    return torch.empty(512, dtype=torch.uint8, device="cuda")


def _oracle_rows(inp, got, rows, what):
    rows = np.asarray(rows)
    o = mqa_logits(inp.q[rows], inp.kv, inp.kv_scale, inp.weights[rows], inp.ks[rows], inp.ke[rows])
    assert_logits_close(got[torch.as_tensor(rows, device=got.device)].cpu().numpy(), o, inp.ks[rows],
                        inp.ke[rows], clean=True, what=what)


def _queue_inputs(seed):
    # 600 x 12000: 38 row blocks x 63 key slices = 2394 items, more than the resident workgroups,
    # so workgroups claim items through the counters
    return ragged_inputs(600, 12000, 8, seed=seed)


def test_ragged_logits_on_70_streams_at_once():
    a = _queue_inputs(81)
    da = _dev(a)
    ref = F.indexer_logits_ragged(*da, clean=True)
    torch.cuda.synchronize()
    _oracle_rows(a, ref, [0, 15, 16, 299, 583, 599], "70 streams reference")
    streams = [torch.cuda.Stream() for _ in range(70)]
    outs = [torch.empty_like(ref) for _ in streams]
    wss = [_ws() for _ in streams]
    torch.cuda.synchronize()
    for rep in range(2):
        for o in outs:
            o.fill_(7.0)
        torch.cuda.synchronize()
        for s, o, w in zip(streams, outs, wss):   # round-robin over the streams, nothing waits
            F.indexer_logits_ragged(*da, clean=True, logits=o, workspace=w, stream=s)
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert torch.equal(o, ref), f"stream {i}, round {rep}"


def test_two_graphs_from_one_capture_stream_replayed_concurrently():
    a, b = _queue_inputs(82), ragged_inputs(1000, 9000, 8, seed=83)
    da, db = _dev(a), _dev(b)
    ref_a = F.indexer_logits_ragged(*da, clean=True)
    ref_b = F.indexer_logits_ragged(*db, clean=True)
    torch.cuda.synchronize()
    _oracle_rows(a, ref_a, [0, 17, 598], "graph a reference")
    _oracle_rows(b, ref_b, [1, 500, 999], "graph b reference")
    out_a, out_b, out_e = torch.empty_like(ref_a), torch.empty_like(ref_b), torch.empty_like(ref_b)
    ws_a, ws_b, ws_e = _ws(), _ws(), _ws()
    sg = torch.cuda.Stream()
    torch.cuda.synchronize()
    g1, g2 = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1, stream=sg):
        F.indexer_logits_ragged(*da, clean=True, logits=out_a, workspace=ws_a, stream=sg)
    with torch.cuda.graph(g2, stream=sg):
        F.indexer_logits_ragged(*db, clean=True, logits=out_b, workspace=ws_b, stream=sg)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        out_a.fill_(7.0)
        out_b.fill_(7.0)
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            g1.replay()
        with torch.cuda.stream(s2):
            g2.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_a, ref_a), f"graph 1 replayed beside graph 2, round {rep}"
        assert torch.equal(out_b, ref_b), f"graph 2 replayed beside graph 1, round {rep}"
    # a replay running beside an eager launch on the capture stream
    for rep in range(3):
        out_a.fill_(7.0)
        out_e.fill_(7.0)
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            g1.replay()
        F.indexer_logits_ragged(*db, clean=True, logits=out_e, workspace=ws_e, stream=sg)
        torch.cuda.synchronize()
        assert torch.equal(out_a, ref_a), f"replay beside an eager launch, round {rep}"
        assert torch.equal(out_e, ref_b), f"eager launch beside a replay, round {rep}"


def test_fused_graphs_replayed_concurrently():
    """The fused loop (its logits counters, chunk logits and top-k candidates all in the workspace),
    captured twice on one stream with two workspaces and replayed on two streams at once."""
    a = ragged_inputs(300, 20000, 512, seed=84)
    da = _dev(a)
    ld = (a.n + 3) // 4 * 4
    cap = 64 * ld * 4
    ref = F.indexer_logits_topk_ragged(*da, a.k, logits_cap_bytes=cap)
    need = F.fp8idx_workspace_bytes(F.OP_LOGITS_TOPK_RAGGED, a.m, a.n, a.k, cap)
    ws = [torch.empty(need + 256, dtype=torch.uint8, device="cuda") for _ in range(2)]
    outs = [torch.empty_like(ref) for _ in range(2)]
    sg = torch.cuda.Stream()
    torch.cuda.synchronize()
    graphs = []
    for i in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=sg):
            F.indexer_logits_topk_ragged(*da, a.k, logits_cap_bytes=cap, out=outs[i], workspace=ws[i], stream=sg)
        graphs.append(g)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for o in outs:
            o.fill_(-7)
        torch.cuda.synchronize()
        for g, s in zip(graphs, streams):
            with torch.cuda.stream(s):
                g.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert torch.equal(o, ref), f"fused graph {i}, round {rep}"


def test_overlap_calls_from_two_threads():
    """Each call creates its own ordering events, so two host threads running the overlapped loop at
    the same time (each with its own streams and workspace) cannot cross their dependencies."""
    a = ragged_inputs(400, 16000, 256, seed=85)
    da = _dev(a)
    ld = (a.n + 3) // 4 * 4
    cap = 50 * ld * 4                      # 8 chunks
    ref = F.indexer_logits_topk_ragged(*da, a.k, logits_cap_bytes=cap)
    need = F.fp8idx_workspace_bytes(F.OP_LOGITS_TOPK_RAGGED_OVERLAP, a.m, a.n, a.k, cap)
    torch.cuda.synchronize()
    results, errors = {}, []

    def worker(t):
        try:
            s, side = torch.cuda.Stream(), torch.cuda.Stream()
            ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
            outs = [torch.full_like(ref, -7) for _ in range(4)]
            torch.cuda.synchronize()
            for o in outs:
                F.indexer_logits_topk_ragged_overlap(*da, a.k, side_stream=side, logits_cap_bytes=cap, out=o,
                                                     workspace=ws, stream=s)
            s.synchronize()
            side.synchronize()
            results[t] = outs
        except Exception as e:  # pragma: no cover - reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not errors, errors
    for t in range(2):
        for i, o in enumerate(results[t]):
            assert torch.equal(o, ref), f"thread {t} call {i}"


def _invalid_page_inputs():
    inp = paged_inputs(5, 4, 300, 1200, 16, seed=91, page_size=64)
    P = inp.kv_pool.shape[0]
    bt = inp.block_table.copy()
    bt[0, 2] = -1            # a hole inside request 0's windows
    bt[1, 0] = P + 3         # past the last page
    bt[1, 1] = -5
    bt[3, :] = -1            # request 3: no page at all, every key of its rows is -inf
    inp.block_table = bt
    return inp, P


@pytest.mark.parametrize("clean", [False, True])
def test_paged_logits_invalid_pages_are_minus_inf(clean):
    inp, P = _invalid_page_inputs()
    width = inp.max_pages * 64
    args = [to_dev(a) for a in (inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len, inp.block_table)]
    lg = torch.full((inp.rows, width), 12345.0, dtype=torch.float32, device="cuda")
    F.indexer_logits_paged(*args, width=width, clean=clean, logits=lg)
    torch.cuda.synchronize()
    g = lg.cpu().numpy().astype(np.float64)
    L = paged_mqa_logits(inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len, inp.block_table, 64,
                         width=width)
    for r in range(inp.rows):
        n_r = int(inp.row_len[r])
        o, x = L[r, :n_r], g[r, :n_r]
        hole = np.isneginf(o)
        assert np.all(np.isneginf(x[hole])), f"row {r}: a key on an invalid page is not -inf"
        assert np.all(np.abs(x[~hole] - o[~hole]) <= ATOL + RTOL * np.abs(o[~hole])), f"row {r}"
        if clean:
            assert np.all(np.isneginf(g[r, n_r:])), f"row {r}: clean tail"
        else:
            assert np.all(g[r, n_r:] == 12345.0), f"row {r}: clean = 0 wrote past the window"


def test_fused_paged_invalid_pages_against_oracle():
    inp, P = _invalid_page_inputs()
    width = inp.max_pages * 64
    args = [to_dev(a) for a in (inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len, inp.block_table)]
    rows = list(range(inp.rows))
    zeros = np.zeros(inp.rows, np.int64)
    ld = (width + 3) // 4 * 4
    for cap in (0, 8 * ld * 4):
        need = F.fp8idx_workspace_bytes_paged(inp.B, inp.next_n, width, inp.k, cap)
        # a workspace full of large stale values: none may reach the selection
        ws = torch.full(((need + 256 + 3) // 4,), 3.0e38, dtype=torch.float32, device="cuda").view(torch.uint8)
        slots = F.indexer_logits_topk_paged(*args, inp.k, width=width, logits_cap_bytes=cap, workspace=ws)
        raw = F.indexer_logits_topk_paged(*args, inp.k, width=width, map_to_slots=False, logits_cap_bytes=cap,
                                          workspace=ws)
        logits = F.indexer_logits_paged(*args, width=width, clean=True)
        torch.cuda.synchronize()
        g = logits.cpu().numpy().astype(np.float64)
        exact = topk_indices(g, zeros, inp.row_len, inp.k)
        assert_topk_exact(raw.cpu().numpy(), exact, what=f"invalid pages cap {cap}")
        # against the oracle (-inf for keys on invalid pages) within the tolerance band at the k-th value
        L = paged_mqa_logits(inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len, inp.block_table, 64,
                             width=width)
        assert_topk_tolerant(raw.cpu().numpy(), L, zeros, inp.row_len, inp.k, what=f"invalid pages cap {cap}")
        want = map_block_table(exact, rows, inp.next_n, inp.block_table, 64, P)
        got = slots.cpu().numpy()
        for r in rows:
            assert set(got[r].tolist()) == set(want[r].tolist()), f"slots row {r}"
        for r in range(12, 16):          # request 3: all -inf, the first k positions, all mapped to -1
            assert np.all(got[r] == -1)
            assert sorted(raw.cpu().numpy()[r].tolist()) == list(range(inp.k))


def test_topk_block_table_bounds_page_ids():
    """indexer_topk with a block table whose ids run past the pool: those keys map to -1."""
    rows, width, k = 4, 640, 40
    rng = np.random.default_rng(92)
    x = rng.standard_normal((rows, width)).astype(np.float32)
    ke = np.full(rows, width, np.int32)
    bt = rng.permutation(50)[:10].astype(np.int32).reshape(1, 10)
    bt[0, 3] = 50
    bt[0, 7] = 1000
    m = F.TopkMap(kind=F.MAP_BLOCK_TABLE, table=to_dev(bt), rows_per_req=rows, page_size=64, num_pages=50)
    g = F.indexer_topk(to_dev(x), to_dev(ke), k, map=m)
    torch.cuda.synchronize()
    raw = topk_indices(x.astype(np.float64), np.zeros(rows, np.int64), ke, k)
    want = map_block_table(raw, list(range(rows)), rows, bt, 64, 50)
    got = g.cpu().numpy()
    for r in range(rows):
        assert sorted(got[r].tolist()) == sorted(want[r].tolist())

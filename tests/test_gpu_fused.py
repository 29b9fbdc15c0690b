"""Fused logits + top-k: equivalence with the unfused calls, oracle parity on sampled rows of the
full-size workloads, determinism, HIP-graph replay and concurrent streams."""

import numpy as np
import pytest
import torch

import fp8_mqa_logits_amd as F
from oracle import mqa_logits, topk_indices, paged_topk_mapped, map_block_table, map_token_table
from tests.parity import assert_logits_close, assert_topk_exact, assert_topk_tolerant, to_dev
from workloads.generate import config_inputs, multi_request_ragged, paged_inputs, ragged_inputs

pytestmark = pytest.mark.gpu


def _dev(inp):
    return [to_dev(a) for a in (inp.q, inp.kv, inp.kv_scale, inp.weights, inp.ks, inp.ke)]


def _unfused(d, inp, k, map_=None):
    logits = F.indexer_logits_ragged(*d, clean=False)
    return F.indexer_topk(logits, d[5], k, ks=d[4], map=map_)


@pytest.mark.parametrize("cap_rows", [0, 1, 7, 16, 23])
def test_fused_equals_unfused_bytes(cap_rows):
    inp = ragged_inputs(61, 2500, 100, seed=41)
    d = _dev(inp)
    ref = _unfused(d, inp, 100)
    ld = (inp.n + 3) // 4 * 4
    cap = cap_rows * ld * 4
    got = F.indexer_logits_topk_ragged(*d, 100, logits_cap_bytes=cap)
    torch.cuda.synchronize()
    assert F.fp8idx_rows_per_chunk(cap, inp.n, inp.m) == (cap_rows if cap_rows else inp.m)
    assert torch.equal(ref, got)


def test_fused_multi_request_token_table():
    inp = multi_request_ragged([(700, 9), (1500, 30), (90, 5)], k=64, seed=42)
    d = _dev(inp)
    m = F.TopkMap(kind=F.MAP_TOKEN_TABLE, table=to_dev(inp.table), cu_rows=to_dev(inp.cu_rows))
    ld = (inp.n + 3) // 4 * 4
    got = F.indexer_logits_topk_ragged(*d, inp.k, map=m, logits_cap_bytes=11 * ld * 4)
    raw = F.indexer_logits_topk_ragged(*d, inp.k, logits_cap_bytes=11 * ld * 4)
    logits = F.indexer_logits_ragged(*d, clean=True)
    torch.cuda.synchronize()
    g_logits = logits.cpu().numpy().astype(np.float64)
    o = mqa_logits(inp.q, inp.kv, inp.kv_scale, inp.weights, inp.ks, inp.ke)
    assert_logits_close(g_logits, o, inp.ks, inp.ke, clean=True)
    raw = raw.cpu().numpy()
    assert_topk_tolerant(raw, o, inp.ks, inp.ke, inp.k)
    assert_topk_exact(raw, topk_indices(g_logits, inp.ks, inp.ke, inp.k))
    want = map_token_table(raw, list(range(inp.m)), inp.ks, inp.cu_rows, inp.table)
    assert np.array_equal(got.cpu().numpy(), want)


def test_fused_paged_small():
    inp = paged_inputs(5, 4, 300, 3000, 128, seed=43, page_size=64)
    width = inp.max_pages * 64
    args = [to_dev(a) for a in (inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len, inp.block_table)]
    ld = (width + 3) // 4 * 4
    for cap in (0, 4 * ld * 4, 9 * ld * 4):
        slots = F.indexer_logits_topk_paged(*args, inp.k, width=width, logits_cap_bytes=cap)
        raw = F.indexer_logits_topk_paged(*args, inp.k, width=width, map_to_slots=False, logits_cap_bytes=cap)
        logits = F.indexer_logits_paged(*args, width=width, clean=True)
        torch.cuda.synchronize()
        L, _, _ = paged_topk_mapped(inp, width=width)
        raw = raw.cpu().numpy()
        zeros = np.zeros(inp.rows, np.int64)
        assert_topk_tolerant(raw, L, zeros, inp.row_len, inp.k, what=f"paged cap {cap}")
        g_logits = logits.cpu().numpy().astype(np.float64)
        assert_topk_exact(raw, topk_indices(g_logits, zeros, inp.row_len, inp.k))
        want = map_block_table(raw, list(range(inp.rows)), 4, inp.block_table, 64)
        assert np.array_equal(slots.cpu().numpy(), want)


@pytest.mark.parametrize("mode", ["random", "rising_scale", "zero_weights", "bad_pages"])
@pytest.mark.parametrize("k", [2048, 300])
def test_fused_paged_fragment_maxima(mode, k):
    """Long decode rows, where the fused paged top-k (one workgroup per row) takes its threshold from
    the logits kernel's per-16-key fragment maxima and reads only the fragments that reach it.  Value
    mixes: scales rising along each context (the top keys crowd into the last pages), zero weights
    (every logit ties, so the exact whole-row path runs), and page ids outside the pool (-inf
    fragments).  Rows from 9000 to 131072 keys (shorter ones take the sampled threshold), three
    chunks through one workspace.  Checked against the exact selection on the device's own logits."""
    ctx = np.array([131072, 100000, 65537, 40000, 32769, 20000, 9000, 131071, 70000, 50001, 33000, 120000])
    inp = paged_inputs(len(ctx), 3, 0, 131072, k, seed=70 + k, ctx=ctx)
    if mode == "rising_scale":
        for b, c in enumerate(ctx):
            for p in range((int(c) + 63) // 64):
                t = p * 64 + np.arange(64)
                inp.scale_pool[inp.block_table[b, p]] = (0.5 + t / float(c)).astype(np.float32)
    elif mode == "zero_weights":
        inp.weights[:] = 0.0
    elif mode == "bad_pages":
        rng = np.random.default_rng(5)
        for b, c in enumerate(ctx):
            n_pages = (int(c) + 63) // 64
            bad = rng.choice(n_pages, size=max(1, n_pages // 10), replace=False)
            inp.block_table[b, bad] = np.where(rng.random(bad.size) < 0.5, -1, inp.kv_pool.shape[0] + 7)
    width = inp.max_pages * 64
    args = [to_dev(a) for a in (inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len, inp.block_table)]
    ld = (width + 3) // 4 * 4
    cap = 12 * ld * 4                                  # 4 requests per chunk: three chunks
    slots = F.indexer_logits_topk_paged(*args, k, width=width, logits_cap_bytes=cap)
    raw = F.indexer_logits_topk_paged(*args, k, width=width, map_to_slots=False, logits_cap_bytes=cap)
    logits = F.indexer_logits_paged(*args, width=width, clean=True)
    torch.cuda.synchronize()
    g = logits.cpu().numpy().astype(np.float64)
    zeros = np.zeros(inp.rows, np.int64)
    exact = topk_indices(g, zeros, inp.row_len, k)
    assert_topk_exact(raw.cpu().numpy(), exact, what=f"fragment maxima {mode} k{k}")
    want = map_block_table(exact, list(range(inp.rows)), inp.next_n, inp.block_table, 64, inp.kv_pool.shape[0])
    got = slots.cpu().numpy()
    for i in range(inp.rows):
        assert set(got[i].tolist()) == set(want[i].tolist()), f"{mode} k{k} slots row {i}"


@pytest.mark.parametrize("B,next_n,cap_requests", [(64, 1, 0), (20, 2, 8), (9, 6, 4)])
def test_fused_paged_fragment_maxima_row_slots(B, next_n, cap_requests):
    """The fragment maxima's chunk-major blocks with one row slot per block (next_n 1; 64 requests
    over a 2048-page table take the 16-page chunks), two slots (next_n 2) and two 4-row groups per
    request (next_n 6: a 4-row and a 2-row unit), over one or several workspace chunks.  Rows long
    enough for the fragment-maxima path; checked against the exact selection on the device's logits."""
    rng = np.random.default_rng(B * 10 + next_n)
    ctx = rng.integers(50000, 131073, B)
    ctx[0] = 131072
    inp = paged_inputs(B, next_n, 0, 131072, 2048, seed=80 + next_n, ctx=ctx)
    width = inp.max_pages * 64
    args = [to_dev(a) for a in (inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len, inp.block_table)]
    ld = (width + 3) // 4 * 4
    cap = cap_requests * next_n * ld * 4
    slots = F.indexer_logits_topk_paged(*args, inp.k, width=width, logits_cap_bytes=cap)
    raw = F.indexer_logits_topk_paged(*args, inp.k, width=width, map_to_slots=False, logits_cap_bytes=cap)
    logits = F.indexer_logits_paged(*args, width=width, clean=True)
    torch.cuda.synchronize()
    g = logits.cpu().numpy().astype(np.float64)
    zeros = np.zeros(inp.rows, np.int64)
    exact = topk_indices(g, zeros, inp.row_len, inp.k)
    assert_topk_exact(raw.cpu().numpy(), exact, what=f"row slots B{B} next_n{next_n}")
    want = map_block_table(exact, list(range(inp.rows)), next_n, inp.block_table, 64, inp.kv_pool.shape[0])
    got = slots.cpu().numpy()
    for i in range(inp.rows):
        assert set(got[i].tolist()) == set(want[i].tolist()), f"B{B} next_n{next_n} slots row {i}"


def _sample_rows(m, chunk):
    rows = {0, 1, m // 2, m - 2, m - 1}
    if chunk and chunk < m:
        for s in range(chunk, m, chunk):
            rows.update({s - 1, s})
    return sorted(r for r in rows if 0 <= r < m)


@pytest.mark.parametrize("name", ["tiny", "prefill_35k", "prefill_64k", "long_prefix_210k", "tail_80k", "warm_154k"])
def test_full_size_ragged_configs_sampled(name):
    """Sampled rows of each ragged workload through the fused entry at its cap (tail_80k and warm_154k:
    the chunking page's other two scenarios, one shot) against the float64 oracle."""
    inp = config_inputs(name)
    d = _dev(inp)
    cap = inp.cap_bytes
    out = F.indexer_logits_topk_ragged(*d, inp.k, logits_cap_bytes=cap)
    torch.cuda.synchronize()
    cmax = F.fp8idx_rows_per_chunk(cap, inp.n, inp.m)
    chunk = -(-inp.m // -(-inp.m // cmax))   # the entry's chunks: the rows spread evenly over ceil(m / cmax)
    rows = _sample_rows(inp.m, chunk if cap else 0)
    ridx = np.array(rows)
    # the sampled rows' logits from the same kernel (values do not depend on batching)
    lg = F.indexer_logits_ragged(d[0][ridx], d[1], d[2], d[3][ridx], d[4][ridx], d[5][ridx], clean=True)
    torch.cuda.synchronize()
    g_logits = lg.cpu().numpy().astype(np.float64)
    o = mqa_logits(inp.q[ridx], inp.kv, inp.kv_scale, inp.weights[ridx], inp.ks[ridx], inp.ke[ridx])
    assert_logits_close(g_logits, o, inp.ks[ridx], inp.ke[ridx], clean=True, what=name)
    got = out.cpu().numpy()[ridx]
    assert_topk_tolerant(got, o, inp.ks[ridx], inp.ke[ridx], inp.k, what=name)
    assert_topk_exact(got, topk_indices(g_logits, inp.ks[ridx], inp.ke[ridx], inp.k), what=name)


def test_full_size_paged_config_sampled():
    inp = config_inputs("paged_decode")
    width = inp.max_pages * 64
    args = [to_dev(a) for a in (inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len, inp.block_table)]
    slots = F.indexer_logits_topk_paged(*args, inp.k, width=width)
    logits = F.indexer_logits_paged(*args, width=width, clean=True)
    torch.cuda.synchronize()
    rows = [0, 1, 2, 3, 101, 130, 254, 255]
    L, _, mapped = paged_topk_mapped(inp, rows=rows, width=width)
    ridx = np.array(rows)
    g_logits = logits.cpu().numpy()[ridx].astype(np.float64)
    zeros = np.zeros(len(rows), np.int64)
    assert_logits_close(g_logits, L, zeros, inp.row_len[ridx], clean=True, what="paged full")
    exact_raw = topk_indices(g_logits, zeros, inp.row_len[ridx], inp.k)
    want = map_block_table(exact_raw, rows, inp.next_n, inp.block_table, 64)
    got = slots.cpu().numpy()[ridx]
    for i in range(len(rows)):
        assert set(got[i].tolist()) == set(want[i].tolist())


def test_determinism_and_graph_replay():
    inp = ragged_inputs(300, 20000, 2048, seed=44)
    d = _dev(inp)
    ld = (inp.n + 3) // 4 * 4
    cap = 64 * ld * 4
    need = F.fp8idx_workspace_bytes(F.OP_LOGITS_TOPK_RAGGED, inp.m, inp.n, inp.k, cap)
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    out_a = torch.empty((inp.m, inp.k), dtype=torch.int32, device="cuda")
    out_b = torch.empty_like(out_a)
    F.indexer_logits_topk_ragged(*d, inp.k, logits_cap_bytes=cap, out=out_a, workspace=ws)
    F.indexer_logits_topk_ragged(*d, inp.k, logits_cap_bytes=cap, out=out_b, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)
    s = torch.cuda.Stream()
    out_g = torch.full_like(out_a, -7)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            F.indexer_logits_topk_ragged(*d, inp.k, logits_cap_bytes=cap, out=out_g, workspace=ws)
    for rep in range(3):
        out_g.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_a), f"graph replay {rep} differs from eager"


def test_two_streams_concurrently():
    a = ragged_inputs(120, 9000, 256, seed=45)
    b = ragged_inputs(90, 7000, 256, seed=46)
    da, db = _dev(a), _dev(b)
    ref_a = F.indexer_logits_topk_ragged(*da, 256)
    ref_b = F.indexer_logits_topk_ragged(*db, 256)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            oa = F.indexer_logits_topk_ragged(*da, 256, stream=s1)
        with torch.cuda.stream(s2):
            ob = F.indexer_logits_topk_ragged(*db, 256, stream=s2)
        outs.append((oa, ob))
    torch.cuda.synchronize()
    for oa, ob in outs:
        assert torch.equal(oa, ref_a) and torch.equal(ob, ref_b)


@pytest.mark.parametrize("cap_rows", [0, 1, 7, 16, 23])
def test_overlap_equals_serial_bytes(cap_rows):
    inp = ragged_inputs(61, 2500, 100, seed=41)
    d = _dev(inp)
    ld = (inp.n + 3) // 4 * 4
    cap = cap_rows * ld * 4
    ref = F.indexer_logits_topk_ragged(*d, 100, logits_cap_bytes=cap)
    side = torch.cuda.Stream()
    got = F.indexer_logits_topk_ragged_overlap(*d, 100, side_stream=side, logits_cap_bytes=cap)
    torch.cuda.synchronize()
    assert torch.equal(ref, got)


def test_overlap_token_table_and_back_to_back_calls():
    inp = multi_request_ragged([(700, 9), (1500, 30), (90, 5)], k=64, seed=42)
    d = _dev(inp)
    m = F.TopkMap(kind=F.MAP_TOKEN_TABLE, table=to_dev(inp.table), cu_rows=to_dev(inp.cu_rows))
    ld = (inp.n + 3) // 4 * 4
    cap = 11 * ld * 4
    ref = F.indexer_logits_topk_ragged(*d, inp.k, map=m, logits_cap_bytes=cap)
    need = F.fp8idx_workspace_bytes(F.OP_LOGITS_TOPK_RAGGED_OVERLAP, inp.m, inp.n, inp.k, cap)
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    outs = [F.indexer_logits_topk_ragged_overlap(*d, inp.k, side_stream=side, map=m, logits_cap_bytes=cap,
                                                 workspace=ws) for _ in range(4)]
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, ref)


def test_overlap_graph_replay():
    inp = ragged_inputs(300, 20000, 2048, seed=44)
    d = _dev(inp)
    ld = (inp.n + 3) // 4 * 4
    cap = 64 * ld * 4
    ref = F.indexer_logits_topk_ragged(*d, inp.k, logits_cap_bytes=cap)
    need = F.fp8idx_workspace_bytes(F.OP_LOGITS_TOPK_RAGGED_OVERLAP, inp.m, inp.n, inp.k, cap)
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    s, side = torch.cuda.Stream(), torch.cuda.Stream()
    out_g = torch.full((inp.m, inp.k), -7, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            F.indexer_logits_topk_ragged_overlap(*d, inp.k, side_stream=side, logits_cap_bytes=cap, out=out_g,
                                                 workspace=ws, stream=s)
    for rep in range(3):
        out_g.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref), f"graph replay {rep} differs from eager"

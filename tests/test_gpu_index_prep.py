"""GPU parity of the index preparation entries against the oracle (integer work: exact)."""

import json
import os

import numpy as np
import pytest
import torch

import fp8_mqa_logits_amd as F
import oracle.indexer_oracle as O
from tests.parity import to_dev
from workloads.generate import multi_request_ragged

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
SENTINEL = -12345


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _run_ragged(seq, ql, req, table, max_q, max_keys):
    L = F.load_library()
    B = len(seq)
    d = {k: torch.full((n,), SENTINEL, dtype=torch.int32, device="cuda")
         for k, n in (("cu_seq", B + 1), ("cu_q", B + 1), ("ks", max_q), ("ke", max_q), ("mem", max_keys))}
    # the inputs stay referenced until the kernel has finished reading them
    tab, sq, qq, rq = _i32(table), _i32(seq), _i32(ql), _i32(req)
    st = L.indexer_prepare_ragged(sq.data_ptr(), qq.data_ptr(), rq.data_ptr(), tab.data_ptr(),
                                  tab.shape[1], tab.shape[0], B, d["cu_seq"].data_ptr(), d["cu_q"].data_ptr(),
                                  d["ks"].data_ptr(), d["ke"].data_ptr(), max_q, d["mem"].data_ptr(), max_keys,
                                  torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    del tab, sq, qq, rq
    return {k: v.cpu().numpy().astype(np.int64) for k, v in d.items()}


def _check_against_oracle(seq, ql, req, table, max_q, max_keys):
    g = _run_ragged(seq, ql, req, table, max_q, max_keys)
    o = O.prepare_ragged(seq, ql, req, table)
    assert np.array_equal(g["cu_seq"], o["cu_seq"]) and np.array_equal(g["cu_q"], o["cu_q"])
    nq = min(len(o["ks"]), max_q)
    assert np.array_equal(g["ks"][:nq], o["ks"][:nq]) and np.array_equal(g["ke"][:nq], o["ke"][:nq])
    assert np.all(g["ks"][nq:] == SENTINEL) and np.all(g["ke"][nq:] == SENTINEL)
    nk = min(len(o["ragged_mem"]), max_keys)
    assert np.array_equal(g["mem"][:nk], o["ragged_mem"][:nk])
    assert np.all(g["mem"][nk:] == SENTINEL)


def test_page_example_layout():
    gj = json.load(open(os.path.join(HERE, "golden", "ragged_index_expected.json")))
    table = (1000 * np.arange(gj["table_rows"])[:, None] + np.arange(gj["table_ld"])[None, :]).astype(np.int32)
    g = _run_ragged(gj["seq_len"], [1] * 6, gj["req_idx"], table, 6, gj["capacity"])
    want = np.concatenate([table[2, :40], table[0, :6], np.tile(table[gj["hold"], :2], 4)])
    assert np.array_equal(g["mem"][:54], want)
    assert np.all(g["mem"][54:] == SENTINEL)


@pytest.mark.parametrize("B,seed", [(1, 1), (7, 2), (64, 3), (1000, 4), (4096, 5)])
def test_random_batches(B, seed):
    rng = np.random.default_rng(seed)
    seq = rng.integers(0, 600, B)
    seq[rng.random(B) < 0.1] = 0                         # empty requests
    ql = rng.integers(0, 50, B)
    ql[rng.random(B) < 0.05] = 10 ** 6                   # more queries than tokens: clamped
    rows = max(4, B // 2)
    req = rng.integers(-1, rows + 1, B)                  # includes out-of-range rows
    table = rng.integers(0, 1 << 30, (rows, 512)).astype(np.int32)   # rows shorter than some requests
    tq, tk = int(np.minimum(np.maximum(ql, 0), seq).sum()), int(seq.sum())
    _check_against_oracle(seq, ql, req, table, tq + 5, tk + 7)


def test_capacities_truncate_without_writing_past_them():
    rng = np.random.default_rng(9)
    seq = rng.integers(10, 300, 20)
    ql = rng.integers(1, 10, 20)
    table = rng.integers(0, 1000, (20, 300)).astype(np.int32)
    _check_against_oracle(seq, ql, np.arange(20), table, 17, 1001)


def test_matches_the_multi_request_recipe_windows():
    inp = multi_request_ragged([(700, 9), (1500, 30), (90, 5)], k=64, seed=42)
    seq = np.diff(np.concatenate([[0], np.cumsum([700, 1500, 90])]))
    out = F.indexer_prepare_ragged(_i32(seq), _i32([9, 30, 5]), _i32([0, 1, 2]), _i32(inp.table), max_q=inp.m,
                                   max_keys=int(seq.sum()))
    torch.cuda.synchronize()
    assert np.array_equal(out["ks"].cpu().numpy(), inp.ks) and np.array_equal(out["ke"].cpu().numpy(), inp.ke)
    assert np.array_equal(out["cu_q"].cpu().numpy(), inp.cu_rows)


def test_page_benchmark_shape_8_requests_of_1m_tokens():
    # the PR page's index benchmark: 8 requests x 1M tokens, 16 queries per request
    B, S, Q = 8, 1 << 20, 16
    rng = np.random.default_rng(10)
    table = torch.randint(0, 1 << 30, (B + 2, S), dtype=torch.int32, device="cuda")
    req = np.array([3, 0, 9, 1, 2, 8, 5, 4])
    out = F.indexer_prepare_ragged(_i32(np.full(B, S)), _i32(np.full(B, Q)), _i32(req), table, max_q=B * Q,
                                   max_keys=B * S)
    torch.cuda.synchronize()
    mem = out["ragged_mem"]
    for b in range(B):                                   # the defining property at full size
        assert torch.equal(mem[b * S:(b + 1) * S], table[int(req[b])])
    o = O.prepare_ragged([S] * B, [Q] * B, req, np.zeros((B + 2, 1), np.int32))
    assert np.array_equal(out["ks"].cpu().numpy(), o["ks"]) and np.array_equal(out["ke"].cpu().numpy(), o["ke"])


def test_decode_preparation():
    rng = np.random.default_rng(12)
    B, nn, rows, mp = 64, 4, 80, 2048
    seq = rng.integers(0, 131072, B)
    seq[:3] = [0, 1, 3]
    req = rng.integers(-2, rows + 2, B)
    r2p = rng.integers(-1, 1 << 20, (rows, mp + 16)).astype(np.int32)
    row_len, bt = F.indexer_prepare_decode(_i32(seq), _i32(req), _i32(r2p), nn, max_pages=mp)
    torch.cuda.synchronize()
    o = O.prepare_decode(seq, nn, req, r2p[:, :mp])
    assert np.array_equal(row_len.cpu().numpy(), o["row_len"])
    assert np.array_equal(bt.cpu().numpy(), o["block_table"])


def test_graph_replay_equals_eager():
    rng = np.random.default_rng(13)
    seq, ql = _i32(rng.integers(0, 2000, 50)), _i32(rng.integers(0, 30, 50))
    req, table = _i32(rng.permutation(50)), _i32(rng.integers(0, 1 << 20, (50, 2000)))
    ref = F.indexer_prepare_ragged(seq, ql, req, table, max_q=2000, max_keys=120000)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            got = F.indexer_prepare_ragged(seq, ql, req, table, max_q=2000, max_keys=120000, stream=s)
    for rep in range(3):
        for v in got.values():
            v.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        nq, nk = int(ref["cu_q"][-1]), int(ref["cu_seq"][-1])
        assert torch.equal(got["cu_seq"], ref["cu_seq"]) and torch.equal(got["cu_q"], ref["cu_q"])
        assert torch.equal(got["ks"][:nq], ref["ks"][:nq]) and torch.equal(got["ke"][:nq], ref["ke"][:nq])
        assert torch.equal(got["ragged_mem"][:nk], ref["ragged_mem"][:nk]), f"replay {rep}"

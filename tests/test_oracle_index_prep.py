"""Pins for the oracle's index preparation (prepare_ragged, prepare_decode)."""

import json
import os

import numpy as np

import oracle.indexer_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def _table(rows, ld):
    return (1000 * np.arange(rows)[:, None] + np.arange(ld)[None, :]).astype(np.int32)


def test_ragged_buffer_layout_of_the_page_example():
    g = json.load(open(os.path.join(HERE, "golden", "ragged_index_expected.json")))
    table = _table(g["table_rows"], g["table_ld"])
    out = O.prepare_ragged(g["seq_len"], [1] * 6, g["req_idx"], table)
    want = np.concatenate([table[2, :40], table[0, :6], np.tile(table[g["hold"], :2], 4)])
    assert np.array_equal(out["ragged_mem"], want)
    buf = np.full(g["capacity"], -1)
    buf[:len(want)] = out["ragged_mem"]
    assert np.all(buf[len(want):] == -1) and len(want) == 54


def test_single_request_matches_the_chunking_bench_windows():
    # one request of n tokens whose last m are queries: ks = 0, ke[i] = n - m + i + 1 (the _build recipe)
    n, m = 500, 37
    out = O.prepare_ragged([n], [m], [0], _table(1, n))
    assert np.all(out["ks"] == 0)
    assert np.array_equal(out["ke"], n - m + np.arange(m) + 1)
    assert np.array_equal(out["ragged_mem"], np.arange(n))


def test_windows_stay_inside_their_request_and_end_causally():
    rng = np.random.default_rng(5)
    seq = rng.integers(0, 300, 9)
    ql = rng.integers(0, 40, 9)
    out = O.prepare_ragged(seq, ql, rng.permutation(9), _table(9, 300))
    ql = np.minimum(ql, seq)
    assert out["cu_seq"][-1] == seq.sum() and out["cu_q"][-1] == ql.sum()
    for b in range(9):
        qs = slice(out["cu_q"][b], out["cu_q"][b + 1])
        assert np.all(out["ks"][qs] == out["cu_seq"][b])
        assert np.all(out["ke"][qs] <= out["cu_seq"][b + 1])
        if ql[b]:
            assert out["ke"][qs][-1] == out["cu_seq"][b + 1]          # the last query sees its whole request
            assert np.all(np.diff(out["ke"][qs]) == 1)


def test_out_of_range_entries_are_minus_one():
    out = O.prepare_ragged([5, 3], [1, 1], [7, 0], _table(2, 4))
    assert np.array_equal(out["ragged_mem"], [-1, -1, -1, -1, -1, 0, 1, 2])
    out = O.prepare_ragged([6], [2], [1], _table(2, 4))
    assert np.array_equal(out["ragged_mem"], [1000, 1001, 1002, 1003, -1, -1])


def test_decode_rows_are_causal_and_tables_follow_req_idx():
    r2p = _table(5, 8)
    out = O.prepare_decode([100, 3, 64], 4, [4, 0, 9], r2p)
    assert np.array_equal(out["row_len"], [97, 98, 99, 100, 0, 1, 2, 3, 61, 62, 63, 64])
    assert np.array_equal(out["block_table"][0], r2p[4])
    assert np.array_equal(out["block_table"][1], r2p[0])
    assert np.all(out["block_table"][2] == -1)


def _mutant(variant):
    real = O.prepare_ragged.__wrapped__ if hasattr(O.prepare_ragged, "__wrapped__") else O.prepare_ragged

    def prep(seq_len, q_len, req_idx, table):
        if variant == "req_is_b":
            req_idx = list(range(len(seq_len)))
        out = real(seq_len, q_len, req_idx, table)
        out = {k: v.copy() for k, v in out.items()}
        if variant == "ke_off_by_one":
            out["ke"] = out["ke"] - 1
        elif variant == "ks_from_cu_q":
            qcount = np.diff(out["cu_q"])
            out["ks"] = np.repeat(out["cu_q"][:-1], qcount)
        elif variant == "window_from_start":
            qcount = np.diff(out["cu_q"])
            t = np.concatenate([np.arange(c) for c in qcount]) if len(qcount) else np.zeros(0, np.int64)
            out["ke"] = out["ks"] + t + 1
        return out
    return prep


import pytest  # noqa: E402


@pytest.mark.parametrize("variant", ["req_is_b", "ke_off_by_one", "ks_from_cu_q", "window_from_start"])
def test_pins_catch_planted_index_mistakes(variant, monkeypatch):
    monkeypatch.setattr(O, "prepare_ragged", _mutant(variant))
    checks = [test_ragged_buffer_layout_of_the_page_example, test_single_request_matches_the_chunking_bench_windows,
              test_windows_stay_inside_their_request_and_end_causally, test_out_of_range_entries_are_minus_one]
    failed = 0
    for c in checks:
        try:
            c()
        except AssertionError:
            failed += 1
    assert failed > 0, f"no pin caught mutant {variant}"

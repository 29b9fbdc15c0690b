"""Pins of the oracle's top-k selection and index maps."""

import numpy as np
import pytest

from oracle import (topk_indices, map_token_table, map_block_table, rows_per_chunk,
                    ragged_topk_mapped, paged_topk_mapped, mqa_logits)
from workloads.generate import multi_request_ragged, paged_inputs


def _brute_topk(row, a, b, k):
    # plain Python sort, independent of numpy's lexsort
    items = sorted(range(a, b), key=lambda j: (-float(row[j]), j))[:k]
    return items + [-1] * (k - len(items))


def _random_rows(rng, rows, n, tie_heavy):
    if tie_heavy:
        x = rng.integers(-5, 6, size=(rows, n)).astype(np.float64) * 0.5
        x[x == 0] = np.where(rng.random((x == 0).sum()) < 0.5, -0.0, 0.0)
    else:
        x = rng.standard_normal((rows, n))
    return x


@pytest.mark.parametrize("tie_heavy", [False, True])
def test_topk_matches_python_sorted(tie_heavy):
    rng = np.random.default_rng(31 + tie_heavy)
    rows, n, k = 12, 57, 9
    x = _random_rows(rng, rows, n, tie_heavy)
    ks = rng.integers(0, 20, rows)
    ke = np.minimum(n, ks + rng.integers(0, 45, rows))
    got = topk_indices(x, ks, ke, k)
    for r in range(rows):
        assert got[r].tolist() == _brute_topk(x[r], ks[r], ke[r], k)


def test_topk_invariants_large():
    rng = np.random.default_rng(33)
    rows, n, k = 6, 5000, 300
    x = np.round(rng.standard_normal((rows, n)) * 8) / 8      # many exact ties
    ks = np.array([0, 10, 100, 4000, 0, 2500])
    ke = np.array([5000, 4000, 350, 4100, 200, 2500])
    got = topk_indices(x, ks, ke, k)
    for r in range(rows):
        a, b = int(ks[r]), int(ke[r])
        sel = got[r][got[r] >= 0]
        assert sel.size == min(k, max(0, b - a))
        assert np.all(got[r][sel.size:] == -1)
        assert np.unique(sel).size == sel.size
        assert np.all((sel >= a) & (sel < b))
        if sel.size and sel.size < b - a:
            unsel = np.setdiff1d(np.arange(a, b), sel)
            vmin = x[r, sel].min()
            assert vmin >= x[r, unsel].max()
            # ties at the threshold: every selected tie index is below every unselected one
            tie_sel = sel[x[r, sel] == vmin]
            tie_uns = unsel[x[r, unsel] == vmin]
            if tie_uns.size:
                assert tie_sel.max() < tie_uns.min()


def test_topk_signed_zero_ties_by_index():
    x = np.array([[-0.0, 0.0, -0.0, 0.0, -1.0]])
    assert topk_indices(x, [0], [5], 2).tolist() == [[0, 1]]


def test_token_table_map_independent_expectation():
    inp = multi_request_ragged([(40, 5), (17, 3), (60, 8)], k=6, seed=34)
    # replace the table by a closed-form one so the expected map is a formula
    R, ld = inp.table.shape
    table = (1000 * np.arange(R)[:, None] + np.arange(ld)[None, :] + 7).astype(np.int32)
    rng = np.random.default_rng(3)
    rows = list(range(inp.m))
    raw = np.full((inp.m, 6), -1, np.int64)
    for i in rows:
        a, b = int(inp.ks[i]), int(inp.ke[i])
        cnt = min(6, b - a)
        raw[i, :cnt] = rng.choice(np.arange(a, b), cnt, replace=False)
    got = map_token_table(raw, rows, inp.ks, inp.cu_rows, table)
    for i in rows:
        req = int(np.nonzero(inp.cu_rows <= i)[0].max())
        for c in range(6):
            j = raw[i, c]
            want = -1 if j < 0 else 1000 * req + (j - inp.ks[i]) + 7
            assert got[i, c] == want


def test_block_table_map_inverse_roundtrip():
    inp = paged_inputs(4, 3, 100, 700, 32, seed=35, page_size=64)
    rng = np.random.default_rng(4)
    rows = list(range(inp.rows))
    raw = np.stack([rng.choice(int(inp.row_len[r]), 32, replace=False) for r in rows])
    got = map_block_table(raw, rows, inp.next_n, inp.block_table, 64)
    for o, r in enumerate(rows):
        b = r // inp.next_n
        for c in range(32):
            slot = int(got[o, c])
            page, off = divmod(slot, 64)
            p = int(np.nonzero(inp.block_table[b] == page)[0][0])
            assert p * 64 + off == raw[o, c]


def test_ragged_mapped_pipeline_small():
    inp = multi_request_ragged([(90, 4), (33, 2)], k=16, seed=36)
    L, raw, mapped = ragged_topk_mapped(inp)
    for i in range(inp.m):
        a, b = int(inp.ks[i]), int(inp.ke[i])
        assert raw[i].tolist() == _brute_topk(L[i], a, b, 16)
        req = 0 if i < inp.cu_rows[1] else 1
        sel = raw[i] >= 0
        assert np.array_equal(mapped[i, sel], inp.table[req, raw[i, sel] - a])


def test_paged_mapped_pipeline_small():
    inp = paged_inputs(2, 4, 130, 300, 20, seed=37, page_size=64)
    L, raw, mapped = paged_topk_mapped(inp)
    for r in range(inp.rows):
        assert raw[r].tolist() == _brute_topk(L[r], 0, int(inp.row_len[r]), 20)
        b = r // 4
        j = raw[r]
        assert np.array_equal(mapped[r], inp.block_table[b, j // 64].astype(np.int64) * 64 + j % 64)


def test_block_table_invalid_pages_map_to_minus_one():
    """Page ids outside [0, num_pages) map to -1; a row whose keys are all on such pages is all -inf,
    its top-k takes the lowest positions (ties by index) and every one maps to -1."""
    bt = np.array([[5, -1, 9, 12]], dtype=np.int32)
    raw = np.array([[0, 63, 64, 127, 128, 191, 192, -1]])
    got = map_block_table(raw, [0], 1, bt, 64, num_pages=10)
    assert got.tolist() == [[5 * 64, 5 * 64 + 63, -1, -1, 9 * 64, 9 * 64 + 63, -1, -1]]
    # without a page count only negative ids are invalid
    assert map_block_table(raw, [0], 1, bt, 64)[0, 6] == 12 * 64
    L = np.full((1, 100), -np.inf)
    sel = topk_indices(L, np.zeros(1, np.int64), np.array([100]), 8)
    assert sel.tolist() == [list(range(8))]
    assert np.all(map_block_table(sel, [0], 1, np.full((1, 2), -1, np.int32), 64, num_pages=10) == -1)


def test_rows_per_chunk_chunking_page_formula():
    # max(1, int(gb * 1e9) // (n * 4)) rows per chunk, decimal gigabytes
    assert rows_per_chunk(2_000_000_000, 210000, 7500) == 2380
    assert rows_per_chunk(2_000_000_000, 65536, 8192) == 7629
    assert rows_per_chunk(0, 65536, 8192) == 8192
    assert rows_per_chunk(10, 65536, 8192) == 1
    r = rows_per_chunk(2_000_000_000, 210000, 7500)
    chunks = [min(r, 7500 - s) for s in range(0, 7500, r)]
    assert chunks == [2380, 2380, 2380, 360]

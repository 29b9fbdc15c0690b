"""Pins of the oracle's logits against exact arithmetic, closed forms and invariants."""

import numpy as np
import pytest

from oracle import mqa_logits, scores, gather_paged_kv, paged_mqa_logits
from tests.oracle_pins import ALL_LOGIT_CHECKS, torch_decode
from workloads.generate import H, D, ragged_inputs, paged_inputs


@pytest.mark.parametrize("check", ALL_LOGIT_CHECKS, ids=lambda c: c.__name__)
def test_oracle_logits_pin(check):
    ok, msg = check(mqa_logits)
    assert ok, msg


def test_dot_is_exact_integer_brute_force():
    # Each e4m3fn value times 2**9 is an integer, so each dot times 2**18 is an exact
    # integer sum; the oracle's float64 dot must equal it bit for bit.
    inp = ragged_inputs(2, 7, 4, seed=21)
    Q = torch_decode(inp.q) * 512.0
    K = torch_decode(inp.kv) * 512.0
    assert np.all(Q == np.round(Q)) and np.all(K == np.round(K))
    S = scores(inp.q, inp.kv)
    for i in range(2):
        for h in range(0, H, 5):
            for j in range(7):
                want = sum(int(Q[i, h, d]) * int(K[j, d]) for d in range(D))
                assert S[i, h, j] * 2.0 ** 18 == float(want)


def test_dot_exact_at_extremes():
    # largest magnitudes: 448 * 448 * 128 must be exact too
    q = np.full((1, 1, D), 0x7E, np.uint8)
    kv = np.full((2, D), 0x7E, np.uint8)
    kv[1, ::2] = 0xFE
    S = scores(q, kv)
    assert S[0, 0, 0] == 448.0 * 448.0 * 128
    assert S[0, 0, 1] == 0.0


def test_paged_equals_ragged_on_hand_gathered_kv():
    inp = paged_inputs(3, 2, 70, 300, 16, seed=22, page_size=64)
    L = paged_mqa_logits(inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len,
                         inp.block_table, inp.page_size)
    for r in range(inp.rows):
        b = r // inp.next_n
        n_r = int(inp.row_len[r])
        # independent token-by-token gather
        kv = np.stack([inp.kv_pool[inp.block_table[b, j // 64], j % 64] for j in range(n_r)])
        sc = np.array([inp.scale_pool[inp.block_table[b, j // 64], j % 64] for j in range(n_r)],
                      np.float32)
        q = inp.q.reshape(inp.rows, H, D)[r:r + 1]
        want = mqa_logits(q, kv, sc, inp.weights[r:r + 1], np.array([0]), np.array([n_r]))
        assert np.array_equal(L[r, :n_r], want[0])
        assert np.all(L[r, n_r:] == -np.inf)


def test_gather_paged_kv_contiguity():
    inp = paged_inputs(2, 1, 100, 200, 8, seed=23, page_size=64)
    kv, sc, real = gather_paged_kv(inp.kv_pool, inp.scale_pool, inp.block_table[1], int(inp.ctx[1]), 64)
    assert kv.shape == (int(inp.ctx[1]), D)
    assert real.all()
    j = int(inp.ctx[1]) - 1
    assert np.array_equal(kv[j], inp.kv_pool[inp.block_table[1, j // 64], j % 64])
    assert sc[j] == inp.scale_pool[inp.block_table[1, j // 64], j % 64]


def test_paged_invalid_pages_bruteforce():
    """A key on a page id outside the pool (-1 past a request's pages, or an id past the last page)
    has no kv: its logit is -inf; every other key is the formula, evaluated here one key at a time
    from torch's fp8 decode with a scalar epilogue."""
    from tests.oracle_pins import torch_decode
    inp = paged_inputs(2, 2, 150, 260, 8, seed=24, page_size=64)
    P = inp.kv_pool.shape[0]
    bt = inp.block_table.copy()
    bt[0, 1] = -1          # a hole inside request 0's window
    bt[1, 0] = P           # one past the last page
    bt[1, 2] = P + 7
    L = paged_mqa_logits(inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len, bt, 64)
    Q = torch_decode(inp.q).reshape(inp.rows, H, D)
    K = torch_decode(inp.kv_pool)
    for r in range(inp.rows):
        b = r // inp.next_n
        n_r = int(inp.row_len[r])
        for j in range(n_r):
            page = int(bt[b, j // 64])
            if page < 0 or page >= P:
                assert L[r, j] == -np.inf, (r, j)
                continue
            k = K[page, j % 64]
            sc = float(inp.scale_pool[page, j % 64])
            want = 0.0
            for h in range(H):
                x = float(np.dot(Q[r, h], k)) * sc
                want += float(inp.weights[r, h]) * max(x, 0.0)
            assert abs(L[r, j] - want) <= 1e-12 * max(1.0, abs(want)), (r, j)
        assert np.all(L[r, n_r:] == -np.inf)

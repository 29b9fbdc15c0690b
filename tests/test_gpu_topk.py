"""Exact parity of the HIP top-k (selection + index maps) with the oracle's selection."""

import numpy as np
import pytest
import torch

import fp8_mqa_logits_amd as F
from oracle import topk_indices, map_token_table, map_block_table
from tests.parity import assert_topk_exact, to_dev

pytestmark = pytest.mark.gpu


def _logits(rng, rows, width, kind):
    if kind == "normal":
        x = (rng.standard_normal((rows, width)) * 10 + 70).astype(np.float32)
    elif kind == "ties":
        x = (rng.integers(-20, 21, (rows, width)) * 0.25).astype(np.float32)
        z = x == 0
        x[z] = np.where(rng.random(z.sum()) < 0.5, np.float32(-0.0), np.float32(0.0))
    elif kind == "all_equal":
        x = np.full((rows, width), 3.5, np.float32)
    elif kind == "wide_range":
        x = (rng.standard_normal((rows, width)) * np.exp(rng.uniform(-30, 30, (rows, width)))).astype(np.float32)
    elif kind == "trend":
        # rising along the row: the top keys crowd into the last part of a long row
        x = (np.arange(width, dtype=np.float64)[None, :] * 1e-3 + rng.standard_normal((rows, width))).astype(np.float32)
    elif kind == "neg_inf_mix":
        x = (rng.standard_normal((rows, width))).astype(np.float32)
        x[rng.random((rows, width)) < 0.3] = -np.inf
    else:
        raise ValueError(kind)
    return x


def _run_topk(x, ks, ke, k, width=None, map_=None, row0=0):
    g = F.indexer_topk(to_dev(x), to_dev(ke), k, ks=None if ks is None else to_dev(ks), width=width,
                       map=map_, row0=row0)
    torch.cuda.synchronize()
    return g.cpu().numpy()


@pytest.mark.parametrize("kind", ["normal", "ties", "all_equal", "wide_range", "neg_inf_mix"])
@pytest.mark.parametrize("rows,width,k", [(7, 300, 16), (40, 4096, 512), (3, 5000, 2048), (5, 70000, 100),
                                          (2, 140000, 2048), (1200, 2000, 64),
                                          # few long rows: one 512-thread workgroup per whole row
                                          (48, 131072, 2048), (9, 131072, 2800), (512, 20000, 64),
                                          (30, 16385, 2048)])
def test_topk_exact(kind, rows, width, k):
    rng = np.random.default_rng(rows * 7 + width + k)
    x = _logits(rng, rows, width, kind)
    ks = rng.integers(0, max(1, width // 4), rows).astype(np.int32)
    ke = np.minimum(width, ks + rng.integers(width // 2, width + 1, rows)).astype(np.int32)
    ke[0] = ks[0] + min(k // 2, width - ks[0])    # a window shorter than k: -1 padding
    if rows > 1:
        ke[1] = ks[1]                              # empty window
    g = _run_topk(x, ks, ke, k)
    e = topk_indices(x, ks, ke, k)
    assert_topk_exact(g, e, what=f"{kind} rows{rows} width{width} k{k}")
    # this library writes the selected keys in ascending index order
    for r in range(rows):
        sel = g[r][g[r] >= 0]
        assert np.all(np.diff(sel) > 0)


def test_topk_without_ks_and_row_stride():
    rng = np.random.default_rng(1)
    base = _logits(rng, 9, 1200, "normal")
    x = torch.from_numpy(base).cuda()[:, :1000]          # ld 1200, width 1000 (strided view)
    ke = np.full(9, 1000, np.int32)
    g = F.indexer_topk(x, to_dev(ke), 50, width=1000)
    torch.cuda.synchronize()
    e = topk_indices(base[:, :1000], np.zeros(9, np.int64), ke, 50)
    assert_topk_exact(g.cpu().numpy(), e)


def test_token_table_map_with_cu_rows_and_row0():
    rng = np.random.default_rng(2)
    rows, width, k = 30, 800, 40
    x = _logits(rng, rows, width, "normal")
    cu = np.array([0, 5, 17, 30, 45], np.int32)   # global rows; this call sees rows 10..39
    row0 = 10
    ks = rng.integers(0, 200, rows).astype(np.int32)
    ke = np.minimum(width, ks + 400).astype(np.int32)
    table = rng.permutation(4 * 1000).astype(np.int32).reshape(4, 1000)
    m = F.TopkMap(kind=F.MAP_TOKEN_TABLE, table=to_dev(table), cu_rows=to_dev(cu))
    g = _run_topk(x, ks, ke, k, map_=m, row0=row0)
    raw = topk_indices(x, ks, ke, k)
    # expected map of the oracle's selection, computed with global row ids
    ks_glob = np.zeros(row0 + rows, np.int64)
    ks_glob[row0:] = ks
    e = map_token_table(raw, list(range(row0, row0 + rows)), ks_glob, cu, table)
    for r in range(rows):
        assert set(g[r].tolist()) == set(e[r].tolist())


def test_block_table_map():
    rng = np.random.default_rng(3)
    B, nn, width, k = 4, 3, 700, 32
    rows = B * nn
    x = _logits(rng, rows, width, "normal")
    ke = rng.integers(100, width + 1, rows).astype(np.int32)
    max_pages = (width + 63) // 64
    bt = rng.permutation(200)[: B * max_pages].astype(np.int32).reshape(B, max_pages)
    m = F.TopkMap(kind=F.MAP_BLOCK_TABLE, table=to_dev(bt), rows_per_req=nn, page_size=64, num_pages=200)
    g = _run_topk(x, None, ke, k, map_=m)
    raw = topk_indices(x, np.zeros(rows, np.int64), ke, k)
    e = map_block_table(raw, list(range(rows)), nn, bt, 64)
    for r in range(rows):
        assert set(g[r].tolist()) == set(e[r].tolist())


def test_topk_determinism():
    rng = np.random.default_rng(4)
    x = _logits(rng, 64, 90000, "ties")
    ke = np.full(64, 90000, np.int32)
    a = _run_topk(x, None, ke, 2048)
    b = _run_topk(x, None, ke, 2048)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("kind", ["normal", "ties", "wide_range"])
@pytest.mark.parametrize("rows,width,k", [(3, 40000, 3000), (50, 20000, 8192), (2, 70000, 16384),
                                          (4, 16384, 16384)])
def test_topk_large_k(kind, rows, width, k):
    # k past ~2800 selects with the 16384-entry candidate list; k = 16384 is the largest supported
    rng = np.random.default_rng(rows + width + k)
    x = _logits(rng, rows, width, kind)
    ks = np.zeros(rows, np.int32)
    ke = np.full(rows, width, np.int32)
    ke[0] = min(width, k - 5)                      # fewer keys than k
    g = _run_topk(x, ks, ke, k)
    assert_topk_exact(g, topk_indices(x, ks, ke, k), what=f"{kind} rows{rows} width{width} k{k}")


@pytest.mark.parametrize("col0,ld", [(1, 1003), (3, 5003), (0, 5001), (1, 40003), (2, 131075)])
def test_topk_unaligned_rows(col0, ld):
    # rows that do not start on 16 bytes take the 4-byte load path
    rng = np.random.default_rng(col0 + ld)
    rows, width, k = 6, ld - col0 - 2, 200
    base = _logits(rng, rows, ld, "normal")
    x = torch.from_numpy(base).cuda()[:, col0:col0 + width]
    ks = rng.integers(0, 50, rows).astype(np.int32)
    ke = np.full(rows, width, np.int32)
    g = F.indexer_topk(x, to_dev(ke), k, ks=to_dev(ks), width=width)
    torch.cuda.synchronize()
    e = topk_indices(base[:, col0:col0 + width], ks, ke, k)
    assert_topk_exact(g.cpu().numpy(), e, what=f"col0 {col0} ld {ld}")


@pytest.mark.parametrize("kind", ["normal", "trend", "ties", "wide_range", "neg_inf_mix"])
def test_topk_long_rows_value_mixes(kind):
    """Few long rows (the one-workgroup-per-row path) over value distributions that stress the sampled
    threshold: rising along the row (trend), heavy ties, a huge dynamic range and -inf runs.  Window
    lengths range from under k to the full 131072 keys at unaligned starts; three calls on two inputs
    share one workspace."""
    rng = np.random.default_rng(4242)
    rows, width, k = 64, 131072, 2048
    x = _logits(rng, rows, width, kind)
    lens = np.array([32768, 32769, 65536, 65537, 98304, 98305, 131072, 1000, 2048, 40000, 131071, 100003]
                    * 6)[:rows - 4]
    lens = np.concatenate([lens, rng.integers(2049, width + 1, 4)])
    ks = np.array([int(rng.integers(0, width - l + 1)) for l in lens], np.int32)
    ke = (ks + lens).astype(np.int32)
    need = F.fp8idx_workspace_bytes(F.OP_TOPK, rows, width, k, 0)
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    # a second input through the same workspace
    x2 = x[::-1].copy() if kind != "trend" else x[:, ::-1].copy()
    xd, x2d, ksd, ked = to_dev(x), to_dev(x2), to_dev(ks), to_dev(ke)
    g1 = F.indexer_topk(xd, ked, k, ks=ksd, workspace=ws)
    g2 = F.indexer_topk(x2d, ked, k, ks=ksd, workspace=ws)
    g3 = F.indexer_topk(xd, ked, k, ks=ksd, workspace=ws)
    torch.cuda.synchronize()
    assert_topk_exact(g1.cpu().numpy(), topk_indices(x, ks, ke, k), what=f"long rows {kind}")
    assert_topk_exact(g2.cpu().numpy(), topk_indices(x2, ks, ke, k), what=f"long rows {kind}, second input")
    assert torch.equal(g1, g3)
    for g in (g1.cpu().numpy(), g2.cpu().numpy()):
        for r in range(rows):
            sel = g[r][g[r] >= 0]
            assert np.all(np.diff(sel) > 0)

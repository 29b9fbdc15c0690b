"""The boundary without a GPU: fp8idx_validate_only agrees with every entry point's own
host-side check, the top-k plan refuses merges deeper than its level limit, and the
Python binding rejects every mis-sized tensor with ValueError before anything reaches
the C ABI (which takes bare pointers and cannot see sizes)."""

import ctypes
import os

import pytest
import torch

import fp8_mqa_logits_amd as F
from fp8_mqa_logits_amd import binding

OK, EINVAL, EUNSUP, EWS, EDEV = 0, 1, 2, 3, 4
P = 1 << 20           # an aligned non-null fake device address; never dereferenced
S1, S2 = P, P + 4096  # two distinct fake stream handles


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from fp8_mqa_logits_amd.build import build
        build()
    return F.load_library()


# ---------------------------------------------------------------------------
# fp8idx_validate_only
# ---------------------------------------------------------------------------

def _ragged_args(**kw):
    a = binding.CallArgs(q=P, kv=P, kv_scale=P, weights=P, ks=P, ke=P, m=10, n=1000, H=32, D=128,
                         logits=P, ld_logits=1000, clean=1, ws=P, ws_bytes=256)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _paged_args(**kw):
    a = binding.CallArgs(q=P, kv=P, kv_scale=P, weights=P, row_len=P, block_table=P, B=2, next_n=4, H=32,
                         D=128, page_size=64, max_pages=4, num_pages=10, width=256, logits=P, ld_logits=256,
                         clean=1, k=64, map_to_slots=1, out=P, ld_out=64)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _topk_args(**kw):
    a = binding.CallArgs(scores=P, ld_logits=100, rows=3, width=100, ks=P, ke=P, k=10, row0=0, out=P, ld_out=10)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _call_entry(lib, entry, a):
    """Run the real entry point with the struct's fields (no device here, so valid args give EDEV)."""
    mp = ctypes.c_void_p(a.map) if a.map else None
    if entry == binding.ENTRY_LOGITS_RAGGED:
        return lib.indexer_logits_ragged(a.q, a.kv, a.kv_scale, a.weights, a.ks, a.ke, a.m, a.n, a.H, a.D, a.logits,
                                         a.ld_logits, a.clean, a.ws, a.ws_bytes, a.stream)
    if entry == binding.ENTRY_LOGITS_PAGED:
        return lib.indexer_logits_paged(a.q, a.kv, a.kv_scale, a.weights, a.row_len, a.block_table, a.B, a.next_n,
                                        a.H, a.D, a.page_size, a.max_pages, a.num_pages, a.logits, a.ld_logits,
                                        a.width, a.clean, a.stream)
    if entry == binding.ENTRY_TOPK:
        return lib.indexer_topk(a.scores, a.ld_logits, a.rows, a.width, a.ks, a.ke, a.k, a.row0, mp, a.out,
                                a.ld_out, a.ws, a.ws_bytes, a.stream)
    if entry == binding.ENTRY_LOGITS_TOPK_RAGGED:
        return lib.indexer_logits_topk_ragged(a.q, a.kv, a.kv_scale, a.weights, a.ks, a.ke, a.m, a.n, a.H, a.D,
                                              a.k, mp, a.out, a.ld_out, a.logits_cap_bytes, a.ws, a.ws_bytes,
                                              a.stream)
    if entry == binding.ENTRY_LOGITS_TOPK_RAGGED_OVERLAP:
        return lib.indexer_logits_topk_ragged_overlap(a.q, a.kv, a.kv_scale, a.weights, a.ks, a.ke, a.m, a.n, a.H,
                                                      a.D, a.k, mp, a.out, a.ld_out, a.logits_cap_bytes, a.ws,
                                                      a.ws_bytes, a.stream, a.side_stream)
    if entry == binding.ENTRY_LOGITS_TOPK_PAGED:
        return lib.indexer_logits_topk_paged(a.q, a.kv, a.kv_scale, a.weights, a.row_len, a.block_table, a.B,
                                             a.next_n, a.H, a.D, a.page_size, a.max_pages, a.num_pages, a.width,
                                             a.k, a.map_to_slots, a.out, a.ld_out, a.logits_cap_bytes, a.ws,
                                             a.ws_bytes, a.stream)
    raise AssertionError(entry)


def _fused_args(lib, overlap=False, **kw):
    a = _ragged_args(k=64, out=P, ld_out=64, logits_cap_bytes=4 * 1000 * 4, stream=S1,
                     side_stream=S2 if overlap else None)
    op = binding.OP_LOGITS_TOPK_RAGGED_OVERLAP if overlap else binding.OP_LOGITS_TOPK_RAGGED
    a.ws_bytes = lib.fp8idx_workspace_bytes(op, 10, 1000, 64, a.logits_cap_bytes)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


# (entry, builder, {field: bad value}, expected status)
CASES = [
    (binding.ENTRY_LOGITS_RAGGED, "ragged", {}, OK),
    (binding.ENTRY_LOGITS_RAGGED, "ragged", {"H": 16}, EUNSUP),
    (binding.ENTRY_LOGITS_RAGGED, "ragged", {"D": 64}, EUNSUP),
    (binding.ENTRY_LOGITS_RAGGED, "ragged", {"q": None}, EINVAL),
    (binding.ENTRY_LOGITS_RAGGED, "ragged", {"q": P + 8}, EINVAL),
    (binding.ENTRY_LOGITS_RAGGED, "ragged", {"ld_logits": 999}, EINVAL),
    (binding.ENTRY_LOGITS_RAGGED, "ragged", {"n": 0}, EINVAL),
    (binding.ENTRY_LOGITS_RAGGED, "ragged", {"ws": None}, EWS),
    (binding.ENTRY_LOGITS_RAGGED, "ragged", {"ws_bytes": 128}, EWS),
    (binding.ENTRY_LOGITS_RAGGED, "ragged", {"ws": P + 64}, EINVAL),
    (binding.ENTRY_LOGITS_RAGGED, "ragged", {"m": 0, "q": None, "ws": None}, OK),
    (binding.ENTRY_LOGITS_PAGED, "paged", {}, OK),
    (binding.ENTRY_LOGITS_PAGED, "paged", {"page_size": 32}, EUNSUP),
    (binding.ENTRY_LOGITS_PAGED, "paged", {"width": 257}, EINVAL),
    (binding.ENTRY_LOGITS_PAGED, "paged", {"num_pages": 0}, EINVAL),
    (binding.ENTRY_LOGITS_PAGED, "paged", {"block_table": None}, EINVAL),
    (binding.ENTRY_LOGITS_PAGED, "paged", {"ld_logits": 255}, EINVAL),
    (binding.ENTRY_TOPK, "topk", {}, OK),
    (binding.ENTRY_TOPK, "topk", {"k": 0}, EUNSUP),
    (binding.ENTRY_TOPK, "topk", {"k": 16385}, EUNSUP),
    (binding.ENTRY_TOPK, "topk", {"ld_out": 9}, EINVAL),
    (binding.ENTRY_TOPK, "topk", {"width": 101}, EINVAL),
    (binding.ENTRY_TOPK, "topk", {"ke": None}, EINVAL),
    (binding.ENTRY_TOPK, "topk", {"ks": None}, OK),
    (binding.ENTRY_TOPK, "topk", {"rows": 2, "ld_logits": 200000, "width": 200000, "k": 2048, "ld_out": 2048}, EWS),
    (binding.ENTRY_TOPK, "topk", {"rows": 1, "ld_logits": 2**31 - 1, "width": 2**31 - 1, "k": 16384,
                                  "ld_out": 16384}, EUNSUP),
    (binding.ENTRY_LOGITS_TOPK_PAGED, "paged", {"ws": P, "ws_bytes": 1 << 40}, OK),
    (binding.ENTRY_LOGITS_TOPK_PAGED, "paged", {}, EWS),
    (binding.ENTRY_LOGITS_TOPK_PAGED, "paged", {"ws": P, "ws_bytes": 1 << 40, "ld_out": 63}, EINVAL),
]

_BUILD = {"ragged": _ragged_args, "paged": _paged_args, "topk": _topk_args}


@pytest.mark.parametrize("entry,kind,bad,want", CASES)
def test_validate_only_matches_entry(lib, entry, kind, bad, want):
    a = _BUILD[kind](**bad)
    got = F.fp8idx_validate_only(entry, a)
    assert got == want, (entry, bad, got)
    # the entry itself runs the same check first; valid arguments then look for a device (none here)
    via_entry = _call_entry(lib, entry, a)
    if want == OK and not (a.m == 0 and kind == "ragged" and a.q is None):
        assert via_entry == EDEV
    else:
        assert via_entry == want


@pytest.mark.parametrize("overlap", [False, True])
@pytest.mark.parametrize("bad,want", [({}, OK), ({"ws_bytes": 0}, EWS), ({"ws": P + 16}, EINVAL),
                                      ({"k": 0}, EUNSUP), ({"ld_out": 63}, EINVAL), ({"H": 64}, EUNSUP)])
def test_validate_only_fused_ragged(lib, overlap, bad, want):
    entry = binding.ENTRY_LOGITS_TOPK_RAGGED_OVERLAP if overlap else binding.ENTRY_LOGITS_TOPK_RAGGED
    a = _fused_args(lib, overlap, **bad)
    assert F.fp8idx_validate_only(entry, a) == want
    assert _call_entry(lib, entry, a) == (EDEV if want == OK else want)


def test_validate_only_overlap_streams(lib):
    a = _fused_args(lib, True, side_stream=S1)
    assert F.fp8idx_validate_only(binding.ENTRY_LOGITS_TOPK_RAGGED_OVERLAP, a) == EINVAL   # same stream
    a = _fused_args(lib, True, side_stream=None)
    assert F.fp8idx_validate_only(binding.ENTRY_LOGITS_TOPK_RAGGED_OVERLAP, a) == EINVAL


def test_validate_only_bad_calls(lib):
    assert lib.fp8idx_validate_only(binding.ENTRY_TOPK, None) == EINVAL
    assert F.fp8idx_validate_only(99, _topk_args()) == EINVAL


# ---------------------------------------------------------------------------
# top-k level limit
# ---------------------------------------------------------------------------

def test_topk_plan_level_limit(lib):
    # k = 16384 shrinks the candidates 4x per merge level: 2^30 keys still end in one segment at
    # the eighth level, 2^31 - 1 would need a ninth and is refused everywhere
    wide = 2**31 - 1
    assert lib.fp8idx_workspace_bytes(binding.OP_TOPK, 1, wide, 16384, 0) == 0
    assert F.fp8idx_validate_only(binding.ENTRY_TOPK, _topk_args(rows=1, ld_logits=wide, width=wide, k=16384,
                                                                  ld_out=16384)) == EUNSUP
    assert lib.fp8idx_workspace_bytes(binding.OP_TOPK, 1, 2**30, 16384, 0) > 0
    a = _topk_args(rows=1, ld_logits=2**30, width=2**30, k=16384, ld_out=16384, ws=P, ws_bytes=1 << 50)
    assert F.fp8idx_validate_only(binding.ENTRY_TOPK, a) == OK


# ---------------------------------------------------------------------------
# binding size checks (CPU tensors: every shape check runs before the device check)
# ---------------------------------------------------------------------------

def _ragged_cpu(m=6, n=50):
    return dict(q=torch.zeros((m, 32, 128), dtype=torch.uint8), kv=torch.zeros((n, 128), dtype=torch.uint8),
                kv_scale=torch.ones(n), weights=torch.ones((m, 32)), ks=torch.zeros(m, dtype=torch.int32),
                ke=torch.full((m,), n, dtype=torch.int32))


def _paged_cpu(B=2, nn=4, pages=6, mp=3):
    return dict(q=torch.zeros((B, nn, 32, 128), dtype=torch.uint8),
                kv_pool=torch.zeros((pages, 64, 128), dtype=torch.uint8),
                scale_pool=torch.ones((pages, 64)), weights=torch.ones((B * nn, 32)),
                row_len=torch.full((B * nn,), 100, dtype=torch.int32),
                block_table=torch.zeros((B, mp), dtype=torch.int32))


RAGGED_BAD = [
    ("kv_scale", torch.ones(49), "kv_scale must be 1-D with 50"),
    ("kv_scale", torch.ones((50, 1)), "kv_scale must be 1-D"),
    ("weights", torch.ones((6, 31)), "weights must have shape (6, 32)"),
    ("weights", torch.ones((5, 32)), "weights must have shape (6, 32)"),
    ("ks", torch.zeros(5, dtype=torch.int32), "ks must be 1-D with 6"),
    ("ke", torch.zeros(7, dtype=torch.int32), "ke must be 1-D with 6"),
    ("q", torch.zeros((6, 16, 128), dtype=torch.uint8), "q must be [m, 32, 128]"),
    ("kv", torch.zeros((50, 64), dtype=torch.uint8), "kv must be [n, 128]"),
    ("ke", torch.zeros(6, dtype=torch.int64), "ke: dtype"),
]


@pytest.mark.parametrize("name,value,msg", RAGGED_BAD)
@pytest.mark.parametrize("fn", ["logits", "fused", "overlap"])
def test_binding_ragged_sizes(name, value, msg, fn):
    a = _ragged_cpu()
    a[name] = value
    args = [a[k] for k in ("q", "kv", "kv_scale", "weights", "ks", "ke")]
    with pytest.raises(ValueError, match=msg.replace("[", r"\[").replace("(", r"\(").replace(")", r"\)")):
        if fn == "logits":
            F.indexer_logits_ragged(*args)
        elif fn == "fused":
            F.indexer_logits_topk_ragged(*args, 8)
        else:
            F.indexer_logits_topk_ragged_overlap(*args, 8, side_stream=None)


def test_binding_ragged_output_sizes():
    a = _ragged_cpu()
    args = [a[k] for k in ("q", "kv", "kv_scale", "weights", "ks", "ke")]
    with pytest.raises(ValueError, match="logits must be"):
        F.indexer_logits_ragged(*args, logits=torch.empty((5, 50)))
    with pytest.raises(ValueError, match="logits must be"):
        F.indexer_logits_ragged(*args, logits=torch.empty((6, 49)))
    with pytest.raises(ValueError, match="out must be"):
        F.indexer_logits_topk_ragged(*args, 8, out=torch.empty((5, 8), dtype=torch.int32))
    with pytest.raises(ValueError, match="out must be"):
        F.indexer_logits_topk_ragged(*args, 8, out=torch.empty((6, 7), dtype=torch.int32))
    # right sizes on the host: the last check is the device
    with pytest.raises(ValueError, match="device tensor"):
        F.indexer_logits_ragged(*args)


PAGED_BAD = [
    ("scale_pool", torch.ones((6, 63)), "scale_pool must hold pages"),
    ("scale_pool", torch.ones((5, 64)), "scale_pool must hold pages"),
    ("weights", torch.ones((7, 32)), "weights must have shape (8, 32)"),
    ("row_len", torch.zeros(7, dtype=torch.int32), "row_len must be 1-D with 8"),
    ("block_table", torch.zeros((1, 3), dtype=torch.int32), "block_table must be"),
    ("block_table", torch.zeros((2, 1), dtype=torch.int32), "width must lie in"),
    ("kv_pool", torch.zeros((6, 64, 64), dtype=torch.uint8), "kv_pool must be"),
    ("q", torch.zeros((8, 32, 128), dtype=torch.uint8), "q must be"),
]


@pytest.mark.parametrize("name,value,msg", PAGED_BAD)
@pytest.mark.parametrize("fused", [False, True])
def test_binding_paged_sizes(name, value, msg, fused):
    a = _paged_cpu()
    a[name] = value
    args = [a[k] for k in ("q", "kv_pool", "scale_pool", "weights", "row_len", "block_table")]
    with pytest.raises(ValueError, match=msg.replace("(", r"\(").replace(")", r"\)")):
        if fused:
            F.indexer_logits_topk_paged(*args, 16, width=192)
        else:
            F.indexer_logits_paged(*args, width=192)


def test_binding_paged_output_sizes():
    a = _paged_cpu()
    args = [a[k] for k in ("q", "kv_pool", "scale_pool", "weights", "row_len", "block_table")]
    with pytest.raises(ValueError, match="logits must be"):
        F.indexer_logits_paged(*args, width=192, logits=torch.empty((8, 191)))
    with pytest.raises(ValueError, match="out must be"):
        F.indexer_logits_topk_paged(*args, 16, width=192, out=torch.empty((7, 16), dtype=torch.int32))
    with pytest.raises(ValueError, match="device tensor"):
        F.indexer_logits_paged(*args, width=192)


def test_binding_topk_sizes():
    lg = torch.zeros((4, 100))
    ke = torch.full((4,), 100, dtype=torch.int32)
    with pytest.raises(ValueError, match="ke must be 1-D with 4"):
        F.indexer_topk(lg, ke[:3], 8)
    with pytest.raises(ValueError, match="ks must be 1-D with 4"):
        F.indexer_topk(lg, ke, 8, ks=torch.zeros(5, dtype=torch.int32))
    with pytest.raises(ValueError, match="width must lie in"):
        F.indexer_topk(lg, ke, 8, width=101)
    with pytest.raises(ValueError, match="out must be"):
        F.indexer_topk(lg, ke, 8, out=torch.empty((4, 7), dtype=torch.int32))
    with pytest.raises(ValueError, match="unit column stride"):
        F.indexer_topk(lg.t(), ke, 8)
    tok = F.TopkMap(kind=F.MAP_TOKEN_TABLE, table=torch.zeros((3, 100), dtype=torch.int32),
                    cu_rows=torch.zeros(3, dtype=torch.int32))
    with pytest.raises(ValueError, match="cu_rows must be 1-D with 4"):
        F.indexer_topk(lg, ke, 8, map=tok)
    blk = F.TopkMap(kind=F.MAP_BLOCK_TABLE, table=torch.zeros((1, 2), dtype=torch.int32), rows_per_req=4,
                    page_size=64)
    with pytest.raises(ValueError, match="num_pages"):
        F.indexer_topk(lg, ke, 8, map=blk)
    with pytest.raises(ValueError, match="device tensor"):
        F.indexer_topk(lg, ke, 8)


def test_binding_prep_sizes():
    i32 = lambda *s: torch.zeros(s, dtype=torch.int32)
    with pytest.raises(ValueError, match="q_len must be 1-D with 3"):
        F.indexer_prepare_ragged(i32(3), i32(2), i32(3), i32(3, 10), max_q=8)
    with pytest.raises(ValueError, match="req_idx must be 1-D with 3"):
        F.indexer_prepare_ragged(i32(3), i32(3), i32(4), i32(3, 10), max_q=8)
    with pytest.raises(ValueError, match="req_idx must be 1-D with 3"):
        F.indexer_prepare_decode(i32(3), i32(2), i32(3, 10), 4)
    with pytest.raises(ValueError, match="max_pages must lie in"):
        F.indexer_prepare_decode(i32(3), i32(3), i32(3, 10), 4, max_pages=11)

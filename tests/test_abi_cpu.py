"""The C ABI without a GPU: every declared symbol is exported, host-side validation
returns the documented status before touching any pointer, and the workspace /
chunking arithmetic follows the chunking page's formula."""

import ctypes
import os
import re

import pytest

import fp8_mqa_logits_amd as F
from fp8_mqa_logits_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8idx.h")

OK, EINVAL, EUNSUP, EWS, EDEV, EHIP = 0, 1, 2, 3, 4, 5
P = 1 << 20          # an aligned non-null fake device address; validation never dereferences it
NULL = None


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from fp8_mqa_logits_amd.build import build
        build()
    return F.load_library()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"FP8IDX_API\s+[\w\s\*]+?\b((?:indexer|fp8idx)_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) == 21, names
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(binding.EXPORTED) == names


def test_status_strings(lib):
    for s in range(6):
        assert lib.fp8idx_status_string(s).decode().startswith("FP8IDX")
    assert b"unknown" in lib.fp8idx_status_string(99)
    assert lib.fp8idx_version().decode().startswith("fp8idx")


def _ragged(lib, q=P, kv=P, sc=P, w=P, ks=P, ke=P, m=4, n=64, H=32, D=128, lg=P, ld=64, clean=1, ws=P, wsb=256):
    return lib.indexer_logits_ragged(q, kv, sc, w, ks, ke, m, n, H, D, lg, ld, clean, ws, wsb, None)


def test_ragged_validation(lib):
    assert _ragged(lib, H=16) == EUNSUP
    assert _ragged(lib, D=64) == EUNSUP
    assert _ragged(lib, q=NULL) == EINVAL
    assert _ragged(lib, ke=NULL) == EINVAL
    assert _ragged(lib, lg=NULL) == EINVAL
    assert _ragged(lib, q=P + 8) == EINVAL        # q must be 16-byte aligned
    assert _ragged(lib, w=P + 4) == EINVAL        # weights are read as float4
    assert _ragged(lib, ks=P + 2) == EINVAL
    assert _ragged(lib, ld=63) == EINVAL          # ld < n
    assert _ragged(lib, m=-1) == EINVAL
    assert _ragged(lib, n=0) == EINVAL
    assert _ragged(lib, m=0, q=NULL, lg=NULL, ws=NULL, wsb=0) == OK   # empty call is a no-op
    # the work-queue counters come from the workspace: 256 bytes, 256-byte aligned
    assert lib.fp8idx_workspace_bytes(binding.OP_LOGITS_RAGGED, 4, 64, 1, 0) == 256
    assert _ragged(lib, ws=NULL, wsb=0) == EWS
    assert _ragged(lib, wsb=255) == EWS
    assert _ragged(lib, ws=P + 128) == EINVAL
    # the allocation-free variant: the same checks without a workspace
    nf = lambda **kw: lib.indexer_logits_ragged_noalloc(*[kw.get(k, P) for k in ("q", "kv", "sc", "w", "ks", "ke")],
                                                        kw.get("m", 4), 64, kw.get("H", 32), 128,
                                                        kw.get("lg", P), kw.get("ld", 64), 1, None)
    assert nf(H=16) == EUNSUP
    assert nf(q=NULL) == EINVAL
    assert nf(lg=NULL) == EINVAL
    assert nf(ld=63) == EINVAL
    assert nf(m=0, q=NULL, lg=NULL) == OK
    assert nf() == EDEV
    # valid arguments but no gfx950 device in this process
    assert _ragged(lib) == EDEV


def _paged(lib, q=P, pool=P, sp=P, w=P, rl=P, bt=P, B=2, nn=4, H=32, D=128, page=64, maxp=4, npages=10,
           lg=P, ld=256, width=256, clean=1):
    return lib.indexer_logits_paged(q, pool, sp, w, rl, bt, B, nn, H, D, page, maxp, npages, lg, ld, width,
                                    clean, None)


def test_paged_validation(lib):
    assert _paged(lib, page=32) == EUNSUP
    assert _paged(lib, H=64) == EUNSUP
    assert _paged(lib, width=257) == EINVAL       # past max_pages * page_size
    assert _paged(lib, ld=128) == EINVAL
    assert _paged(lib, nn=0) == EINVAL
    assert _paged(lib, bt=NULL) == EINVAL
    assert _paged(lib, pool=P + 4) == EINVAL
    assert _paged(lib, npages=1 << 26) == EUNSUP  # slot ids would not fit int32
    assert _paged(lib, B=0, q=NULL) == OK
    assert _paged(lib) == EDEV


def _topk(lib, lg=P, ld=100, rows=3, width=100, ks=P, ke=P, k=10, row0=0, mp=None, out=P, ldo=10,
          ws=None, wsb=0):
    return lib.indexer_topk(lg, ld, rows, width, ks, ke, k, row0, mp, out, ldo, ws, wsb, None)


def test_topk_validation(lib):
    assert _topk(lib, k=0) == EUNSUP
    assert _topk(lib, k=16385) == EUNSUP
    assert _topk(lib, ldo=9) == EINVAL
    assert _topk(lib, width=101) == EINVAL
    assert _topk(lib, ke=NULL) == EINVAL
    assert _topk(lib, ks=NULL) == EDEV            # ks is optional
    bad = binding._CMap()
    bad.kind = 7
    assert _topk(lib, mp=ctypes.byref(bad)) == EINVAL
    tok = binding._CMap()
    tok.kind = binding.MAP_TOKEN_TABLE
    assert _topk(lib, mp=ctypes.byref(tok)) == EINVAL     # no table
    tok.table, tok.ld, tok.num_req = P, 8, 2
    assert _topk(lib, mp=ctypes.byref(tok)) == EDEV
    blk = binding._CMap()
    blk.kind, blk.table, blk.ld, blk.num_req, blk.rows_per_req, blk.page_size = binding.MAP_BLOCK_TABLE, P, 4, 2, 0, 64
    blk.num_pages = 100
    assert _topk(lib, mp=ctypes.byref(blk)) == EINVAL     # rows_per_req < 1
    blk.rows_per_req = 4
    assert _topk(lib, mp=ctypes.byref(blk)) == EDEV
    blk.num_pages = 0
    assert _topk(lib, mp=ctypes.byref(blk)) == EINVAL     # the pool's page count bounds page ids
    # a split plan needs workspace: few rows of a long window
    need = lib.fp8idx_workspace_bytes(binding.OP_TOPK, 2, 200000, 2048, 0)
    assert need > 0
    assert _topk(lib, rows=2, ld=200000, width=200000, k=2048, ldo=2048) == EWS
    assert _topk(lib, rows=2, ld=200000, width=200000, k=2048, ldo=2048, ws=P + 64, wsb=need) == EINVAL
    assert _topk(lib, rows=2, ld=200000, width=200000, k=2048, ldo=2048, ws=P, wsb=need) == EDEV


def test_fused_validation(lib):
    f = lib.indexer_logits_topk_ragged
    args = [P, P, P, P, P, P, 10, 1000, 32, 128, 64, None, P, 64, 0, P, 0, None]
    need = lib.fp8idx_workspace_bytes(binding.OP_LOGITS_TOPK_RAGGED, 10, 1000, 64, 0)
    assert need >= 10 * 1000 * 4
    assert f(*args) == EWS
    args[16] = need
    assert f(*args) == EDEV
    args[15] = P + 16
    assert f(*args) == EINVAL                    # workspace must be 256-byte aligned
    g = lib.indexer_logits_topk_paged
    pargs = [P, P, P, P, P, P, 2, 4, 32, 128, 64, 4, 10, 256, 64, 1, P, 64, 0, P, 0, None]
    assert g(*pargs) == EWS
    pargs[20] = lib.fp8idx_workspace_bytes_paged(2, 4, 256, 64, 0)
    assert g(*pargs) == EDEV
    # the size query answers 0 where the entry rejects the rows (B * next_n past int32)
    assert lib.fp8idx_workspace_bytes_paged(1 << 20, 1 << 12, 256, 64, 0) == 0
    assert lib.fp8idx_workspace_bytes_paged(2, 0, 256, 64, 0) == 0


def test_rows_per_chunk_follows_chunking_page(lib):
    # rows per chunk = max(1, int(gb * 1e9) // (n * 4)); n is a multiple of 4 in all of these
    assert F.fp8idx_rows_per_chunk(2_000_000_000, 210000, 7500) == 2380
    assert F.fp8idx_rows_per_chunk(2_000_000_000, 65536, 8192) == 7629
    assert F.fp8idx_rows_per_chunk(8_000_000_000, 65536, 8192) == 8192
    assert F.fp8idx_rows_per_chunk(500_000_000, 150000 + 4096, 512) == 512
    assert F.fp8idx_rows_per_chunk(1, 65536, 8192) == 1
    assert F.fp8idx_rows_per_chunk(0, 65536, 8192) == 8192
    # non-multiple of 4: the workspace row stride is rounded up to 4 floats
    assert F.fp8idx_rows_per_chunk(4004 * 4 * 10, 4001, 100) == 10


def test_fused_workspace_covers_chunk_and_candidates(lib):
    cap = 2_000_000_000
    ws = F.fp8idx_workspace_bytes(F.OP_LOGITS_TOPK_RAGGED, 7500, 210000, 2048, cap)
    # the cap allows 2380 rows per chunk: 4 chunks, so 1875 rows each
    logits = 1875 * 210000 * 4
    cand = 1875 * 3 * 2048 * 8          # 3 segments of 70000 keys per row
    assert ws >= logits + cand
    assert ws <= logits + cand + 4096
    # one-shot on 8192 x 65536: the work-queue counters and the full 2 GiB buffer, single-segment top-k
    assert F.fp8idx_workspace_bytes(F.OP_LOGITS_TOPK_RAGGED, 8192, 65536, 2048, 0) == 256 + 8192 * 65536 * 4


def test_fused_paged_workspace_holds_fragment_maxima(lib):
    # decode: 256 rows of 131072 keys, one top-k workgroup per row -> the chunk's logits, then one word
    # per row and 16-key fragment, and no top-k candidates
    assert F.fp8idx_workspace_bytes_paged(64, 4, 131072, 2048, 0) == 256 * 131072 * 4 + 256 * 8192 * 4
    # rows longer than one workgroup takes (segmented top-k): no fragment maxima, the top-k's own
    # candidate buffers instead
    ws = F.fp8idx_workspace_bytes_paged(4, 4, 200000, 2048, 0)
    assert ws == 16 * 200000 * 4 + F.fp8idx_workspace_bytes(F.OP_TOPK, 16, 200000, 2048, 0)


def test_quant_validation(lib):
    f = lib.indexer_quant_fp8
    assert f(P, 128, 4, 130, P, 132, P, None) == EUNSUP      # D % 4 != 0
    assert f(P, 4096, 4, 4096, P, 4096, P, None) == EUNSUP   # D > 2048
    assert f(P, 128, -1, 128, P, 128, P, None) == EINVAL
    assert f(NULL, 128, 0, 128, NULL, 128, NULL, None) == OK  # empty call is a no-op
    assert f(NULL, 128, 4, 128, P, 128, P, None) == EINVAL
    assert f(P + 4, 128, 4, 128, P, 128, P, None) == EINVAL  # x rows are read as 16-byte vectors
    assert f(P, 126, 4, 128, P, 128, P, None) == EINVAL      # ld_x < D
    assert f(P, 130, 4, 128, P, 128, P, None) == EINVAL      # ld_x % 4 != 0
    assert f(P, 128, 4, 128, P + 2, 128, P, None) == EINVAL  # codes written as 4-byte words
    assert f(P, 128, 4, 128, P, 130, P, None) == EINVAL
    assert f(P, 128, 4, 128, P, 128, P, None) == EDEV


def test_overlap_validation(lib):
    f = lib.indexer_logits_topk_ragged_overlap
    S1, S2 = P, P + 4096                                  # two distinct fake stream handles
    cap = 4 * 1000 * 4                                    # 4 rows per chunk: chunks of 4, 4, 2 rows
    args = [P, P, P, P, P, P, 10, 1000, 32, 128, 64, None, P, 64, cap, None, 0, S1, S2]
    need = lib.fp8idx_workspace_bytes(binding.OP_LOGITS_TOPK_RAGGED_OVERLAP, 10, 1000, 64, cap)
    one = lib.fp8idx_workspace_bytes(binding.OP_LOGITS_TOPK_RAGGED, 10, 1000, 64, cap)
    # two chunk buffers (each 16000 bytes rounded up to 256) instead of one
    assert need == one + 16128
    assert f(*args) == EWS
    args[15], args[16] = P, need
    bad = list(args); bad[18] = S1
    assert f(*bad) == EINVAL                              # side stream must differ from the stream
    bad = list(args); bad[18] = None
    assert f(*bad) == EINVAL
    assert f(*args) == EDEV
    # one chunk needs only one buffer
    assert lib.fp8idx_workspace_bytes(binding.OP_LOGITS_TOPK_RAGGED_OVERLAP, 10, 1000, 64, 0) == \
        lib.fp8idx_workspace_bytes(binding.OP_LOGITS_TOPK_RAGGED, 10, 1000, 64, 0)


def test_prepare_validation(lib):
    f = lib.indexer_prepare_ragged
    #        seq q  req table ld rows B  cu_s cu_q ks ke max_q mem max_keys
    ok = [P, P, P, P, 64, 4, 3, P, P, P, P, 10, P, 100, None]
    assert f(*ok) == EDEV
    bad = list(ok); bad[6] = 4097
    assert f(*bad) == EUNSUP                               # more requests than one call scans
    bad = list(ok); bad[6] = -1
    assert f(*bad) == EINVAL
    bad = list(ok); bad[9] = None
    assert f(*bad) == EINVAL                               # ks needed when max_q > 0
    bad = list(ok); bad[3] = None
    assert f(*bad) == EINVAL                               # the copy needs the table
    bad = list(ok); bad[3], bad[12] = None, None
    assert f(*bad) == EDEV                                 # ... unless it is skipped
    bad = list(ok); bad[7] = P + 2
    assert f(*bad) == EINVAL
    bad = list(ok); bad[6] = 0
    assert f(*bad) == OK
    g = lib.indexer_prepare_decode
    okd = [P, P, P, 32, 4, 3, 4, P, P, 32, None]
    assert g(*okd) == EDEV
    bad = list(okd); bad[6] = 0
    assert g(*bad) == EINVAL                               # next_n >= 1
    bad = list(okd); bad[3] = 16
    assert g(*bad) == EINVAL                               # table rows shorter than max_pages
    bad = list(okd); bad[5] = 0
    assert g(*bad) == OK


def test_sparse_mla_validation(lib):
    f = lib.indexer_sparse_mla
    #      q  kv sc  S    idx  ld  T  H   D    Dv  topk scale out lse ws   wsb  stream
    ok = [P, P, P, 1000, P, 64, 4, 64, 576, 512, 64, 0.1, P, P, None, 0, None]

    def call(**kw):
        a = list(ok)
        names = ["q", "kv", "sc", "S", "idx", "ld", "T", "H", "D", "Dv", "topk", "scale", "out", "lse", "ws",
                 "wsb", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    need = lib.fp8idx_sparse_mla_workspace_bytes(4, 64, 64)
    assert need == 0                              # 4 tokens x 1 step of 64 keys: nothing to split
    assert call() == EDEV
    assert call(D=128) == EUNSUP and call(Dv=576) == EUNSUP
    assert call(H=24) == EUNSUP and call(H=0) == EUNSUP
    assert call(topk=0) == EINVAL
    assert call(ld=63) == EINVAL                  # ld_indices < topk
    assert call(S=0) == EINVAL                    # masked keys read slot 0, so the pool must hold one
    assert call(T=-1) == EINVAL
    assert call(T=0, q=NULL, kv=NULL, sc=NULL, idx=NULL, out=NULL) == OK
    assert call(q=NULL) == EINVAL and call(idx=NULL) == EINVAL and call(out=NULL) == EINVAL
    assert call(q=P + 8) == EINVAL                # q rows are read as 16-byte vectors
    assert call(out=P + 4) == EINVAL
    assert call(lse=P + 2) == EINVAL
    assert call(lse=NULL) == EDEV                 # lse is optional
    # few tokens split their lists: partial outputs of 513 floats per (token, split, head)
    need = lib.fp8idx_sparse_mla_workspace_bytes(2, 64, 2048)
    nsplit = 32                                   # 2048 keys in 64-key steps, 2 token groups -> 32 splits
    assert need == 2 * nsplit * 64 * 513 * 4 + 256
    assert call(T=2, topk=2048, ld=2048) == EWS
    assert call(T=2, topk=2048, ld=2048, ws=P + 16, wsb=need) == EINVAL   # 256-byte alignment
    assert call(T=2, topk=2048, ld=2048, ws=P, wsb=need) == EDEV
    assert lib.fp8idx_sparse_mla_workspace_bytes(256, 64, 2048) == 0     # one workgroup per token already


def test_mfma_probe_validation(lib):
    flops = ctypes.c_double(0.0)
    assert lib.fp8idx_probe_mfma_fp8(0, 8, P, ctypes.byref(flops), NULL) == EINVAL
    assert lib.fp8idx_probe_mfma_fp8(4, 0, P, ctypes.byref(flops), NULL) == EINVAL
    assert lib.fp8idx_probe_mfma_fp8(4, 8, NULL, ctypes.byref(flops), NULL) == EINVAL
    assert lib.fp8idx_probe_mfma_fp8(4, 8, P + 2, ctypes.byref(flops), NULL) == EINVAL
    assert lib.fp8idx_probe_mfma_fp8(4, 8, P, ctypes.byref(flops), NULL) == EDEV


def test_logits_core_probe_validation(lib):
    flops = ctypes.c_double(0.0)
    f = lib.fp8idx_probe_logits_core
    assert f(0, 8, P, ctypes.byref(flops), NULL) == EINVAL
    assert f(4, 0, P, ctypes.byref(flops), NULL) == EINVAL
    assert f(4, 8, NULL, ctypes.byref(flops), NULL) == EINVAL
    assert f(4, 8, P + 2, ctypes.byref(flops), NULL) == EINVAL
    assert f(4, 8, P, ctypes.byref(flops), NULL) == EDEV

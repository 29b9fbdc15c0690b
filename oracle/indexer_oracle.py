"""Float64 reference for the sparse-attention indexer hot path.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH: imported only by the
tests, by ``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of
``bench.py``.  Nothing here is shared with the HIP library.

What is computed (sources are the five pages; none of them writes the logit
formula out, so the formula below is the plain reading of the call
``fp8_mqa_logits(q, (kv, kv_scales), weights, ks, ke)`` used on the
bench_mqa_logits_chunking.py page and of the indexer described on the
vessl-ai/sglang PR #87 page):

    logits[i, j] = sum_h weights[i, h] * max(dot(q[i, h, :], kv[j, :]) * kv_scale[j], 0)
                   for ks[i] <= j < ke[i], and -inf elsewhere.

Then, per row, the indices of the k largest logits inside [ks, ke), padded
with -1 when the window holds fewer than k keys, mapped through a page
table (``fast_topk_transform_fused(score, lengths, page_table_size_1,
cu_seqlens_q, topk, row_starts)`` on the chunking page).

Readings where the pages are silent (each is also listed in the design notes):
* ties at the k-th value: the lower key index wins, so the selected set is
  unique; the output is a set (its order is not part of the contract), and
  this oracle returns it sorted by (value desc, index asc);
* ragged token-table position of key j for row i is ``j - ks[i]`` in the
  row's request (request found from ``cu_rows``);
* paged decode: key j of request b lives in physical slot
  ``block_table[b, j // page] * page + j % page``; a key whose page id lies
  outside the pool [0, pages) holds no kv (block tables carry -1 past a
  request's pages), so its logit is -inf and, when the top-k takes it (a row
  with fewer than k real keys), it maps to -1 like the padding.

Exactness: every e4m3fn code is an integer multiple of 2**-9 with magnitude
at most 448, so every product q*kv is a multiple of 2**-18 and a sum of 128
of them stays below 2**43 units of 2**-18 < 2**53.  The dot products are
therefore exact in float64 whatever order BLAS sums them in.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "e4m3fn_value_table", "decode_e4m3fn", "encode_e4m3fn", "scores", "mqa_logits",
    "gather_paged_kv", "paged_mqa_logits", "topk_indices", "map_token_table",
    "map_block_table", "ragged_topk_mapped", "paged_topk_mapped", "rows_per_chunk",
]


# ---------------------------------------------------------------------------
# fp8 e4m3fn codec, from the bit layout (OCP 8-bit float, E4M3 "fn" flavour:
# exponent bias 7, no infinities, S.1111.111 is NaN, max finite 448).  The
# vessl-ai/sglang PR #87 page tests an encoder against torch.float8_e4m3fn
# (round-to-nearest-even ties 1.0625, 1.1875, 15.5; subnormals; saturation to
# +-448; NaN); the same flavour is decoded here.
# ---------------------------------------------------------------------------

def e4m3fn_value_table() -> np.ndarray:
    """float64[256]: value of each e4m3fn byte, NaN for 0x7F and 0xFF."""
    t = np.empty(256, dtype=np.float64)
    for b in range(256):
        sign = -1.0 if (b >> 7) & 1 else 1.0
        e = (b >> 3) & 0xF
        f = b & 0x7
        if e == 0xF and f == 0x7:
            t[b] = math.nan
        elif e == 0:
            t[b] = sign * f * 2.0 ** -9          # subnormal: 0.f * 2**(1-7)
        else:
            t[b] = sign * (8 + f) * 2.0 ** (e - 10)  # 1.f * 2**(e-7)
    return t


_TABLE = e4m3fn_value_table()


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """Decode raw e4m3fn bytes (any shape, uint8) to float64."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode_e4m3fn(x: np.ndarray, saturate: bool = True) -> np.ndarray:
    """Round float values to e4m3fn bytes, nearest with ties to even mantissa.

    ``saturate``: magnitudes past the largest finite value (448) become +-448
    (the behaviour the PR #87 page pins for its software encoder); otherwise
    they become NaN (0x7F with the sign bit of x).  NaN input gives 0x7F.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    flat_x = x.reshape(-1)
    flat_o = out.reshape(-1)
    for idx in range(flat_x.size):
        v = float(flat_x[idx])
        if math.isnan(v):
            flat_o[idx] = 0x7F
            continue
        s = 0x80 if math.copysign(1.0, v) < 0 else 0
        a = abs(v)
        # candidate grid: scaled magnitude in units of the code's quantum
        if a < 2.0 ** -6:
            units = a / 2.0 ** -9                   # subnormal quantum 2**-9
            f = _round_half_even(units)             # 0..8; 8 is the smallest normal
            code = f                                # f == 8 encodes e=1, f=0
        else:
            e = math.floor(math.log2(a))
            # guard against log2 rounding at exact powers of two
            if 2.0 ** e > a:
                e -= 1
            elif 2.0 ** (e + 1) <= a:
                e += 1
            mant = a / 2.0 ** e                     # in [1, 2)
            f = _round_half_even((mant - 1.0) * 8.0)
            if f == 8:
                e, f = e + 1, 0
            eb = e + 7
            if eb > 15 or (eb == 15 and f == 7):
                code = 0x7E if saturate else 0x7F   # +-448 or NaN
            else:
                code = (eb << 3) | f
        flat_o[idx] = code | s
    return out


E4M3_MAX = 448.0


def quant_fp8_rows(x: np.ndarray):
    """Per-row e4m3fn quantisation: (codes uint8 [rows, D], scale float32 [rows]).

    This is the step that produces the path's fp8 inputs: kv codes with their
    per-token kv_scale, and q codes (per row and head).  The PR #87 page
    names an ``act_quant`` kernel and pins the e4m3fn encoder (ties to even,
    subnormals, saturation to +-448, NaN); it does not print the scale rule,
    so this takes the plainest reading that makes the largest magnitude of a
    row land on the largest finite code:

        amax  = max_d |x[r, d]|            (a row of zeros takes amax = 448)
        inv   = float32(448 / amax)        one float32 division
        y     = float32(x[r, d] * inv)     one float32 multiply
        codes = e4m3fn(y)                  nearest, ties to even, saturating
        scale = float32(amax / 448)        so that x ~ decode(code) * scale

    The code is decided in float32 (the precision the GPU kernel computes y
    in), so both sides round the same float32 y.  Inputs must be finite.
    """
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("x must be [rows, D]")
    amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    amax = np.where(amax > 0, amax, np.float32(E4M3_MAX)).astype(np.float32)
    inv = (np.float32(E4M3_MAX) / amax).astype(np.float32)
    y = (x * inv[:, None]).astype(np.float32)
    codes = encode_e4m3fn(y.astype(np.float64))
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    return codes, scale


def _round_half_even(u: float) -> int:
    fl = math.floor(u)
    r = u - fl
    if r > 0.5:
        return fl + 1
    if r < 0.5:
        return fl
    return fl if fl % 2 == 0 else fl + 1


# ---------------------------------------------------------------------------
# Logits
# ---------------------------------------------------------------------------

def scores(q: np.ndarray, kv: np.ndarray) -> np.ndarray:
    """S[i, h, j] = sum_d q[i, h, d] * kv[j, d] on decoded values (float64, exact)."""
    Q = decode_e4m3fn(q)                      # [m, H, D]
    K = decode_e4m3fn(kv)                     # [n, D]
    m, Hh, Dd = Q.shape
    S = Q.reshape(m * Hh, Dd) @ K.T           # library dgemm; exact (see module doc)
    return S.reshape(m, Hh, K.shape[0])


def _logits_rows(Q: np.ndarray, K: np.ndarray, kv_scale: np.ndarray, w: np.ndarray,
                 ks: np.ndarray, ke: np.ndarray, width: int) -> np.ndarray:
    """Logits of a block of rows against keys K[lo:hi], written into [rows, width]."""
    r, Hh, Dd = Q.shape
    out = np.full((r, width), -np.inf, dtype=np.float64)
    lo = int(ks.min()) if r else 0
    hi = int(ke.max()) if r else 0
    if hi <= lo:
        return out
    S = (Q.reshape(r * Hh, Dd) @ K[lo:hi].T).reshape(r, Hh, hi - lo)   # dot products
    X = S * kv_scale[lo:hi].astype(np.float64)[None, None, :]          # times kv_scale[j]
    R = np.maximum(X, 0.0)                                             # ReLU
    L = np.einsum("rh,rhj->rj", w.astype(np.float64), R)               # head-weighted sum
    cols = np.arange(lo, hi)
    valid = (cols[None, :] >= ks[:, None]) & (cols[None, :] < ke[:, None])
    out[:, lo:hi] = np.where(valid, L, -np.inf)
    return out


def mqa_logits(q: np.ndarray, kv: np.ndarray, kv_scale: np.ndarray, weights: np.ndarray,
               ks: np.ndarray, ke: np.ndarray, width: Optional[int] = None,
               block_bytes: int = 1 << 28) -> np.ndarray:
    """Ragged-prefill logits, float64 [m, width] (width defaults to n).

    q uint8 [m, H, D], kv uint8 [n, D] (e4m3fn codes), kv_scale float32 [n],
    weights float32 [m, H], ks/ke int [m].  Entries outside [ks, ke) are -inf.
    Rows are processed in blocks only to bound the float64 temporaries.
    """
    q = np.asarray(q)
    m, Hh, _ = q.shape
    n = kv.shape[0]
    width = n if width is None else int(width)
    ks = np.asarray(ks, dtype=np.int64)
    ke = np.asarray(ke, dtype=np.int64)
    K = decode_e4m3fn(kv)
    out = np.empty((m, width), dtype=np.float64)
    rb = max(1, int(block_bytes // max(1, Hh * n * 8 * 4)))
    for s in range(0, m, rb):
        e = min(m, s + rb)
        out[s:e] = _logits_rows(decode_e4m3fn(q[s:e]), K, kv_scale, weights[s:e],
                                ks[s:e], ke[s:e], width)
    return out


def gather_paged_kv(kv_pool: np.ndarray, scale_pool: np.ndarray, block_table_row: np.ndarray,
                    length: int, page_size: int):
    """Contiguous (kv codes [length, D], scales [length], real [length]) of one request's keys.

    real[j] is False for keys on a page id outside [0, pages); their kv and
    scale are placeholders (page 0) that the caller must not score.
    """
    pages = (int(length) + page_size - 1) // page_size
    phys = np.asarray(block_table_row[:pages], dtype=np.int64)
    ok = (phys >= 0) & (phys < kv_pool.shape[0])
    phys = np.where(ok, phys, 0)
    kv = kv_pool[phys].reshape(pages * page_size, kv_pool.shape[-1])[:length]
    sc = scale_pool[phys].reshape(pages * page_size)[:length]
    real = np.repeat(ok, page_size)[:length]
    return kv, sc, real


def paged_mqa_logits(q: np.ndarray, kv_pool: np.ndarray, scale_pool: np.ndarray,
                     weights: np.ndarray, row_len: np.ndarray, block_table: np.ndarray,
                     page_size: int, width: Optional[int] = None,
                     rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Paged-decode logits, float64 [len(rows), width].

    q uint8 [B, next_n, H, D]; row r = b * next_n + t sees keys [0, row_len[r])
    of request b, whose key j is kv_pool[block_table[b, j // page], j % page]
    (-inf for a key whose page id lies outside the pool).  ``rows`` selects a
    subset of rows (default: all); ``width`` defaults to max(row_len).
    """
    B, nn, Hh, Dd = q.shape
    row_len = np.asarray(row_len, dtype=np.int64)
    rows = list(range(B * nn)) if rows is None else [int(r) for r in rows]
    width = int(row_len.max(initial=0)) if width is None else int(width)
    out = np.full((len(rows), width), -np.inf, dtype=np.float64)
    qf = q.reshape(B * nn, Hh, Dd)
    for o, r in enumerate(rows):
        b = r // nn
        L = int(row_len[r])
        if L <= 0:
            continue
        kv_b, sc_b, real = gather_paged_kv(kv_pool, scale_pool, block_table[b], L, page_size)
        out[o] = mqa_logits(qf[r:r + 1], kv_b, sc_b, weights[r:r + 1],
                            np.zeros(1, np.int64), np.array([L]), width=width)[0]
        out[o, :L][~real[:width]] = -np.inf
    return out


# ---------------------------------------------------------------------------
# Top-k and index maps
# ---------------------------------------------------------------------------

def topk_indices(logits: np.ndarray, ks: np.ndarray, ke: np.ndarray, k: int) -> np.ndarray:
    """Raw key indices of the k largest logits in each row's [ks, ke), int64 [rows, k].

    Order within a row: value descending, then key index ascending (so the
    lower index wins a tie at the k-th value).  Rows with fewer than k keys in
    their window are padded with -1.  -0.0 and +0.0 compare equal.
    """
    logits = np.asarray(logits)
    rows = logits.shape[0]
    out = np.full((rows, int(k)), -1, dtype=np.int64)
    for r in range(rows):
        a, b = int(ks[r]), int(ke[r])
        if b <= a:
            continue
        v = logits[r, a:b].astype(np.float64)
        idx = np.arange(a, b, dtype=np.int64)
        order = np.lexsort((idx, -v))       # primary: -v ascending; secondary: idx ascending
        take = order[: min(int(k), b - a)]
        out[r, : take.size] = idx[take]
    return out


def map_token_table(raw: np.ndarray, rows: Sequence[int], ks: np.ndarray,
                    cu_rows: Optional[np.ndarray], table: Optional[np.ndarray]) -> np.ndarray:
    """Ragged map: raw key j of row i -> table[req(i), j - ks[i]] (page size 1).

    ``rows`` are the global row ids of raw's rows; ``ks`` is indexed by global
    row id.  req(i) is the r with cu_rows[r] <= i < cu_rows[r+1] (request 0
    when cu_rows is None).  Without a table the raw index is returned.
    -1 stays -1.
    """
    raw = np.asarray(raw, dtype=np.int64)
    if table is None:
        return raw.copy()
    out = np.full(raw.shape, -1, dtype=np.int64)
    for o, i in enumerate(rows):
        req = 0 if cu_rows is None else int(np.searchsorted(cu_rows, i, side="right") - 1)
        sel = raw[o] >= 0
        out[o, sel] = table[req, raw[o, sel] - int(ks[i])]
    return out


def map_block_table(raw: np.ndarray, rows: Sequence[int], next_n: int,
                    block_table: np.ndarray, page_size: int, num_pages: Optional[int] = None) -> np.ndarray:
    """Paged map: raw key j of row r -> block_table[r // next_n, j // page] * page + j % page.

    A page id outside [0, num_pages) (any negative id when num_pages is None)
    maps to -1, as does -1 padding.
    """
    raw = np.asarray(raw, dtype=np.int64)
    out = np.full(raw.shape, -1, dtype=np.int64)
    for o, r in enumerate(rows):
        b = int(r) // int(next_n)
        sel = raw[o] >= 0
        j = raw[o, sel]
        page = block_table[b, j // page_size].astype(np.int64)
        real = (page >= 0) & (page < (num_pages if num_pages is not None else np.iinfo(np.int64).max))
        out[o, sel] = np.where(real, page * page_size + j % page_size, -1)
    return out


def ragged_topk_mapped(inp, rows: Optional[Sequence[int]] = None):
    """(logits f64 [len(rows), n], raw top-k, mapped top-k) of a RaggedInputs-like object."""
    rows = list(range(inp.m)) if rows is None else [int(r) for r in rows]
    ridx = np.asarray(rows, dtype=np.int64)
    L = mqa_logits(inp.q[ridx], inp.kv, inp.kv_scale, inp.weights[ridx],
                   inp.ks[ridx], inp.ke[ridx])
    raw = topk_indices(L, inp.ks[ridx], inp.ke[ridx], inp.k)
    mapped = map_token_table(raw, rows, inp.ks, inp.cu_rows, inp.table)
    return L, raw, mapped


def paged_topk_mapped(inp, rows: Optional[Sequence[int]] = None, width: Optional[int] = None):
    """(logits f64, raw top-k, physical-slot top-k) of a PagedInputs-like object."""
    rows = list(range(inp.rows)) if rows is None else [int(r) for r in rows]
    L = paged_mqa_logits(inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len,
                         inp.block_table, inp.page_size, width=width, rows=rows)
    ridx = np.asarray(rows, dtype=np.int64)
    raw = topk_indices(L, np.zeros(len(rows), np.int64), inp.row_len[ridx], inp.k)
    mapped = map_block_table(raw, rows, inp.next_n, inp.block_table, inp.page_size, inp.kv_pool.shape[0])
    return L, raw, mapped


# ---------------------------------------------------------------------------
# Index preparation (the gen_nsa_ks_ke step on the lightllm PR pages)
# ---------------------------------------------------------------------------

def prepare_ragged(seq_len, q_len, req_idx, table):
    """Ragged prefill indices for a batch of requests, written out one element at a time.

    Request b holds seq_len[b] tokens whose last q_len[b] are this step's queries
    (q_len is clamped to [0, seq_len]).  The keys of all requests are laid out
    back to back (the ragged key space), request b's first at cu_seq[b]; its
    token p is kv slot table[req_idx[b], p] (the req -> token table).

    Returns a dict of int64 arrays:
      cu_seq [B+1], cu_q [B+1]   prefix sums of the lengths
      ks, ke [total_q]           query t of request b (global index cu_q[b] + t) sees
                                 ragged keys [cu_seq[b], cu_seq[b] + seq_len[b] - q_len[b] + t + 1)
      ragged_mem [total_seq]     ragged key cu_seq[b] + p -> table[req_idx[b], p]
                                 (-1 when p lies past the table row or req_idx is out of range)
    """
    seq_len = [max(0, int(v)) for v in seq_len]
    q_len = [min(max(0, int(v)), s) for v, s in zip(q_len, seq_len)]
    table = np.asarray(table)
    B = len(seq_len)
    cu_seq = [0]
    cu_q = [0]
    for b in range(B):
        cu_seq.append(cu_seq[-1] + seq_len[b])
        cu_q.append(cu_q[-1] + q_len[b])
    ks, ke, mem = [], [], []
    for b in range(B):
        for t in range(q_len[b]):
            ks.append(cu_seq[b])
            ke.append(cu_seq[b] + seq_len[b] - q_len[b] + t + 1)
        r = int(req_idx[b])
        for p in range(seq_len[b]):
            ok = 0 <= r < table.shape[0] and p < table.shape[1]
            mem.append(int(table[r, p]) if ok else -1)
    as64 = lambda v: np.asarray(v, dtype=np.int64)
    return {"cu_seq": as64(cu_seq), "cu_q": as64(cu_q), "ks": as64(ks), "ke": as64(ke), "ragged_mem": as64(mem)}


def prepare_decode(seq_len, next_n, req_idx, req_to_page):
    """Paged decode / MTP indices: request b's next_n query rows are its last next_n tokens.

      row_len [B * next_n]          row t of request b sees keys [0, seq_len[b] - next_n + t + 1)
                                    (at least 0)
      block_table [B, max_pages]    row b is req_to_page[req_idx[b]] (-1 past the table or for
                                    an out-of-range req_idx)
    """
    next_n = int(next_n)
    req_to_page = np.asarray(req_to_page)
    B = len(seq_len)
    max_pages = req_to_page.shape[1]
    row_len = []
    bt = np.full((B, max_pages), -1, dtype=np.int64)
    for b in range(B):
        for t in range(next_n):
            row_len.append(max(0, int(seq_len[b]) - next_n + t + 1))
        r = int(req_idx[b])
        if 0 <= r < req_to_page.shape[0]:
            for p in range(max_pages):
                bt[b, p] = int(req_to_page[r, p])
    return {"row_len": np.asarray(row_len, dtype=np.int64), "block_table": bt}


def rows_per_chunk(cap_bytes: int, row_stride_elems: int, rows: int) -> int:
    """Rows per chunk of the row-chunked loop: floor(cap / (stride * 4)), at least 1.

    The chunking page sizes chunks as ``max(1, int(gb * 1e9) // (n * 4))``
    rows (decimal gigabytes, 4-byte logits) and a cap of 0 means one shot.
    """
    if cap_bytes <= 0:
        return max(1, rows)
    return max(1, min(rows, int(cap_bytes) // (int(row_stride_elems) * 4)))

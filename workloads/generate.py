"""Seeded input recipes for the indexer workloads.

Recipe (the ``_build`` helper and ``SCENARIOS`` table of the
bench_mqa_logits_chunking.py page, plus the paged-decode form named on the
vessl-ai/sglang PR #87 page):

* q  = randn(m, H, D).clamp(-2, 2) cast to fp8 e4m3fn
* kv = randn(n, D).clamp(-2, 2) cast to fp8 e4m3fn
* kv_scale = rand(n) + 0.5            (U[0.5, 1.5))
* weights  = rand(m, H)               (U[0, 1))
* ks = 0, ke[i] = rank_start + i + 1  (the query rows are the last m
  positions of the sequence, so the mask is causal)

All draws come from one torch CPU generator seeded with ``seed``, in the
order q, kv, kv_scale, weights; recipes that need more (context lengths,
page permutation, token tables) draw those first / last as documented at
each function.  The fp8 bytes are produced by torch's own float32 ->
float8_e4m3fn cast and returned as raw uint8 codes, so the device and the
CPU oracle always see identical bytes.
"""

from __future__ import annotations

import dataclasses
from typing import Callable, Dict, Optional, Sequence, Tuple

import numpy as np
import torch

H = 32  # indexer heads (index_n_heads on the chunking micro-benchmark page)
D = 128  # indexer head dim (index_head_dim on the same page)


def _fp8_codes(t: torch.Tensor) -> np.ndarray:
    """Cast a float32 tensor to fp8 e4m3fn with torch and return raw bytes."""
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _randn_fp8(g: torch.Generator, shape: Sequence[int], clamp: float = 2.0,
               chunk_rows: int = 0) -> np.ndarray:
    """randn(shape).clamp(-clamp, clamp) cast to e4m3fn.

    For very large tensors the draw is made in slices of ``chunk_rows`` along
    the first dimension (the slicing is part of the recipe, so it is
    deterministic for a given seed).
    """
    shape = tuple(int(s) for s in shape)
    if chunk_rows <= 0 or shape[0] <= chunk_rows:
        return _fp8_codes(torch.randn(shape, generator=g).clamp_(-clamp, clamp))
    out = np.empty(shape, dtype=np.uint8)
    for s in range(0, shape[0], chunk_rows):
        e = min(shape[0], s + chunk_rows)
        out[s:e] = _fp8_codes(torch.randn((e - s,) + shape[1:], generator=g).clamp_(-clamp, clamp))
    return out


@dataclasses.dataclass
class RaggedInputs:
    """Ragged-prefill inputs: one flat kv, per-row key windows [ks, ke)."""

    name: str
    q: np.ndarray          # uint8 [m, H, D]  e4m3fn codes
    kv: np.ndarray         # uint8 [n, D]     e4m3fn codes
    kv_scale: np.ndarray   # float32 [n]
    weights: np.ndarray    # float32 [m, H]
    ks: np.ndarray         # int32 [m]
    ke: np.ndarray         # int32 [m]
    k: int                 # top-k width
    cu_rows: Optional[np.ndarray] = None  # int32 [num_req + 1] row offsets
    table: Optional[np.ndarray] = None    # int32 [num_req, ld] token -> slot table
    cap_bytes: int = 0     # logits workspace cap for the row-chunked entry (0 = one shot)

    @property
    def m(self) -> int:
        return int(self.q.shape[0])

    @property
    def n(self) -> int:
        return int(self.kv.shape[0])

    @property
    def valid_pairs(self) -> int:
        return int(np.maximum(self.ke.astype(np.int64) - self.ks, 0).sum())


@dataclasses.dataclass
class PagedInputs:
    """Paged-decode inputs: kv lives in fixed-size pages reached through a block table."""

    name: str
    q: np.ndarray           # uint8 [B, next_n, H, D]
    kv_pool: np.ndarray     # uint8 [P, page_size, D]
    scale_pool: np.ndarray  # float32 [P, page_size]
    weights: np.ndarray     # float32 [B * next_n, H]
    ctx: np.ndarray         # int32 [B] context length of each request
    row_len: np.ndarray     # int32 [B * next_n]; row r of request b sees keys [0, row_len)
    block_table: np.ndarray # int32 [B, max_pages]; -1 past the request's pages
    page_size: int
    k: int

    @property
    def B(self) -> int:
        return int(self.q.shape[0])

    @property
    def next_n(self) -> int:
        return int(self.q.shape[1])

    @property
    def rows(self) -> int:
        return self.B * self.next_n

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def valid_pairs(self) -> int:
        return int(self.row_len.astype(np.int64).sum())

    @property
    def kv_bytes(self) -> int:
        """Bytes of kv codes plus scales the requests actually reference."""
        return int(self.ctx.astype(np.int64).sum()) * (self.q.shape[-1] + 4)


def ragged_inputs(m: int, n: int, k: int, seed: int, *, name: str = "ragged",
                  ks: Optional[np.ndarray] = None, ke: Optional[np.ndarray] = None,
                  weight_mode: str = "uniform", scale_mode: str = "uniform",
                  clamp: float = 2.0, cap_bytes: int = 0) -> RaggedInputs:
    """Single-request ragged prefill.

    Default mask: ks = 0, ke[i] = n - m + i + 1 clamped to n (the m query rows
    are the last m positions; the chunking page's ``_build`` with the rank's
    last slice).  ``weight_mode``: "uniform" (U[0,1)), "signed" (U[-1,1)),
    "zero".  ``scale_mode``: "uniform" (U[0.5,1.5)), "zero", "one".
    """
    g = torch.Generator().manual_seed(int(seed))
    q = _randn_fp8(g, (m, H, D), clamp, chunk_rows=4096)
    kv = _randn_fp8(g, (n, D), clamp, chunk_rows=1 << 16)
    kv_scale = (torch.rand(n, generator=g) + 0.5).numpy().astype(np.float32)
    weights = torch.rand(m, H, generator=g).numpy().astype(np.float32)
    if scale_mode == "zero":
        kv_scale[:] = 0.0
    elif scale_mode == "one":
        kv_scale[:] = 1.0
    if weight_mode == "signed":
        weights = (weights * 2.0 - 1.0).astype(np.float32)
    elif weight_mode == "zero":
        weights[:] = 0.0
    if ke is None:
        ke = np.minimum(np.arange(m, dtype=np.int64) + (n - m) + 1, n)
        ke = np.maximum(ke, 0)
    if ks is None:
        ks = np.zeros(m, dtype=np.int64)
    return RaggedInputs(name=name, q=q, kv=kv, kv_scale=kv_scale, weights=weights,
                        ks=np.asarray(ks, dtype=np.int32), ke=np.asarray(ke, dtype=np.int32),
                        k=int(k), cap_bytes=int(cap_bytes))


def multi_request_ragged(requests: Sequence[Tuple[int, int]], k: int, seed: int, *,
                         name: str = "multi_request", table_slack: int = 3) -> RaggedInputs:
    """Several requests packed into one flat kv.

    ``requests`` is a list of (kv_len, q_rows).  Request r owns keys
    [off_r, off_r + kv_len) of the flat kv; its q_rows rows are its last
    positions (causal): ks = off_r, ke = off_r + kv_len - q_rows + t + 1.
    After q, kv, kv_scale and weights, a random permutation of
    ``table_slack * total_kv`` slots is drawn and request r's token table row
    holds the next kv_len slots of it (so the token -> slot map is a
    non-trivial injection).  Unused table entries are -1.
    """
    g = torch.Generator().manual_seed(int(seed))
    lens = [int(a) for a, _ in requests]
    rows = [int(b) for _, b in requests]
    n, m = sum(lens), sum(rows)
    q = _randn_fp8(g, (m, H, D))
    kv = _randn_fp8(g, (n, D))
    kv_scale = (torch.rand(n, generator=g) + 0.5).numpy().astype(np.float32)
    weights = torch.rand(m, H, generator=g).numpy().astype(np.float32)
    perm = torch.randperm(max(1, table_slack * n), generator=g).numpy().astype(np.int64)
    ld = max(1, max(lens))
    table = np.full((len(requests), ld), -1, dtype=np.int32)
    ks = np.empty(m, dtype=np.int32)
    ke = np.empty(m, dtype=np.int32)
    cu = np.zeros(len(requests) + 1, dtype=np.int32)
    off_k, off_r = 0, 0
    for r, (L, R) in enumerate(zip(lens, rows)):
        table[r, :L] = perm[off_k:off_k + L]
        t = np.arange(R)
        ks[off_r:off_r + R] = off_k
        ke[off_r:off_r + R] = off_k + np.clip(L - R + t + 1, 0, L)
        off_k += L
        off_r += R
        cu[r + 1] = off_r
    return RaggedInputs(name=name, q=q, kv=kv, kv_scale=kv_scale, weights=weights,
                        ks=ks, ke=ke, k=int(k), cu_rows=cu, table=table)


def paged_inputs(B: int, next_n: int, ctx_lo: int, ctx_hi: int, k: int, seed: int, *,
                 page_size: int = 64, name: str = "paged",
                 ctx: Optional[np.ndarray] = None) -> PagedInputs:
    """Paged decode / multi-token prediction.

    Draw order: context lengths ctx_b ~ U{ctx_lo..ctx_hi} (unless given),
    q [B, next_n, H, D], the kv pool [P, page, D] (P = sum ceil(ctx_b/page)),
    the per-token scale pool [P, page], weights [B*next_n, H], and last a
    random permutation of the P physical pages.  Request b's logical page p
    lives in physical page perm[off_b + p]; table entries past the request's
    pages are -1.  Row r of request b is causal: it sees keys
    [0, ctx_b - next_n + r + 1).
    """
    g = torch.Generator().manual_seed(int(seed))
    if ctx is None:
        ctx = torch.randint(ctx_lo, ctx_hi + 1, (B,), generator=g).numpy()
    ctx = np.asarray(ctx, dtype=np.int64)
    pages = (ctx + page_size - 1) // page_size
    P = int(pages.sum())
    max_pages = max(1, int((max(int(ctx_hi), int(ctx.max(initial=0))) + page_size - 1) // page_size))
    q = _randn_fp8(g, (B, next_n, H, D))
    kv_pool = _randn_fp8(g, (P, page_size, D), chunk_rows=4096)
    scale_pool = (torch.rand(P, page_size, generator=g) + 0.5).numpy().astype(np.float32)
    weights = torch.rand(B * next_n, H, generator=g).numpy().astype(np.float32)
    perm = torch.randperm(P, generator=g).numpy().astype(np.int32)
    block_table = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        block_table[b, :pages[b]] = perm[off:off + pages[b]]
        off += int(pages[b])
    row_len = np.empty(B * next_n, dtype=np.int32)
    for b in range(B):
        for r in range(next_n):
            row_len[b * next_n + r] = max(0, int(ctx[b]) - next_n + r + 1)
    return PagedInputs(name=name, q=q, kv_pool=kv_pool, scale_pool=scale_pool,
                       weights=weights, ctx=ctx.astype(np.int32), row_len=row_len,
                       block_table=block_table, page_size=int(page_size), k=int(k))


# The five synthetic workloads.  Seeds are the workload's ordinal.
def quant_inputs(rows: int, D: int, seed: int, *, spread: float = 3.0) -> np.ndarray:
    """float32 [rows, D] activations for the fp8 quantiser: randn per element times a
    per-row magnitude 10**U[-spread, spread), so row scales span many octaves."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn(rows, D, generator=g, dtype=torch.float32)
    mag = torch.pow(10.0, (torch.rand(rows, 1, generator=g) * 2.0 - 1.0) * spread)
    return (x * mag).to(torch.float32).numpy()


def _tiny() -> RaggedInputs:
    return ragged_inputs(64, 4096, 512, seed=1, name="tiny_ragged_m64_n4096")


def _cold64k() -> RaggedInputs:
    # cold_chunk1_64K: prefix 0, extend 65536 -> m = 8192, n = 65536, ke = 57344 + i + 1
    return ragged_inputs(8192, 65536, 2048, seed=2, name="prefill_m8192_n65536")


def _square35k() -> RaggedInputs:
    return ragged_inputs(8192, 35000, 2048, seed=3, name="prefill_m8192_n35000")


def _paged() -> PagedInputs:
    return paged_inputs(64, 4, 8192, 131072, 2048, seed=4, page_size=64,
                        name="paged_decode_b64x4_ctx8k-128k")


def _paged_sequential() -> PagedInputs:
    """The decode workload with each request's pages physically consecutive (block table rows in
    ascending page order instead of the random permutation): same lengths and work, used to measure
    what the random page order costs the paged logits kernel."""
    inp = paged_inputs(64, 4, 8192, 131072, 2048, seed=4, page_size=64,
                       name="paged_decode_b64x4_ctx8k-128k_sequential_pages")
    pages = (inp.ctx.astype(np.int64) + 63) // 64
    bt = np.full_like(inp.block_table, -1)
    off = 0
    for b in range(inp.B):
        bt[b, :pages[b]] = np.arange(off, off + pages[b], dtype=np.int32)
        off += int(pages[b])
    inp.block_table = bt
    return inp


def _long210k() -> RaggedInputs:
    # warm_long_150K+60K: prefix 150000, extend 60000 -> m = 7500, n = 210000
    return ragged_inputs(7500, 210000, 2048, seed=5, name="prefill_m7500_n210000_cap2GB",
                         cap_bytes=2_000_000_000)


def _tail80k() -> RaggedInputs:
    # 80K_tail_chunk_14K of the chunking page: prefix 65536, extend 14464 -> m = 1808, n = 80000
    return ragged_inputs(1808, 80000, 2048, seed=6, name="prefill_m1808_n80000")


def _warm154k() -> RaggedInputs:
    # warm_cont_150K+4K of the chunking page: prefix 150000, extend 4096 -> m = 512, n = 154096
    return ragged_inputs(512, 154096, 2048, seed=7, name="prefill_m512_n154096")


CONFIGS: Dict[str, Callable[[], object]] = {
    "tiny": _tiny,
    "prefill_64k": _cold64k,
    "prefill_35k": _square35k,
    "paged_decode": _paged,
    "paged_decode_sequential": _paged_sequential,
    "long_prefix_210k": _long210k,
    "tail_80k": _tail80k,
    "warm_154k": _warm154k,
}


def config_inputs(name: str):
    return CONFIGS[name]()


# ---------------------------------------------------------------------------
# Sparse MLA attention over the top-k slots (the step after the indexer)
# ---------------------------------------------------------------------------

MLA_DQK = 576   # KV row: 512 latent values + 64 rotary values
MLA_DV = 512


@dataclasses.dataclass
class SparseMlaInputs:
    """Sparse MLA inputs: bf16 queries, an fp8 KV pool with per-slot scales, top-k slot lists."""

    name: str
    q_bits: np.ndarray      # uint16 [T, H, 576], bf16 bit patterns
    kv_codes: np.ndarray    # uint8 [S, 576], e4m3fn codes
    kv_scale: np.ndarray    # float32 [S]
    indices: np.ndarray     # int32 [T, topk]; -1 = no slot
    sm_scale: float

    @property
    def T(self) -> int:
        return int(self.q_bits.shape[0])

    @property
    def H(self) -> int:
        return int(self.q_bits.shape[1])

    @property
    def topk(self) -> int:
        return int(self.indices.shape[1])


def sparse_mla_inputs(T: int, H: int, S: int, topk: int, seed: int, *, invalid_tail: int = 0,
                      duplicates: int = 0, q_clamp: float = 2.0, kv_clamp: float = 2.0,
                      sm_scale: Optional[float] = None, name: str = "sparse_mla") -> SparseMlaInputs:
    """Draw order: q randn [T, H, 576] clamped to [-q_clamp, q_clamp] and rounded to bf16, the KV
    codes randn [S, 576] clamped and cast to e4m3fn, kv_scale ~ U[0.5, 1.5), then per token a
    random choice of `topk` distinct slots (without replacement while S allows).  The last
    `invalid_tail` entries of each list become -1 (the top-k stage's padding) and `duplicates`
    entries repeat an earlier slot of the same list.  sm_scale defaults to 1 / sqrt(576)."""
    g = torch.Generator().manual_seed(int(seed))
    q = torch.randn((T, H, MLA_DQK), generator=g).clamp_(-q_clamp, q_clamp).to(torch.bfloat16)
    q_bits = q.view(torch.int16).numpy().astype(np.uint16)
    kv = _randn_fp8(g, (S, MLA_DQK), clamp=kv_clamp, chunk_rows=65536)
    kv_scale = (torch.rand(S, generator=g) + 0.5).numpy().astype(np.float32)
    idx = np.empty((T, topk), dtype=np.int32)
    for t in range(T):
        if topk <= S:
            idx[t] = torch.randperm(S, generator=g)[:topk].numpy()
        else:
            idx[t] = torch.randint(0, S, (topk,), generator=g).numpy()
    if duplicates > 0:
        for t in range(T):
            pos = torch.randint(1, topk, (duplicates,), generator=g).numpy()
            src = torch.randint(0, topk, (duplicates,), generator=g).numpy()
            idx[t, pos] = idx[t, np.minimum(src, pos - 1)]
    if invalid_tail > 0:
        idx[:, topk - invalid_tail:] = -1
    scale = float(1.0 / np.sqrt(MLA_DQK)) if sm_scale is None else float(sm_scale)
    return SparseMlaInputs(name=name, q_bits=q_bits, kv_codes=kv, kv_scale=kv_scale, indices=idx,
                           sm_scale=scale)

"""Float64 reference for the sparse MLA attention that consumes the indexer's top-k slots.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH: imported only by the
tests, by ``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of
``bench.py``.  Nothing here is shared with the HIP library.

What is computed.  The vessl-ai/sglang PR #87 page names the step after the
indexer: sparse MLA attention kernels (a prefill kernel, and a decode kernel
run as a split-K "partial" kernel whose per-split results a "combine" kernel
merges) that read an MLA KV pool kept in fp8 e4m3 and widen it to bf16 inside
the kernel.  The page does not write the attention out.  The plain reading,
evaluated here literally, is softmax attention of every query token over the
KV rows that its top-k list selects:

    s[t, h, i] = sm_scale * dot(q[t, h, :], kv_scale[j] * e4m3(kv[j, :]))      for slot j = idx[t, i]
    lse[t, h]  = log(sum_i exp(s[t, h, i]))
    o[t, h, :] = sum_i exp(s[t, h, i] - lse[t, h]) * kv_scale[j] * e4m3(kv[j, :dv])

Readings where the page is silent (each is also listed in the design notes):
* a slot j is valid when 0 <= j < num_slots; other entries (the -1 padding of
  the top-k output) are skipped, and a slot listed twice counts twice;
* every KV row holds the compressed latent followed by its rotary part: the
  score uses the whole row (576 values) and the value is its first dv = 512
  values (the DeepSeek-style MLA latent layout);
* the KV pool stores e4m3fn codes with one float32 scale per slot, the same
  per-token scaling as the indexer's key pool;
* q arrives in bf16 (raw uint16 bit patterns here, widened exactly);
* a token with no valid slot gets o = 0 and lse = -inf.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .indexer_oracle import decode_e4m3fn

MLA_DQK = 576   # score dimension: 512 latent + 64 rotary
MLA_DV = 512    # value dimension: the latent part


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of a float32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def sparse_mla(q_bits: np.ndarray, kv_codes: np.ndarray, kv_scale: np.ndarray, indices: np.ndarray,
               sm_scale: float, dv: int = MLA_DV, tokens: Optional[Sequence[int]] = None):
    """(o float64 [T', H, dv], lse float64 [T', H]) for the listed tokens (all by default).

    q_bits [T, H, D] uint16 (bf16), kv_codes [S, D] uint8 (e4m3fn), kv_scale [S] float32,
    indices [T, topk] int32 slot ids.
    """
    q_bits = np.asarray(q_bits, dtype=np.uint16)
    T, H, D = q_bits.shape
    S = int(kv_codes.shape[0])
    tokens = list(range(T)) if tokens is None else [int(t) for t in tokens]
    o = np.zeros((len(tokens), H, dv), dtype=np.float64)
    lse = np.full((len(tokens), H), -np.inf, dtype=np.float64)
    for n, t in enumerate(tokens):
        idx = np.asarray(indices[t], dtype=np.int64)
        sel = idx[(idx >= 0) & (idx < S)]
        if sel.size == 0:
            continue
        # dequantised rows of the selected slots (duplicates kept)
        K = decode_e4m3fn(kv_codes[sel]) * np.asarray(kv_scale, dtype=np.float64)[sel][:, None]
        Q = decode_bf16(q_bits[t])                       # [H, D]
        s = sm_scale * (Q @ K.T)                          # [H, n]
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        o[n] = (e / z) @ K[:, :dv]
        lse[n] = (m + np.log(z))[:, 0]
    return o, lse


"""Comparison helpers between the HIP path and the float64 oracle.

Tolerances
----------
Logits: |gpu - oracle| <= 1e-3 + 2e-3 * |oracle| inside each row's window,
and exactly -inf outside it when the call asked for clean logits.

When weights of both signs make the head sum cancel, that relative band no
longer bounds the device's own rounding: the fp8 MFMA accumulates each
128-term dot product with an error up to about 2**-11 of its largest term
(measured on the device).  For those cases the band is widened by
2**-10 * scale_j * max_d |k_jd| * sum_h |w_h| * max_d |q_hd|: twice the
measured accumulation error, passed through the ReLU (1-Lipschitz) and the
head weights and scale.

Top-k against the oracle: with v_k the oracle's k-th largest value in the
window and T = 1e-3 + 2e-3 * |v_k|, the device must return exactly
min(k, window) distinct in-window indices (then -1s), include every index
whose oracle value exceeds v_k + T, and include none whose oracle value is
below v_k - T.

Top-k exactness: on the device's own float32 logits, the device selection
must equal the oracle's selection (value desc, lower index wins ties) as a
set, with no tolerance.
"""

from __future__ import annotations

import numpy as np
import torch

ATOL = 1e-3
RTOL = 2e-3


def to_dev(a, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def assert_logits_close(gpu: np.ndarray, ora: np.ndarray, ks, ke, clean: bool, extra_tol=None, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    rows, width = ora.shape
    cols = np.arange(width)
    inside = (cols[None, :] >= np.asarray(ks)[:, None]) & (cols[None, :] < np.asarray(ke)[:, None])
    assert np.all(np.isfinite(ora[inside])), "oracle produced non-finite in-window values"
    tol = ATOL + RTOL * np.abs(ora)
    if extra_tol is not None:
        tol = tol + extra_tol
    with np.errstate(invalid="ignore"):
        diff = np.abs(gpu - ora)
    bad = inside & ~(diff <= tol)
    if bad.any():
        r, c = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} logits out of tolerance; first at row {r} col {c}: "
                             f"gpu {gpu[r, c]!r} oracle {ora[r, c]!r} tol {tol[r, c]!r}")
    if clean:
        outside = ~inside
        ok = np.all(gpu[outside] == -np.inf)
        assert ok, f"{what}: clean logits not -inf outside the window"


def cancellation_tol(q_codes, kv_codes, kv_scale, weights, rows, lo, hi):
    """Extra tolerance for signed weights: 2**-10 * scale_j * max|k_j| * sum_h |w_h| * max|q_h|."""
    from tests.oracle_pins import torch_decode
    Q = np.abs(torch_decode(q_codes[rows]))                     # [r, H, D]
    K = np.abs(torch_decode(kv_codes[lo:hi]))                   # [n, D]
    qmax = Q.max(axis=2)                                       # [r, H]
    kmax = K.max(axis=1)                                       # [n]
    wsum = (np.abs(weights[rows]).astype(np.float64) * qmax).sum(axis=1)   # [r]
    return 2.0 ** -10 * wsum[:, None] * (kmax * kv_scale[lo:hi].astype(np.float64))[None, :]


def assert_topk_tolerant(gpu_idx: np.ndarray, ora_logits: np.ndarray, ks, ke, k: int, what=""):
    gpu_idx = np.asarray(gpu_idx, dtype=np.int64)
    for r in range(gpu_idx.shape[0]):
        a, b = int(ks[r]), int(ke[r])
        cnt = max(0, min(k, b - a))
        row = gpu_idx[r]
        sel = row[:cnt]
        assert np.all(row[cnt:] == -1), f"{what} row {r}: padding is not -1"
        assert np.unique(sel).size == cnt, f"{what} row {r}: duplicate or missing indices"
        assert np.all((sel >= a) & (sel < b)), f"{what} row {r}: index outside [ks, ke)"
        if cnt == 0 or cnt == b - a:
            continue
        v = ora_logits[r, a:b]
        vk = np.sort(v)[::-1][cnt - 1]
        if vk == -np.inf:
            # fewer than k keys with a value (keys on pages outside the pool are -inf): every one
            # that has a value is selected, the rest of the selection is -inf keys
            assert np.isin(np.nonzero(np.isfinite(v))[0] + a, sel).all(), f"{what} row {r}: a finite key is missing"
            continue
        T = ATOL + RTOL * abs(vk)
        must = np.nonzero(v > vk + T)[0] + a
        assert np.isin(must, sel).all(), f"{what} row {r}: a clearly-top index is missing"
        assert np.all(ora_logits[r, sel] >= vk - T), f"{what} row {r}: a clearly-low index was selected"


def assert_topk_exact(gpu_idx: np.ndarray, exact_idx: np.ndarray, what=""):
    gpu_idx = np.asarray(gpu_idx, dtype=np.int64)
    exact_idx = np.asarray(exact_idx, dtype=np.int64)
    for r in range(gpu_idx.shape[0]):
        g = gpu_idx[r]
        e = exact_idx[r]
        ng = int((g >= 0).sum())
        ne = int((e >= 0).sum())
        assert ng == ne, f"{what} row {r}: {ng} selected, expected {ne}"
        assert np.all(g[ng:] == -1), f"{what} row {r}: padding"
        if set(g[:ng].tolist()) != set(e[:ne].tolist()):
            missing = sorted(set(e[:ne].tolist()) - set(g[:ng].tolist()))[:5]
            extra = sorted(set(g[:ng].tolist()) - set(e[:ne].tolist()))[:5]
            raise AssertionError(f"{what} row {r}: sets differ; missing {missing} extra {extra}")

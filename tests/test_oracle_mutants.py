"""Plant plausible mistakes in copies of the oracle (on the CPU) and show that the pins catch each.

Every mutant below differs from the oracle's logits routine in one place; the
test asserts that at least one pin in tests/oracle_pins.py fails for it.
"""

import numpy as np
import pytest

import oracle.indexer_oracle as O
from tests.oracle_pins import ALL_LOGIT_CHECKS


def _make(variant):
    def logits(q, kv, kv_scale, weights, ks, ke):
        q = np.asarray(q)
        m, Hh, Dd = q.shape
        n = kv.shape[0]
        table = O.e4m3fn_value_table()
        if variant == "decode_bias8":
            table = table.copy()
            nz = np.isfinite(table) & (np.arange(256) & 0x78 != 0)
            table[nz] = table[nz] / 2
        Q = table[q]
        K = table[kv]
        if variant == "transposed_kv":
            K = K[:, ::-1]
        S = Q.reshape(m * Hh, Dd) @ K.T
        S = S.reshape(m, Hh, n)
        sc = kv_scale.astype(np.float64)
        w = np.asarray(weights, dtype=np.float64)
        if variant == "no_scale":
            X = S
        else:
            X = S * sc[None, None, :]
        if variant == "relu_after_weight":
            L = np.maximum(np.einsum("ih,ihj->ihj", w, X), 0).sum(axis=1)
        elif variant == "no_relu":
            L = np.einsum("ih,ihj->ij", w, X)
        elif variant == "abs_not_relu":
            L = np.einsum("ih,ihj->ij", w, np.abs(X))
        elif variant == "drop_last_head":
            L = np.einsum("ih,ihj->ij", w[:, :-1], np.maximum(X, 0)[:, :-1])
        elif variant == "mean_heads":
            L = np.einsum("ih,ihj->ij", w, np.maximum(X, 0)) / Hh
        elif variant == "weights_reversed":
            L = np.einsum("ih,ihj->ij", w[:, ::-1], np.maximum(X, 0))
        else:
            L = np.einsum("ih,ihj->ij", w, np.maximum(X, 0))
        cols = np.arange(n)
        ks_ = np.asarray(ks)[:, None]
        ke_ = np.asarray(ke)[:, None]
        if variant == "inclusive_end":
            valid = (cols[None, :] >= ks_) & (cols[None, :] <= ke_)
        elif variant == "ks_off_by_one":
            valid = (cols[None, :] > ks_) & (cols[None, :] < ke_)
        else:
            valid = (cols[None, :] >= ks_) & (cols[None, :] < ke_)
        return np.where(valid, L, -np.inf)
    return logits


MUTANTS = ["decode_bias8", "transposed_kv", "no_scale", "relu_after_weight", "no_relu",
           "abs_not_relu", "drop_last_head", "mean_heads", "weights_reversed",
           "inclusive_end", "ks_off_by_one"]


def test_unmutated_copy_passes_all_pins():
    fn = _make("none")
    for check in ALL_LOGIT_CHECKS:
        ok, msg = check(fn)
        assert ok, (check.__name__, msg)


@pytest.mark.parametrize("variant", MUTANTS)
def test_mutant_is_caught(variant):
    fn = _make(variant)
    failed = []
    for check in ALL_LOGIT_CHECKS:
        try:
            ok, _ = check(fn)
        except Exception:
            ok = False
        if not ok:
            failed.append(check.__name__)
    assert failed, f"mutant {variant} passed every pin"

"""Pin checks for the float64 oracle, written as functions of the logits routine.

Each check compares a logits implementation with something other than
itself: exact rational arithmetic, a closed form, a library routine fed by
torch's own fp8 decode, or an invariant of the definition.  The same checks
run against deliberately broken copies of the oracle (tests/test_oracle_mutants.py)
to show that a plausible mistake fails at least one of them.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch

from workloads.generate import H, D, ragged_inputs


def torch_decode(codes: np.ndarray) -> np.ndarray:
    """Decode e4m3fn bytes with torch's own upcast (independent of the oracle's table)."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _tiny(seed=11, m=3, n=9, heads=H, weight_mode="uniform", scale_mode="uniform"):
    inp = ragged_inputs(m, n, 4, seed=seed, weight_mode=weight_mode, scale_mode=scale_mode)
    if heads != H:
        inp.q = np.ascontiguousarray(inp.q[:, :heads])
        inp.weights = np.ascontiguousarray(inp.weights[:, :heads])
    inp.ks = np.zeros(m, np.int32)
    inp.ke = np.full(m, n, np.int32)
    return inp


def exact_logits_fraction(inp) -> list:
    """Exact rational logits: every fp8 value, float32 scale and weight is a dyadic rational."""
    Q = torch_decode(inp.q)
    K = torch_decode(inp.kv)
    out = []
    for i in range(inp.q.shape[0]):
        row = []
        for j in range(inp.kv.shape[0]):
            acc = Fraction(0)
            for h in range(inp.q.shape[1]):
                s = sum((Fraction(float(Q[i, h, d])) * Fraction(float(K[j, d])) for d in range(D)),
                        Fraction(0))
                x = s * Fraction(float(inp.kv_scale[j]))
                r = x if x > 0 else Fraction(0)
                acc += Fraction(float(inp.weights[i, h])) * r
            row.append(acc)
        out.append(row)
    return out


def check_exact_small(logits_fn, seed=11, weight_mode="signed"):
    """Oracle logits agree with exact rational arithmetic to float64 rounding."""
    inp = _tiny(seed=seed, m=2, n=5, heads=6, weight_mode=weight_mode)
    L = logits_fn(inp.q, inp.kv, inp.kv_scale, inp.weights, inp.ks, inp.ke)
    ex = exact_logits_fraction(inp)
    for i in range(2):
        for j in range(5):
            e = float(ex[i][j])
            bound = 1e-12 * (abs(e) + float(np.abs(inp.weights[i]).sum()) * 1000.0)
            if not abs(float(L[i, j]) - e) <= bound:
                return False, f"row {i} key {j}: oracle {L[i, j]!r} exact {e!r}"
    return True, ""


def check_relu_matmul_special_case(logits_fn, seed=12):
    """H=1, weight 1, scale 1: logits = max(Q K^T, 0), Q and K decoded by torch."""
    inp = _tiny(seed=seed, m=4, n=33, heads=1, scale_mode="one")
    inp.weights = np.ones((4, 1), np.float32)
    L = logits_fn(inp.q, inp.kv, inp.kv_scale, inp.weights, inp.ks, inp.ke)
    Qt = torch.from_numpy(torch_decode(inp.q)[:, 0, :])
    Kt = torch.from_numpy(torch_decode(inp.kv))
    want = torch.clamp(Qt @ Kt.T, min=0).numpy()
    if not np.array_equal(L, want):
        return False, f"max diff {np.abs(L - want).max()}"
    return True, ""


def check_nonnegative_closed_form(logits_fn, seed=13):
    """All q, kv >= 0: the ReLU is the identity, so
    logits[i, j] = kv_scale[j] * (sum_h w[i,h] q[i,h,:]) . kv[j, :]."""
    inp = _tiny(seed=seed, m=3, n=40)
    inp.q = inp.q & 0x7F     # clear sign bits
    inp.kv = inp.kv & 0x7F
    L = logits_fn(inp.q, inp.kv, inp.kv_scale, inp.weights, inp.ks, inp.ke)
    Q = torch.from_numpy(torch_decode(inp.q))
    K = torch.from_numpy(torch_decode(inp.kv))
    w = torch.from_numpy(inp.weights.astype(np.float64))
    qw = torch.einsum("ih,ihd->id", w, Q)
    want = (qw @ K.T) * torch.from_numpy(inp.kv_scale.astype(np.float64))[None, :]
    want = want.numpy()
    if not np.allclose(L, want, rtol=1e-12, atol=1e-12):
        return False, f"max rel diff {np.max(np.abs(L - want) / np.maximum(1, np.abs(want)))}"
    return True, ""


def check_key_permutation(logits_fn, seed=14):
    """Permuting keys (kv rows with their scales) permutes logits columns identically."""
    inp = _tiny(seed=seed, m=3, n=50)
    perm = np.random.default_rng(seed).permutation(50)
    L = logits_fn(inp.q, inp.kv, inp.kv_scale, inp.weights, inp.ks, inp.ke)
    Lp = logits_fn(inp.q, inp.kv[perm], inp.kv_scale[perm], inp.weights, inp.ks, inp.ke)
    if not np.array_equal(L[:, perm], Lp):
        return False, "column permutation not equivariant"
    return True, ""


def check_head_permutation(logits_fn, seed=15):
    """Permuting heads of q together with weights leaves logits unchanged."""
    inp = _tiny(seed=seed, m=3, n=30, weight_mode="signed")
    perm = np.random.default_rng(seed).permutation(H)
    L = logits_fn(inp.q, inp.kv, inp.kv_scale, inp.weights, inp.ks, inp.ke)
    Lp = logits_fn(np.ascontiguousarray(inp.q[:, perm]), inp.kv, inp.kv_scale,
                   np.ascontiguousarray(inp.weights[:, perm]), inp.ks, inp.ke)
    if not np.allclose(L, Lp, rtol=1e-12, atol=1e-12):
        return False, "head permutation changed logits"
    return True, ""


def check_linearity_in_weights(logits_fn, seed=16):
    """logits(w1 + w2) = logits(w1) + logits(w2) (the ReLU does not see w)."""
    inp = _tiny(seed=seed, m=3, n=30, weight_mode="signed")
    w2 = np.random.default_rng(seed).uniform(-1, 1, inp.weights.shape).astype(np.float32)
    L1 = logits_fn(inp.q, inp.kv, inp.kv_scale, inp.weights, inp.ks, inp.ke)
    L2 = logits_fn(inp.q, inp.kv, inp.kv_scale, w2, inp.ks, inp.ke)
    w12 = inp.weights.astype(np.float64) + w2.astype(np.float64)
    # w1 + w2 may not be a float32; feed the float64 sum directly
    L12 = logits_fn(inp.q, inp.kv, inp.kv_scale, w12, inp.ks, inp.ke)
    if not np.allclose(L12, L1 + L2, rtol=1e-11, atol=1e-9):
        return False, "not linear in the weights"
    return True, ""


def check_scale_homogeneity(logits_fn, seed=17):
    """Doubling kv_scale[j] (>= 0) doubles column j; zero scale gives zero logits."""
    inp = _tiny(seed=seed, m=3, n=30)
    L = logits_fn(inp.q, inp.kv, inp.kv_scale, inp.weights, inp.ks, inp.ke)
    L2 = logits_fn(inp.q, inp.kv, (inp.kv_scale * 2).astype(np.float32), inp.weights, inp.ks, inp.ke)
    L0 = logits_fn(inp.q, inp.kv, np.zeros_like(inp.kv_scale), inp.weights, inp.ks, inp.ke)
    if not np.array_equal(L2, 2 * L):
        return False, "scale not homogeneous"
    if not np.all(L0 == 0):
        return False, "zero scale gives non-zero logits"
    return True, ""


def check_mask(logits_fn, seed=18):
    """-inf exactly outside [ks, ke), finite inside; empty windows are all -inf."""
    m, n = 6, 64
    inp = _tiny(seed=seed, m=m, n=n)
    ks = np.array([0, 5, 10, 63, 20, 7], np.int32)
    ke = np.array([64, 6, 40, 64, 20, 7], np.int32)   # rows 4, 5 empty
    L = logits_fn(inp.q, inp.kv, inp.kv_scale, inp.weights, ks, ke)
    cols = np.arange(n)
    inside = (cols[None, :] >= ks[:, None]) & (cols[None, :] < ke[:, None])
    if not np.all(np.isfinite(L[inside])):
        return False, "non-finite logit inside the window"
    if not np.all(L[~inside] == -np.inf):
        return False, "outside entry is not -inf"
    return True, ""


def check_window_independence(logits_fn, seed=19):
    """A row's in-window logits do not depend on the window bounds or on other rows."""
    inp = _tiny(seed=seed, m=4, n=48)
    full = logits_fn(inp.q, inp.kv, inp.kv_scale, inp.weights, inp.ks, inp.ke)
    ks = np.array([3, 0, 17, 40], np.int32)
    ke = np.array([30, 48, 18, 48], np.int32)
    part = logits_fn(inp.q, inp.kv, inp.kv_scale, inp.weights, ks, ke)
    for i in range(4):
        if not np.array_equal(part[i, ks[i]:ke[i]], full[i, ks[i]:ke[i]]):
            return False, f"row {i} depends on its window"
    one = logits_fn(inp.q[2:3], inp.kv, inp.kv_scale, inp.weights[2:3], inp.ks[2:3], inp.ke[2:3])
    if not np.array_equal(one[0], full[2]):
        return False, "row depends on other rows"
    return True, ""


ALL_LOGIT_CHECKS = [
    check_exact_small,
    check_relu_matmul_special_case,
    check_nonnegative_closed_form,
    check_key_permutation,
    check_head_permutation,
    check_linearity_in_weights,
    check_scale_homogeneity,
    check_mask,
    check_window_independence,
]

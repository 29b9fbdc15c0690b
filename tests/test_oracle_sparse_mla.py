"""Pins of the sparse MLA oracle (the attention over the indexer's top-k slots) against closed forms,
plus planted mistakes in copies of it that the pins must catch.

Constants are written out by hand: e4m3fn codes 0x38 = 1.0, 0x40 = 2.0, 0x30 = 0.5, 0xB8 = -1.0,
0x44 = 3.0, 0x00 = 0; bf16 bit patterns 0x3F80 = 1.0, 0x3F00 = 0.5, 0xBF80 = -1.0, 0x0000 = 0.
"""

import math

import numpy as np
import pytest

from oracle.indexer_oracle import e4m3fn_value_table
from oracle.sparse_mla_oracle import MLA_DQK, MLA_DV, decode_bf16, sparse_mla

D, DV = MLA_DQK, MLA_DV


def _q(T, H, fill=0x0000):
    return np.full((T, H, D), fill, dtype=np.uint16)


def _kv(S, fill=0x00):
    return np.full((S, D), fill, dtype=np.uint8)


# ---------------------------------------------------------------------------
# pins: each takes the attention function and asserts a property the reading fixes
# ---------------------------------------------------------------------------

def pin_one_valid_slot(fn):
    """One valid slot among invalid entries: o is that slot's scaled latent, lse its score."""
    q = _q(1, 2)
    q[0, 0, :] = 0x3F80          # 1.0
    q[0, 1, :] = 0x3F00          # 0.5
    kv = _kv(4, 0x30)
    kv[2, :] = 0x38              # slot 2: every value 1.0
    sc = np.array([3.0, 3.0, 0.25, 3.0], np.float32)
    idx = np.array([[-1, 2, 7, -3]], np.int32)
    o, lse = fn(q, kv, sc, idx, 0.125)
    assert o.shape == (1, 2, DV) and lse.shape == (1, 2)
    # s = 0.125 * 576 * q * 0.25
    assert np.allclose(lse[0], [18.0, 9.0], rtol=0, atol=1e-12)
    assert np.allclose(o, 0.25, rtol=0, atol=1e-12)


def pin_zero_query_is_mean(fn):
    """q = 0 gives equal scores: o is the plain mean of the selected scaled rows, lse = log n."""
    rng = np.random.default_rng(3)
    codes = np.array([0x38, 0x40, 0x30, 0xB8, 0x44], np.uint8)
    kv = codes[rng.integers(0, 5, (6, D))]
    sc = np.array([0.5, 1.0, 2.0, 0.75, 1.5, 3.0], np.float32)
    val = {0x38: 1.0, 0x40: 2.0, 0x30: 0.5, 0xB8: -1.0, 0x44: 3.0}
    idx = np.array([[0, 3, 4, 1]], np.int32)
    o, lse = fn(_q(1, 3), kv, sc, idx, 0.3)
    want = np.mean([[val[int(c)] * float(sc[j]) for c in kv[j, :DV]] for j in (0, 3, 4, 1)], axis=0)
    for h in range(3):
        assert np.allclose(o[0, h], want, rtol=0, atol=1e-12)
    assert np.allclose(lse, math.log(4.0), rtol=0, atol=1e-12)


def pin_two_slot_logistic(fn):
    """Two slots: the weights are the logistic function of the score gap."""
    q = _q(1, 1)
    q[0, 0, 0] = 0x3F80                        # q = e_0
    kv = _kv(2)
    kv[0, 0], kv[0, 1:DV] = 0x40, 0x38         # row 0: 2.0, then 1.0
    kv[1, 0], kv[1, 1:DV] = 0xB8, 0x30         # row 1: -1.0, then 0.5
    kv[:, DV:] = 0x44                          # rotary part: never a value
    sc = np.array([1.0, 2.0], np.float32)
    o, lse = fn(q, kv, sc, np.array([[1, 0]], np.int32), 0.5)
    s0, s1 = 0.5 * 2.0 * 1.0, 0.5 * -1.0 * 2.0
    p0 = 1.0 / (1.0 + math.exp(s1 - s0))
    p1 = 1.0 - p0
    assert abs(o[0, 0, 0] - (2.0 * p0 - 2.0 * p1)) < 1e-12
    assert np.allclose(o[0, 0, 1:], 1.0 * p0 + 1.0 * p1, rtol=0, atol=1e-12)
    assert abs(lse[0, 0] - math.log(math.exp(s0) + math.exp(s1))) < 1e-12


def pin_duplicates_count_twice(fn):
    """A slot listed twice carries twice the weight."""
    kv = _kv(3)
    kv[0, :] = 0x40      # 2.0
    kv[2, :] = 0xB8      # -1.0
    sc = np.ones(3, np.float32)
    o, lse = fn(_q(1, 1), kv, sc, np.array([[0, 0, 2]], np.int32), 1.0)
    assert np.allclose(o, (2 * 2.0 - 1.0) / 3.0, rtol=0, atol=1e-12)
    assert abs(lse[0, 0] - math.log(3.0)) < 1e-12


def pin_no_valid_slot(fn):
    """No valid slot: o = 0 and lse = -inf."""
    kv = _kv(2, 0x38)
    q = _q(1, 2, 0x3F80)
    o, lse = fn(q, kv, np.ones(2, np.float32), np.array([[-1, 2, 5, -9]], np.int32), 1.0)
    assert np.all(o == 0.0)
    assert np.all(np.isneginf(lse))


def pin_order_and_padding_invariance(fn):
    """The result depends on the multiset of valid slots only: order and invalid entries do not matter."""
    rng = np.random.default_rng(11)
    S = 40
    q1 = np.array([0x3F80, 0x3F00, 0xBF80, 0x0000], np.uint16)[rng.integers(0, 4, (1, 3, D))]
    q = np.concatenate([q1, q1])   # both tokens ask the same query
    kv = np.array([0x38, 0x40, 0x30, 0xB8, 0x00], np.uint8)[rng.integers(0, 5, (S, D))]
    sc = rng.uniform(0.5, 1.5, S).astype(np.float32)
    base = rng.permutation(S)[:12].astype(np.int32)
    a = np.stack([base, base[::-1]])
    shuffled = rng.permutation(base)
    b_row = np.concatenate([shuffled[:5], [-1, S, S + 9], shuffled[5:], [-4]]).astype(np.int32)
    b = np.stack([b_row, b_row])
    oa, la = fn(q, kv, sc, a, 0.05)
    ob, lb = fn(q, kv, sc, b[:, :], 0.05)
    assert np.allclose(oa, ob, rtol=1e-12, atol=1e-12) and np.allclose(la, lb, rtol=1e-12, atol=1e-12)
    # both tokens hold the same slots in opposite order
    assert np.allclose(oa[0], oa[1], rtol=1e-12, atol=1e-12)


def pin_values_are_the_latent(fn):
    """Only the first 512 values of a row are its value; the rotary tail only moves scores.  With q
    on the tail alone and identical tails, scores are equal and o is the mean latent."""
    q = _q(1, 1)
    q[0, 0, DV:] = 0x3F80
    kv = _kv(3)
    kv[:, DV:] = 0x30                                # every tail 0.5
    kv[0, :DV], kv[1, :DV], kv[2, :DV] = 0x38, 0x40, 0xB8
    sc = np.ones(3, np.float32)
    o, lse = fn(q, kv, sc, np.array([[0, 1, 2]], np.int32), 0.25)
    assert np.allclose(o, (1.0 + 2.0 - 1.0) / 3.0, rtol=0, atol=1e-12)
    s = 0.25 * (D - DV) * 0.5
    assert abs(lse[0, 0] - (s + math.log(3.0))) < 1e-12


def pin_heads_are_independent(fn):
    """Each head normalises over the slots on its own: opposite queries pick opposite slots."""
    q = _q(1, 2)
    q[0, 0, 0] = 0x3F80
    q[0, 1, 0] = 0xBF80
    kv = _kv(2)
    kv[0, 0], kv[0, 1:DV] = 0x7E, 0x38      # 0x7E = 448
    kv[1, 0], kv[1, 1:DV] = 0xFE, 0x40      # -448
    sc = np.ones(2, np.float32)
    o, lse = fn(q, kv, sc, np.array([[0, 1]], np.int32), 4.0)
    # score gap 4 * 896 = 3584: the other slot's weight underflows to exactly 0
    assert np.allclose(o[0, 0, 1:], 1.0, rtol=0, atol=1e-12) and o[0, 0, 0] == 448.0
    assert np.allclose(o[0, 1, 1:], 2.0, rtol=0, atol=1e-12) and o[0, 1, 0] == -448.0
    assert abs(lse[0, 0] - 4.0 * 448.0) < 1e-9 and abs(lse[0, 1] - 4.0 * 448.0) < 1e-9


PINS = [pin_one_valid_slot, pin_zero_query_is_mean, pin_two_slot_logistic, pin_duplicates_count_twice,
        pin_no_valid_slot, pin_order_and_padding_invariance, pin_values_are_the_latent,
        pin_heads_are_independent]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pins(pin):
    pin(sparse_mla)


def test_bf16_decode_points():
    bits = np.array([0x3F80, 0x3F00, 0xBF80, 0x0000, 0x4049, 0x7F80, 0x0001], np.uint16)
    want = [1.0, 0.5, -1.0, 0.0, 3.140625, math.inf, 2.0 ** -133]
    assert list(decode_bf16(bits)) == want


# ---------------------------------------------------------------------------
# planted mistakes: each must fail at least one pin
# ---------------------------------------------------------------------------

def _mutant(variant):
    table = e4m3fn_value_table()

    def fn(q_bits, kv_codes, kv_scale, indices, sm_scale, dv=DV):
        T, H, Dd = q_bits.shape
        S = kv_codes.shape[0]
        o = np.zeros((T, H, dv))
        lse = np.full((T, H), -np.inf)
        for t in range(T):
            idx = np.asarray(indices[t], np.int64)
            if variant == "clamp_invalid":
                sel = np.clip(idx, 0, S - 1)
            else:
                sel = idx[(idx >= 0) & (idx < S)]
            if variant == "dedupe":
                sel = np.unique(sel)
            if sel.size == 0:
                continue
            raw = table[kv_codes[sel]]
            sc = np.asarray(kv_scale, np.float64)[sel][:, None]
            K = raw * sc
            V = raw[:, :dv] if variant == "values_unscaled" else K[:, :dv]
            if variant == "values_from_tail":
                V = K[:, Dd - dv:]
            Q = decode_bf16(q_bits[t])
            s = (Q @ K.T) * (1.0 if variant == "no_sm_scale" else sm_scale)
            if variant == "softmax_over_heads":
                m = s.max(axis=0, keepdims=True)
                e = np.exp(s - m)
                z = e.sum(axis=0, keepdims=True)
            else:
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                z = e.sum(axis=1, keepdims=True)
            o[t] = (e / z) @ V
            if variant == "lse_is_max":
                lse[t] = s.max(axis=1)
            else:
                mx = s.max(axis=1, keepdims=True)
                lse[t] = (mx + np.log(np.exp(s - mx).sum(axis=1, keepdims=True)))[:, 0]
        return o, lse
    return fn


MUTANTS = ["clamp_invalid", "dedupe", "values_unscaled", "values_from_tail", "no_sm_scale",
           "softmax_over_heads", "lse_is_max"]


@pytest.mark.parametrize("variant", MUTANTS)
def test_pins_catch_planted_mistake(variant):
    fn = _mutant(variant)
    caught = []
    for pin in PINS:
        try:
            pin(fn)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the '{variant}' mutant"


def test_unmutated_copy_passes_every_pin():
    fn = _mutant("none")
    for pin in PINS:
        pin(fn)

"""Pins for the oracle's per-row fp8 quantiser (quant_fp8_rows).

The encoder itself is pinned by tests/golden/e4m3fn_encoder_pins.json; these
pins fix the per-row scale rule from closed forms and by brute force, so a
plausible slip (the scale inverted, |x| forgotten, a wrong maximum, a code
decided off the row scale) fails at least one of them.
"""

import json
import os

import numpy as np
import pytest

import oracle.indexer_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
PINS = json.load(open(os.path.join(HERE, "golden", "e4m3fn_encoder_pins.json")))
TABLE = O.e4m3fn_value_table()
FINITE = np.nonzero(np.isfinite(TABLE))[0]


def _nearest_code_bruteforce(y: float) -> int:
    """Nearest finite e4m3fn code to y by exhaustive search, ties to the even code
    (lowest mantissa bit 0), magnitudes past 448 saturating."""
    if abs(y) >= 448.0:
        return 0x7E if y > 0 else 0xFE
    d = np.abs(TABLE[FINITE] - y)
    best = FINITE[d == d.min()]
    # +0 and -0 are both at distance |y| from a tiny y: keep y's sign
    best = [c for c in best if (c & 0x80) == (0x80 if np.signbit(y) else 0)] or list(best)
    if len(best) > 1:
        best = [c for c in best if c % 2 == 0]
    return int(best[0])


def test_row_with_amax_448_reuses_the_encoder_pins():
    # amax = 448 gives inv = 1 exactly, so every code is the plain encoding of x
    pins = PINS["ties"] + PINS["subnormals"]
    x = np.array([[448.0] + [p["x"] for p in pins]], dtype=np.float32)
    codes, scale = O.quant_fp8_rows(x)
    assert scale[0] == np.float32(1.0)
    assert codes[0, 0] == 126
    assert [int(c) for c in codes[0, 1:]] == [p["code"] for p in pins]


def test_largest_magnitude_maps_to_largest_code_with_its_sign():
    x = np.array([[-3.0, 1.0, 2.0, 0.5], [0.25, -0.125, 0.0, 0.0625]], dtype=np.float32)
    codes, scale = O.quant_fp8_rows(x)
    assert codes[0, 0] == 0xFE            # -448
    assert codes[1, 0] == 0x7E            # +448
    assert scale[0] == np.float32(3.0) / np.float32(448.0)
    assert scale[1] == np.float32(0.25) / np.float32(448.0)
    # 1.0 * 448/3 = 149.33 -> nearest e4m3fn is 144 = 2**7 * 1.125 (step 16 in [128, 256)):
    # exponent field 14, mantissa 001 -> 0x71
    assert codes[0, 1] == 0x71
    # -0.125 * 448/0.25 = -224 = -(2**7 * 1.75): 0xF6; 0.0625 * 1792 = 112 = 2**6 * 1.75: 0x6E;
    # zero stays +0
    assert codes[1, 1] == 0xF6 and codes[1, 3] == 0x6E and codes[1, 2] == 0


def test_zero_row_has_unit_scale_and_zero_codes():
    codes, scale = O.quant_fp8_rows(np.zeros((2, 16), np.float32))
    assert np.all(codes == 0) and np.all(scale == np.float32(1.0))


@pytest.mark.parametrize("k", [-20, -7, -1, 1, 5, 30])
def test_power_of_two_homogeneity(k):
    # scaling a row by 2**k scales amax and scale by 2**k exactly and leaves y, hence the codes, unchanged
    rng = np.random.default_rng(100 + k)
    x = rng.standard_normal((4, 128)).astype(np.float32)
    c0, s0 = O.quant_fp8_rows(x)
    c1, s1 = O.quant_fp8_rows(x * np.float32(2.0 ** k))
    assert np.array_equal(c0, c1)
    assert np.array_equal(s1, s0 * np.float32(2.0 ** k))


def test_codes_are_the_nearest_representable_value_by_brute_force():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal((3, 40)) * 10.0 ** rng.integers(-4, 4, (3, 1)),
                        rng.uniform(-1, 1, (2, 40)) ** 7], axis=0).astype(np.float32)
    codes, scale = O.quant_fp8_rows(x)
    for r in range(x.shape[0]):
        amax = np.float32(np.abs(x[r]).max())
        inv = np.float32(448.0) / amax
        for d in range(x.shape[1]):
            y = float(np.float32(x[r, d] * inv))
            assert codes[r, d] == _nearest_code_bruteforce(y), (r, d, y)


def test_dequantised_values_are_within_half_a_code_step():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((8, 128)) * 3).astype(np.float32)
    codes, scale = O.quant_fp8_rows(x)
    back = TABLE[codes] * scale[:, None].astype(np.float64)
    # e4m3fn: relative half-step 2**-4 for normal codes; absolute half-step 2**-10 * scale below 2**-6
    tol = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * scale[:, None]) * (1 + 1e-6)
    assert np.all(np.abs(back - x) <= tol)


def _mutant(variant):
    def quant(x):
        x = np.asarray(x, dtype=np.float32)
        if variant == "no_abs":
            amax = np.max(x, axis=1)
        elif variant == "mean_abs":
            amax = np.mean(np.abs(x), axis=1)
        else:
            amax = np.max(np.abs(x), axis=1)
        amax = np.where(amax > 0, amax, np.float32(448.0)).astype(np.float32)
        if variant == "inverted_scale":
            inv = (amax / np.float32(448.0)).astype(np.float32)
        elif variant == "max_447":
            inv = (np.float32(447.0) / amax).astype(np.float32)
        else:
            inv = (np.float32(448.0) / amax).astype(np.float32)
        y = (x * inv[:, None]).astype(np.float32)
        if variant == "truncate":
            y = np.trunc(y * 8) / 8
        codes = O.encode_e4m3fn(y.astype(np.float64))
        scale = (amax / np.float32(448.0)).astype(np.float32)
        if variant == "scale_is_inv":
            scale = inv
        return codes, scale
    return quant


@pytest.mark.parametrize("variant", ["no_abs", "mean_abs", "inverted_scale", "max_447", "truncate", "scale_is_inv"])
def test_pins_catch_planted_quantiser_mistakes(variant, monkeypatch):
    monkeypatch.setattr(O, "quant_fp8_rows", _mutant(variant))
    checks = [test_row_with_amax_448_reuses_the_encoder_pins,
              test_largest_magnitude_maps_to_largest_code_with_its_sign,
              test_codes_are_the_nearest_representable_value_by_brute_force,
              test_dequantised_values_are_within_half_a_code_step]
    failed = 0
    for c in checks:
        try:
            c()
        except AssertionError:
            failed += 1
    assert failed > 0, f"no pin caught mutant {variant}"

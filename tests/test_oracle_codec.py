"""e4m3fn codec pins for the oracle (decode table, encoder) and the input generator's cast."""

import json
import math
import os

import numpy as np
import torch

from oracle import decode_e4m3fn, e4m3fn_value_table, encode_e4m3fn
from tests.oracle_pins import torch_decode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3fn_encoder_pins.json")


def _pins():
    with open(GOLDEN) as f:
        g = json.load(f)
    out = []
    for key in ("ties", "subnormals", "saturating", "nan"):
        for p in g[key]:
            x = float("nan") if p["x"] == "nan" else float(p["x"])
            out.append((key, x, int(p["code"])))
    return out


def test_decode_table_matches_torch_upcast_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3fn_value_table()
    theirs = torch_decode(codes)
    nan_ours = np.isnan(ours)
    assert np.array_equal(nan_ours, np.isnan(theirs))
    assert set(np.nonzero(nan_ours)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan_ours], theirs[~nan_ours])
    # signed zero is kept
    assert math.copysign(1.0, ours[0x80]) == -1.0


def test_decode_definition_points():
    # values that follow from the E4M3 layout by hand
    pts = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
           0x40: 2.0, 0x3F: 1.875, 0x7E: 448.0, 0xFE: -448.0, 0xB8: -1.0, 0x77: 240.0}
    for c, v in pts.items():
        assert decode_e4m3fn(np.uint8(c)) == v, hex(c)


def test_encoder_page_pins():
    for kind, x, code in _pins():
        got = int(encode_e4m3fn(np.array([x]), saturate=True)[0])
        assert got == code, (kind, x, got, code)


def test_generator_cast_page_pins():
    # torch's cast (used by the input generator) on the round-to-nearest-even pins;
    # torch does not saturate, so only in-range pins apply to it.
    for kind, x, code in _pins():
        if kind in ("ties", "subnormals") or (kind == "nan"):
            got = int(torch.tensor([x], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)[0])
            assert got == code, (kind, x, got, code)


def test_encoder_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = decode_e4m3fn(codes)
    assert np.array_equal(encode_e4m3fn(vals), codes)


def test_encoder_matches_torch_cast_in_range():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(4000) * 3,
        rng.uniform(-448, 448, 2000),
        rng.uniform(-2 ** -6, 2 ** -6, 2000),
        # exact midpoints between neighbouring codes
        (decode_e4m3fn(np.arange(0, 0x7E, dtype=np.uint8)) + decode_e4m3fn(np.arange(1, 0x7F, dtype=np.uint8))) / 2,
    ]).astype(np.float32)
    ours = encode_e4m3fn(x.astype(np.float64), saturate=False)
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)

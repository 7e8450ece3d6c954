"""Pins for the E4M3 (8-bit float) part of the CPU oracle.

The value table and the encoder are checked against values the OCP 8-bit
floating point specification fixes (worked by hand into
tests/golden/e4m3_codes.json), against torch's float8_e4m3fn type (an
independent library decoding and round-to-nearest-even cast), and against
brute-force nearest search.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from conftest import GOLDEN
from oracle import fp8


def _golden():
    with open(os.path.join(GOLDEN, "e4m3_codes.json")) as f:
        return json.load(f)


def test_values_fixed_by_the_specification():
    g = _golden()
    for item in g["values"]:
        v = fp8.e4m3_value(item["code"])
        assert v == item["value"], item
        assert math.copysign(1.0, v) == math.copysign(1.0, item["value"]), item
    for c in g["nan_codes"]:
        assert math.isnan(fp8.e4m3_value(c))
    table = fp8.e4m3_table()
    assert int(np.isnan(table).sum()) == 2
    assert np.nanmax(table) == 448.0 and np.nanmin(table) == -448.0


def test_table_matches_torch_float8_e4m3fn():
    ours = fp8.e4m3_table()
    theirs = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(theirs))
    ok = ~np.isnan(ours)
    assert np.array_equal(ours[ok], theirs[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(theirs[ok]))


def test_rounding_cases_worked_by_hand():
    for item in _golden()["rounding"]:
        got = int(fp8.float_to_e4m3(np.float32(item["y"])))
        assert got == item["code"], item


def test_every_finite_code_round_trips():
    for c in range(256):
        v = fp8.e4m3_value(c)
        if math.isnan(v):
            continue
        assert int(fp8.float_to_e4m3(np.float32(v))) == c


def test_encoder_is_nearest_by_brute_force():
    rng = np.random.default_rng(811)
    y = np.concatenate([
        rng.normal(0, 1, 3000), rng.normal(0, 100, 1000), rng.normal(0, 0.01, 1000),
        rng.uniform(-448, 448, 1000)]).astype(np.float32)
    codes = fp8.float_to_e4m3(y)
    table = fp8.e4m3_table()
    finite = np.array([c for c in range(256) if not np.isnan(table[c])])
    for yi, ci in zip(y.astype(np.float64), codes):
        d = np.abs(table[finite] - yi)
        best = d.min()
        assert abs(table[ci] - yi) == best
        if np.count_nonzero(d == best) > 1 and best > 0:
            # a tie between two values: the even mantissa wins
            assert ci % 2 == 0


def test_exact_midpoints_go_to_the_even_code():
    table = fp8.e4m3_table()
    for c in range(0, 0x7E):
        mid = np.float32((table[c] + table[c + 1]) / 2)
        assert float(mid) == (table[c] + table[c + 1]) / 2  # exact in float32
        want = c if c % 2 == 0 else c + 1
        assert int(fp8.float_to_e4m3(mid)) == want
        assert int(fp8.float_to_e4m3(-mid)) == want | 0x80


def test_encoder_matches_torch_cast_in_range():
    rng = np.random.default_rng(812)
    y = np.concatenate([rng.normal(0, 1, 20000), rng.uniform(-448, 448, 5000),
                        rng.normal(0, 0.003, 5000)]).astype(np.float32)
    ours = fp8.float_to_e4m3(y)
    theirs = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_saturation_and_signs():
    y = np.array([448.0, 449.0, 463.9, 464.0, 1e30, -1e30, -0.0, 0.0], dtype=np.float32)
    assert list(fp8.float_to_e4m3(y)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x00]


def test_quantize_divides_in_float32():
    rng = np.random.default_rng(813)
    x = rng.normal(0, 1, 4000).astype(np.float32)
    # a power-of-two scale only moves the exponent
    assert np.array_equal(fp8.quantize(x * np.float32(4), 4.0), fp8.quantize(x, 1.0))
    # otherwise the quotient is the float32 one, not the float64 one
    s = np.float32(0.0123)
    q32 = (x / s).astype(np.float32)
    assert np.array_equal(fp8.quantize(x, s), fp8.float_to_e4m3(q32))
    with pytest.raises(ValueError):
        fp8.quantize(x, 0.0)


def test_dequantize_scales_the_code_values():
    codes = np.array([0x38, 0x40, 0xC5, 0x7E], dtype=np.uint8)
    assert list(fp8.dequantize(codes, 0.5)) == [0.5, 1.0, -1.625, 224.0]

"""Pins for the oracle's number-format routines (CPU only).

Each check compares the oracle with something other than itself: the OCP format
tables under tests/golden/, torch's float8_e4m3fn conversion (a library routine) and
numpy's float64 -> float16 conversion (a library routine, round to nearest even).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from conftest import load_golden


def test_e2m1_all_16_codes_match_ocp_table():
    table = load_golden("ocp_fp4_e2m1_values.txt")
    assert sorted(table) == list(range(16))
    for code, val in table.items():
        got = oracle.e2m1(code)
        assert got == val and math.copysign(1.0, got) == math.copysign(1.0, val), hex(code)


def test_e4m3fn_anchor_codes_match_ocp_table():
    anchors = load_golden("ocp_fp8_e4m3fn_anchors.txt")
    for code, val in anchors.items():
        got = oracle.e4m3fn(code)
        if math.isnan(val):
            assert math.isnan(got), hex(code)
        else:
            assert got == val and math.copysign(1.0, got) == math.copysign(1.0, val), hex(code)


def test_e4m3fn_all_256_codes_match_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    for code in range(256):
        got = oracle.e4m3fn(code)
        want = float(ref[code])
        if code in (0x7F, 0xFF):
            assert math.isnan(got) and math.isnan(want)
            continue
        assert got == want and math.copysign(1.0, got) == math.copysign(1.0, want), hex(code)


def test_e4m3fn_scale_range_used_by_workloads():
    # the synthetic scale codes 0x08..0x20 are exactly the finite positive values in [2^-6, 2^-3]
    vals = sorted(oracle.e4m3fn(c) for c in range(256) if c not in (0x7F, 0xFF))
    in_range = [v for v in vals if 2.0 ** -6 <= v <= 2.0 ** -3]
    assert in_range == [oracle.e4m3fn(c) for c in range(0x08, 0x21)]


def _numpy_f16_bits(x: float) -> int:
    with np.errstate(over="ignore"):
        return int(np.array([x], dtype=np.float64).astype(np.float16).view(np.uint16)[0])


def test_f16_rne_matches_numpy_on_grid_ties_and_edges():
    rng = np.random.default_rng(7)
    xs = []
    # every finite half and the exact midpoints between neighbours (ties), both signs
    halves = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (halves[:-1] + halves[1:]) / 2.0
    xs += list(halves[::7]) + list(mids[::5])
    # just below / above midpoints
    xs += list(np.nextafter(mids[::11], 0)) + list(np.nextafter(mids[::11], np.inf))
    # overflow boundary and beyond
    xs += [65504.0, 65519.999, 65520.0, 65536.0, 1e9, 6.0e-8, 2.0 ** -25, 2.0 ** -24 * 1.5,
           2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 0.0]
    # random magnitudes across the whole range
    xs += list(np.ldexp(rng.random(4000) + 0.5, rng.integers(-30, 18, 4000)))
    for x in xs:
        for s in (1.0, -1.0):
            v = s * float(x)
            assert oracle.f16_rne(v) == _numpy_f16_bits(v), v


def test_ulp16_definition_points():
    bits = np.array([0x0000, 0x0001, 0x0400, 0x3C00, 0x7BFF, 0xBC00], dtype=np.uint16)
    u = oracle.ulp16(bits)
    assert list(u) == [2.0 ** -24, 2.0 ** -24, 2.0 ** -24, 2.0 ** -10, 32.0, 2.0 ** -10]


def test_tolerance_is_two_ulp16_plus_abssum_term():
    # hand-computed bounds: fp16 1.0 (0x3C00) has spacing 2^-10, 2048.0 (0x6800) has 2,
    # 0 and subnormals 2^-24, -0.5 (0xB800) 2^-11, an infinity the top binade's 32
    bits = np.array([0x3C00, 0x6800, 0x0000, 0x0001, 0xB800, 0x7C00], np.uint16)
    abssum = np.array([0.0, 100.0, 1.0, 0.0, 3.0, 0.0])
    want = np.array([2 * 2.0 ** -10, 2 * 2.0 + 1e-3, 2 * 2.0 ** -24 + 1e-5, 2 * 2.0 ** -24,
                     2 * 2.0 ** -11 + 3e-5, 2 * 32.0])
    assert np.allclose(oracle.tolerance(bits, abssum), want, rtol=0, atol=1e-15)
    # the bound scales with the abssum term alone when the value is 0
    assert oracle.tolerance(np.array([0], np.uint16), np.array([1e6]))[0] == 2 * 2.0 ** -24 + 10.0

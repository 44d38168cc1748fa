"""Pins of the oracle's fp8 codecs and bf16 rounding (CPU only).

The oracle's encoder/decoder are checked against things other than
themselves: the format constants the pages and the OCP spec fix, torch's own
CPU float8 casts (an independent implementation), and exact rational
arithmetic for the bf16 output rounding.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import fp8_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TORCH_F8 = {O.E4M3: torch.float8_e4m3fn, O.E5M2: torch.float8_e5m2}


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- constants

def test_format_constants_golden():
    g = _golden("format_constants.json")
    assert O.fmt_max(O.E4M3) == g["e4m3"]["max"]
    assert O.fmt_max(O.E5M2) == g["e5m2"]["max"]
    for fmt, key in ((O.E4M3, "e4m3"), (O.E5M2, "e5m2")):
        for code_hex, val in g[key]["codes"].items():
            got = O.decode(int(code_hex, 16), fmt)
            if val == "nan":
                assert math.isnan(got)
            elif val in ("inf", "-inf"):
                assert got == float(val)
            else:
                assert got == float(Fraction(val)), (key, code_hex)


def test_decode_matches_torch_all_codes():
    for fmt, tdt in TORCH_F8.items():
        codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
        ref = codes.view(tdt).to(torch.float64).numpy()
        got = O.decode_table(fmt)
        assert np.array_equal(np.isnan(ref), np.isnan(got))
        ok = ~np.isnan(ref)
        assert np.array_equal(ref[ok], got[ok])
        # signed zeros
        assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


# ---------------------------------------------------------------- round trip

@pytest.mark.parametrize("fmt", O.FORMATS)
def test_round_trip_all_256_codes(fmt):
    vals = O.decode_table(fmt)
    codes = np.arange(256)
    enc = O.encode(vals.astype(np.float32), fmt)
    for c in range(256):
        v = vals[c]
        sign = c & 0x80
        if math.isnan(v):
            assert enc[c] == (0x7F | sign)
        elif math.isinf(v):  # e5m2 +-inf saturates to +-max
            assert fmt == O.E5M2 and enc[c] == (0x7B | sign)
        else:
            assert enc[c] == codes[c], (fmt, hex(c), v)


# ---------------------------------------------------------------- RNE

@pytest.mark.parametrize("fmt", O.FORMATS)
def test_midpoints_round_to_even_and_neighbours_to_nearest(fmt):
    vals = O.decode_table(fmt)
    finite = [c for c in range(128) if math.isfinite(vals[c])]
    n_mid = 0
    for lo, hi in zip(finite[:-1], finite[1:]):
        mid = np.float32((vals[lo] + vals[hi]) / 2)
        assert float(mid) == (vals[lo] + vals[hi]) / 2  # exact in fp32
        even = lo if lo % 2 == 0 else hi
        up = np.nextafter(mid, np.float32(np.inf))
        dn = np.nextafter(mid, np.float32(-np.inf))
        for sgn in (1, -1):
            got = O.encode(np.array([sgn * mid, sgn * up, sgn * dn], np.float32), fmt)
            s = 0x80 if sgn < 0 else 0
            assert got[0] == (even | s)
            assert got[1] == (hi | s)
            assert got[2] == (lo | s)
        n_mid += 1
    assert n_mid == {O.E4M3: 126, O.E5M2: 123}[fmt]


@pytest.mark.parametrize("fmt", O.FORMATS)
def test_encode_matches_torch_on_all_bf16_in_range(fmt):
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    x = bits.view(torch.bfloat16).to(torch.float32)
    keep = torch.isfinite(x) & (x.abs() <= O.fmt_max(fmt))
    x = x[keep]
    ref = x.to(TORCH_F8[fmt]).view(torch.uint8).numpy()
    got = O.encode(x.numpy(), fmt)
    assert np.array_equal(ref, got)


@pytest.mark.parametrize("fmt", O.FORMATS)
def test_encode_matches_torch_on_random_fp32_in_range(fmt):
    g = np.random.default_rng(1234)
    b = g.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    x = b.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) <= O.fmt_max(fmt))]
    # concentrate half the samples on the interesting exponent range
    y = (g.standard_normal(1_000_000) * O.fmt_max(fmt) / 8).astype(np.float32)
    x = np.concatenate([x, y[np.abs(y) <= O.fmt_max(fmt)]])
    ref = torch.from_numpy(x).to(TORCH_F8[fmt]).view(torch.uint8).numpy()
    assert np.array_equal(ref, O.encode(x, fmt))


@pytest.mark.parametrize("fmt", O.FORMATS)
def test_saturation_and_specials(fmt):
    mx = O.fmt_max(fmt)
    max_code = {O.E4M3: 0x7E, O.E5M2: 0x7B}[fmt]
    x = np.array([mx, mx * (1 + 2**-20), 1e30, np.inf, -np.inf, -mx * 3,
                  0.0, -0.0, 1e-30, -1e-30, np.nan, -np.nan], dtype=np.float32)
    got = O.encode(x, fmt)
    exp = [max_code, max_code, max_code, max_code, 0x80 | max_code, 0x80 | max_code,
           0x00, 0x80, 0x00, 0x80, 0x7F, 0xFF]
    assert list(got) == exp


# ---------------------------------------------------------------- bf16 RNE

def _bf16_exact(fr: Fraction) -> int:
    """Independent exact RNE of a rational to bf16 bits (normal range)."""
    if fr == 0:
        return 0
    sign = 0x8000 if fr < 0 else 0
    a = abs(fr)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    sp = Fraction(2) ** (e - 7)
    q = a / sp
    fl = math.floor(q)
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = float(fl * sp)
    return sign | int(np.array([v], np.float32).view(np.uint32)[0] >> 16)


def test_bf16_rounding_matches_torch_from_fp32():
    g = np.random.default_rng(7)
    x = (g.standard_normal(500_000) * 10.0 ** g.uniform(-20, 20, 500_000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ref, O.bf16_bits(x.astype(np.float64)))


def test_bf16_rounding_exact_on_fp64_ties_and_neighbours():
    g = np.random.default_rng(8)
    vals = []
    for _ in range(3000):
        # a bf16 value plus exactly half a bf16 ulp (a tie), and fp64 neighbours
        m = int(g.integers(128, 256))
        e = int(g.integers(-40, 40))
        tie = (m + 0.5) * 2.0 ** (e - 7)
        vals += [tie, np.nextafter(tie, np.inf), np.nextafter(tie, -np.inf), -tie]
    vals = np.array(vals)
    got = O.bf16_bits(vals)
    for v, b in zip(vals, got):
        assert b == _bf16_exact(Fraction(float(v))), v

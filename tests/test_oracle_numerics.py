"""Pins of the oracle's number formats against library casts, a published spec and exact arithmetic."""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import numerics as nu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- bf16

def test_bf16_decode_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = nu.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_bf16_round_matches_torch_on_fp32_values():
    rng = np.random.default_rng(1)
    raw = rng.integers(0, 2**32, size=400_000, dtype=np.uint64).astype(np.uint32)
    v = raw.view(np.float32)
    v = v[np.isfinite(v)]
    # add values sitting exactly on bf16 midpoints (ties) and next to them
    mids = (rng.integers(0, 2**16, size=20_000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    mids = mids[np.isfinite(mids)]
    v = np.concatenate([v, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
                        np.float32([0.0, -0.0, 1e-45, -1e-45, 3.4e38, -3.4e38])])
    ours = nu.f64_to_bf16_bits(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def _nearest_bf16_exact(x: float) -> Fraction:
    """Brute force: the representable bf16 value nearest to x, ties to an even last bit."""
    fx = Fraction(x)
    a = abs(fx)
    e = math.floor(math.log2(a)) if a else -133
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** max(e - 7, -133)
    lo = (a // q) * q
    hi = lo + q
    if a - lo < hi - a or (a - lo == hi - a and (lo / q) % 2 == 0):
        r = lo
    else:
        r = hi
    return r if fx >= 0 else -r


def test_bf16_round_is_single_rounding_from_fp64():
    # Values just above a bf16 midpoint that fp32 rounding would pull onto the midpoint:
    # a detour through fp32 then ties-to-even would round down; one RNE step rounds up.
    rng = np.random.default_rng(2)
    cases = []
    for _ in range(200):
        hi16 = int(rng.integers(0x3C00, 0x4400)) & ~1   # even last bf16 bit
        mid = np.uint32((hi16 << 16) | 0x8000).view(np.float32).astype(np.float64)
        cases.append(mid * (1 + 2.0 ** -40))
        cases.append(mid * (1 - 2.0 ** -40))
        cases.append(mid)
    cases += [1.0 + 2.0 ** -8 + 2.0 ** -30, -(1.0 + 2.0 ** -8 + 2.0 ** -30), 2.0 ** -130 * 1.3]
    v = np.array(cases)
    ours = nu.bf16_bits_to_f64(nu.f64_to_bf16_bits(v))
    for x, o in zip(v, ours):
        assert Fraction(float(o)) == _nearest_bf16_exact(float(x)), x
    # the double-rounding witness really differs from the fp32 detour
    w = np.array([1.0 + 2.0 ** -8 + 2.0 ** -30])
    detour = torch.from_numpy(w.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert nu.bf16_bits_to_f64(nu.f64_to_bf16_bits(w))[0] != detour[0]


def test_bf16_round_specials():
    v = np.array([np.inf, -np.inf, np.nan, 3.5e38, -0.0])
    b = nu.f64_to_bf16_bits(v)
    assert b[0] == 0x7F80 and b[1] == 0xFF80 and b[2] == 0x7FC0
    assert b[3] == 0x7F80          # above the largest finite bf16 -> inf
    assert b[4] == 0x8000


# ----------------------------------------------------------------------------- e4m3

def test_e4m3_table_matches_ocp_anchors():
    with open(os.path.join(GOLDEN, "ocp_e4m3_anchors.json")) as f:
        g = json.load(f)
    tab = nu.e4m3_value_table()
    for code_s, val_s in g["anchors"]:
        code, val = int(code_s, 16), float(val_s)
        if math.isnan(val):
            assert math.isnan(tab[code])
        else:
            assert tab[code] == val and math.copysign(1, tab[code]) == math.copysign(1, val)


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    ours = nu.e4m3_decode(codes)
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()
    finite = np.isfinite(ours)
    assert finite.sum() == 254 and np.nanmax(ours) == 448.0


def test_e4m3_encode_matches_torch_in_range():
    # every bf16 value (as fp32) times a few fixed scales, restricted to |v| <= 448
    bits = np.arange(65536, dtype=np.uint32)
    base = (bits << 16).astype(np.uint32).view(np.float32)
    rng = np.random.default_rng(3)
    rnd = rng.standard_normal(200_000).astype(np.float32) * np.float32(50)
    tab = nu.e4m3_value_table()
    fin = tab[np.isfinite(tab)]
    srt = np.unique(fin)
    mids = ((srt[:-1] + srt[1:]) / 2).astype(np.float32)   # exact ties
    pts = [base * np.float32(s) for s in (1.0, 2.0 ** -20, 2.0 ** 20, 0.37)]
    v = np.concatenate(pts + [rnd, mids, np.nextafter(mids, np.float32(np.inf)),
                              np.nextafter(mids, np.float32(-np.inf))])
    v = v[np.isfinite(v) & (np.abs(v) <= 448)]
    ours = nu.f32_to_e4m3(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_saturates_and_nan():
    v = np.float32([448.0, 449.0, 463.99, 464.0, 465.0, 1e30, np.inf, -500.0, -np.inf, np.nan])
    c = nu.f32_to_e4m3(v)
    assert list(c[:7]) == [0x7E] * 7
    assert c[7] == 0xFE and c[8] == 0xFE and c[9] == 0x7F


def test_e4m3_roundtrip_of_representables():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = nu.e4m3_decode(codes).astype(np.float32)
    back = nu.f32_to_e4m3(vals)
    assert np.array_equal(back, codes)


# ----------------------------------------------------------------------------- ue8m0

def test_ue8m0_closed_form():
    b = np.arange(256, dtype=np.uint8)
    d = nu.ue8m0_decode(b)
    assert np.isnan(d[255])
    for i in range(255):
        assert d[i] == math.ldexp(1.0, i - 127)
    assert d[127] == 1.0

"""Pins of the oracle's codecs against fixed facts, brute force and torch's own casts."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as fmt

E2M1_SET = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_value_set():
    # the fixed fact: E2M1 magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, code 8 = -0
    vals = fmt.e2m1_decode(np.arange(16))
    assert list(vals[:8]) == E2M1_SET
    assert list(-vals[8:]) == E2M1_SET
    assert np.signbit(vals[8])


def test_e2m1_round_trip_all_codes():
    codes = np.arange(16)
    v = fmt.e2m1_decode(codes).astype(np.float32)
    assert list(fmt.e2m1_round(v)) == list(codes)


def _brute_e2m1(v):
    """argmin |v - g| over the signed grid, ties to the even code, saturate."""
    v = float(v)
    sign = 8 if np.signbit(np.float32(v)) else 0
    a = min(abs(v), 6.0)
    best = None
    for c, g in enumerate(E2M1_SET):
        d = abs(Fraction(a) - Fraction(g))
        key = (d, c % 2)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1] | sign


def _ulp_neighbourhood(points, n):
    out = []
    for p in points:
        b = np.float32(p).view(np.uint32).astype(np.int64)
        ks = np.arange(-n, n + 1)
        bb = np.clip(b + ks, 0, 0x7F7FFFFF).astype(np.uint32)
        out.append(bb.view(np.float32))
    return np.concatenate(out)


def test_e2m1_rounding_brute_force():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] + E2M1_SET[1:]
    v = _ulp_neighbourhood(mids, 300)
    rng = np.random.default_rng(0)
    v = np.concatenate([v, rng.uniform(0, 8, 3000).astype(np.float32), np.float32([0.0, 7.0, 100.0, 1e30])])
    v = np.concatenate([v, -v])
    got = fmt.e2m1_round(v)
    want = np.array([_brute_e2m1(x) for x in v])
    assert np.array_equal(got, want)
    # signed zero: small negatives give -0 (code 8)
    assert fmt.e2m1_round(np.float32([-0.1]))[0] == 8
    assert fmt.e2m1_round(np.float32([-0.0]))[0] == 8


def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = fmt.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    fin = ~np.isnan(ref)
    assert np.array_equal(np.isnan(mine), ~fin)
    assert np.array_equal(mine[fin], ref[fin])
    assert mine[0x7E] == 448.0 and mine[1] == 2.0 ** -9


def test_e4m3_round_trip_all_finite_codes():
    codes = np.arange(127)
    v = fmt.e4m3_decode(codes)
    assert np.array_equal(fmt.e4m3_round_mag(v), codes)


def _brute_e4m3(u, grid):
    u = float(u)
    if u >= 448.0:
        return 126
    best = None
    for c, g in enumerate(grid):
        key = (abs(Fraction(u) - Fraction(float(g))), c % 2)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_e4m3_rounding_brute_force_and_torch():
    grid = fmt.e4m3_decode(np.arange(127))
    mids = list((grid[1:] + grid[:-1]) / 2) + list(grid)
    v = _ulp_neighbourhood(mids[::3], 6)
    rng = np.random.default_rng(1)
    v = np.concatenate([v, np.exp2(rng.uniform(-12, 9.2, 2000)).astype(np.float32), np.float32([0, 448, 449, 1e9])])
    v = np.abs(v)
    got = fmt.e4m3_round_mag(v.astype(np.float64))
    want = np.array([_brute_e4m3(x, grid) for x in v])
    assert np.array_equal(got, want)
    # torch's float32 -> float8_e4m3fn cast is round-to-nearest-even on the same grid
    small = v[v <= 448.0]
    t = torch.from_numpy(small.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fmt.e4m3_round_mag(small.astype(np.float64)), t.astype(np.int64))


def test_e8m0_decode_matches_torch():
    codes = np.arange(255, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).float().double().numpy()
    assert np.array_equal(fmt.e8m0_decode(codes), ref)


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        (rng.standard_normal(1000) * 1e-39).astype(np.float32),
                        np.float32([0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 3e38])])
    # exact ties
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(fmt.bf16_round(x), ref)
    assert np.array_equal(fmt.bf16_to_f32(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def _frac_to_bf16(x):
    fr = Fraction(float(x))
    if fr == 0:
        return 0.0
    a = abs(fr)
    E = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** E > a:
        E -= 1
    E = max(E, -126)
    ulp = Fraction(2) ** (E - 7)
    t = a / ulp
    lo = t.numerator // t.denominator
    rem = t - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return float(lo * ulp) * (1 if fr > 0 else -1)


def test_f64_to_bf16_exact_rational():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000),
                        [1.0 + 2 ** -8, 1.0 + 2 ** -8 + 2 ** -40, -(1.0 + 3 * 2 ** -8)]])
    got = fmt.bf16_to_f32(fmt.f64_to_bf16(x)).astype(np.float64)
    want = np.array([_frac_to_bf16(v) for v in x])
    assert np.array_equal(got, want)

"""Pins of the combine-path quantiser oracle (block Hadamard + 8-bit fixed-point MX).

Page: lhc.media page, paragraph on communication between GPUs (a Hadamard
transform before quantising the returning results, 8.25 bits per value instead
of 16).  The readings of the element format and of the transform are stated in
the oracle module's docstring; these tests pin them against closed forms, hand
derivations, brute force and invariants, never against the oracle itself.
"""
import fractions

import numpy as np
import pytest

from oracle import combine_q as cq
from oracle import formats as fmt
from oracle import layer as olayer


def test_payload_is_8p25_bits_per_value():
    # The page: sixteen bits per value fall to 8.25 (one byte per value plus one
    # scale byte per 32 values).
    for C in (32, 4096, 7168):
        assert cq.payload_bits_per_value(C) == 8.25


def test_hadamard_matrix_defining_properties():
    H = cq.hadamard_matrix(32)
    assert H.shape == (32, 32) and set(np.unique(H)) == {-1, 1}
    assert np.array_equal(H, H.T)
    assert np.array_equal(H @ H, 32 * np.eye(32, dtype=np.int64))
    # natural (Sylvester) order: H[i, j] = (-1)^popcount(i & j)
    ii, jj = np.meshgrid(np.arange(32), np.arange(32), indexing="ij")
    pop = np.vectorize(lambda v: bin(v).count("1"))(ii & jj)
    assert np.array_equal(H, np.where(pop % 2 == 0, 1, -1))


def test_fwht_matches_matrix_on_exact_inputs():
    # Small integers: every butterfly sum is exact in float32, so the transform
    # must equal the exact product with H written out entry by entry.
    rng = np.random.default_rng(3)
    x = rng.integers(-1000, 1000, size=(17, 96)).astype(np.float32)
    y = cq.fwht32_f32(x)
    for r in range(x.shape[0]):
        for b in range(3):
            blk = [int(v) for v in x[r, 32 * b:32 * b + 32]]
            want = [sum(blk[j] * (1 if bin(i & j).count("1") % 2 == 0 else -1) for j in range(32))
                    for i in range(32)]
            assert [int(v) for v in y[r, 32 * b:32 * b + 32]] == want
    # a unit impulse at position j gives column j of H (a sign or index slip fails)
    for j in (0, 1, 5, 31):
        e = np.zeros((1, 32), dtype=np.float32)
        e[0, j] = 1.0
        assert np.array_equal(cq.fwht32_f32(e)[0], cq.hadamard_matrix(32)[:, j].astype(np.float32))


def test_fwht_float32_within_rounding_bound():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((64, 64)) * np.exp(rng.uniform(-8, 8, (64, 64)))).astype(np.float32)
    y = cq.fwht32_f32(x).astype(np.float64)
    H = cq.hadamard_matrix(32).astype(np.float64)
    exact = (x.astype(np.float64).reshape(64, 2, 32) @ H).reshape(64, 64)
    # five rounded stages, each partial sum bounded by the block's sum of |x|
    l1 = np.abs(x.astype(np.float64)).reshape(64, 2, 32).sum(axis=2)
    bound = 5 * 2.0 ** -24 * np.repeat(l1, 32, axis=1)
    assert np.all(np.abs(y - exact) <= bound)


def test_fwht_rounds_stage_by_stage_hand_example():
    # x0 = 1, x1 = x2 = 2^-24.  Stage 1: 1 + 2^-24 is a tie between 1 and
    # 1 + 2^-23 and rounds to even (1); 2^-24 + 0 stays.  Stage 2: again
    # 1 + 2^-24 -> 1.  Later stages add zeros.  So y0 = 1 exactly, although the
    # exact sum 1 + 2^-23 is representable: the float32 stages decide it.
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 1.0
    x[0, 1] = x[0, 2] = 2.0 ** -24
    y = cq.fwht32_f32(x)
    assert y[0, 0] == np.float32(1.0)
    # y1 = (1 - 2^-24) + 2^-24 = 1 exactly; y3 = (1 - 2^-24) - 2^-24 = 1 - 2^-23
    assert y[0, 1] == np.float32(1.0)
    assert y[0, 3] == np.float32(1.0 - 2.0 ** -23)


def test_scale_exponent_closed_form():
    cases = {1.0: 0, 1.9999999: 0, 2.0: 1, 0.75: -1, 3.0: 1, 2.0 ** -126: -126, 2.0 ** -130: -127,
             0.0: -127, 2.0 ** 127: 127, 448.0: 8}
    for a, e in cases.items():
        assert int(cq.scale_exponent(np.array([a]))[0]) == e, a


def test_hand_derived_blocks():
    # x = e_0: H x = all ones -> amax 1, e = 0, every code 1 * 2^6 = 64, byte 127
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 1.0
    c, s = cq.quantize(x)
    assert np.all(c == 64) and s[0, 0] == 127
    # x = 3 e_0: amax 3, e = 1, codes 3 * 2^5 = 96, byte 128
    c, s = cq.quantize(3 * x)
    assert np.all(c == 96) and s[0, 0] == 128
    # x0 = x1 = 1: y_i = 1 + (-1)^i -> 2 (even i), 0 (odd i); e = 1, codes 64 / 0
    x2 = x.copy()
    x2[0, 1] = 1.0
    c, s = cq.quantize(x2)
    assert np.array_equal(c[0], np.array([64, 0] * 16, dtype=np.int8)) and s[0, 0] == 128
    # all three decode exactly back
    for v in (x, 3 * x, x2):
        assert np.array_equal(cq.dequantize(*cq.quantize(v)), v)
    # all-zero block: byte 0 (e = -127), codes 0, decode 0
    c, s = cq.quantize(np.zeros((2, 64), dtype=np.float32))
    assert np.all(c == 0) and np.all(s == 0)
    assert np.all(cq.dequantize(c, s) == 0)


def test_codes_are_nearest_grid_points_brute_force():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((40, 64)) * np.exp(rng.uniform(-20, 20, (40, 1)))).astype(np.float32)
    x[3, :32] = 0.0
    x[4, 5] = 1e6                      # an outlier block
    c, s = cq.quantize(x)
    y = cq.fwht32_f32(x).astype(np.float64)
    codes = np.arange(-127, 128)
    for r in range(x.shape[0]):
        for b in range(2):
            blk = y[r, 32 * b:32 * b + 32]
            amax = np.abs(blk).max()
            e = -127
            if amax > 0:  # largest e with 2^e <= amax, found by stepping
                e = 0
                while 2.0 ** e > amax:
                    e -= 1
                while 2.0 ** (e + 1) <= amax:
                    e += 1
                e = max(e, -127)
            assert s[r, b] == e + 127
            for i in range(32):
                w = fractions.Fraction(float(blk[i])) / fractions.Fraction(2) ** (e - 6)
                dist = [abs(w - int(k)) for k in codes]
                best = min(dist)
                cands = [int(k) for k, dd in zip(codes, dist) if dd == best]
                want = cands[0] if len(cands) == 1 else [k for k in cands if k % 2 == 0][0]
                assert int(c[r, 32 * b + i]) == want, (r, b, i)


def test_decode_exact_and_error_bound():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((64, 128)) * np.exp(rng.uniform(-4, 4, (64, 1)))).astype(np.float32)
    c, s = cq.quantize(x)
    xh = cq.dequantize(c, s).astype(np.float64)
    # exact decode, written with fractions: H c 2^(e-11)
    H = cq.hadamard_matrix(32)
    for r in (0, 17, 63):
        for b in (0, 3):
            e = int(s[r, b]) - 127
            ci = [int(v) for v in c[r, 32 * b:32 * b + 32]]
            for i in range(32):
                v = fractions.Fraction(sum(int(H[i, j]) * ci[j] for j in range(32))) * fractions.Fraction(2) ** (e - 11)
                assert fractions.Fraction(float(xh[r, 32 * b + i])) == v
    # error: in the transformed domain each code is within one step 2^(e-6)
    # (half a step unless clamped), so a block's error has norm <= sqrt(32)
    # steps; the decode divides by 32 after H, whose norm is sqrt(32), so the
    # block's error norm in the original domain is <= one step, plus the
    # float32 rounding of the sender's transform (<= 5 * 2^-24 * sum |x| per
    # value in the transformed domain, carried over the same way).
    e = s.astype(np.int64) - 127
    err = (xh - x.astype(np.float64)).reshape(64, 4, 32)
    step = np.ldexp(1.0, e - 6)
    l1 = np.abs(x.astype(np.float64)).reshape(64, 4, 32).sum(axis=2)
    bound = step + 5 * 2.0 ** -24 * l1
    assert np.all(np.sqrt((err ** 2).sum(axis=2)) <= bound * (1 + 1e-12))


def test_hadamard_spreads_an_outlier():
    # The page's stated purpose: the transform spreads extreme values before the
    # quantisation.  A block of N(0,1) values with one value x1000 loses its
    # small values when quantised directly (the outlier sets the scale and they
    # round to zero); with the transform first the error, spread evenly over
    # the block, is markedly smaller (about 0.6 of it here).
    rng = np.random.default_rng(7)
    x = rng.standard_normal((256, 32)).astype(np.float32)
    x[:, 7] *= 1000.0

    def direct(v):  # the same 8-bit MX format without the transform
        v64 = v.astype(np.float64)
        e = cq.scale_exponent(np.abs(v64).max(axis=1))
        cc = np.clip(np.rint(np.ldexp(v64, (6 - e)[:, None])), -127, 127)
        return np.ldexp(cc, (e - 6)[:, None])

    err_direct = np.sqrt(((direct(x) - x) ** 2).mean())
    err_h = np.sqrt(((cq.dequantize(*cq.quantize(x)).astype(np.float64) - x) ** 2).mean())
    assert err_h < 0.7 * err_direct


def test_combine_payload_is_combine_of_decoded_rows():
    rng = np.random.default_rng(8)
    T, k, d = 9, 3, 64
    Yp = rng.standard_normal((T * k, d)).astype(np.float32)
    gates = rng.uniform(0, 1, (T, k)).astype(np.float32)
    inv = rng.permutation(T * k).astype(np.int32)
    c, s = cq.quantize(Yp)
    y = cq.combine_payload(c, s, gates, inv, k)
    # written out: slot order, float32 product then float32 sum, bf16 at the end
    Yh = cq.dequantize(c, s)
    want = np.zeros((T, d), dtype=np.float32)
    for t in range(T):
        acc = np.zeros(d, dtype=np.float32)
        for j in range(k):
            acc = acc + gates[t, j] * Yh[inv[t * k + j]]
        want[t] = acc
    assert np.array_equal(y, fmt.bf16_round(want))
    assert np.array_equal(olayer.combine(Yh, gates, inv, k), y)

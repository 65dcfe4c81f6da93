"""Pins of the NVFP4 / Four-Over-Six oracle: closed forms, invariants and brute force."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as fmt
from oracle import nvfp4 as nv

E2M1_SET = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _rand(shape, seed, outliers=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32)
    if outliers:
        m = rng.random(shape) < 0.01
        x[m] *= 30
    return x


def test_bits_per_value_is_4_5():
    # lhc.media page: 4-bit values plus one scale per sixteen values, 4.5 bits per value
    R, C = 64, 256
    q = nv.nvfp4_quantize(_rand((R, C), 0), nv.MODE_46)
    nbytes = q["codes"].nbytes + q["sf"].nbytes
    assert nbytes * 8 / (R * C) == 4.5
    assert nbytes == 9 * R * C // 16


def test_tensor_scale_closed_form():
    x = _rand((32, 64), 1)
    amax = np.float32(np.abs(x).max())
    assert nv.tensor_scale(x, nv.MODE_46) == np.float32(amax / np.float32(1792.0))
    assert nv.tensor_scale(x, nv.MODE_6) == np.float32(amax / np.float32(2688.0))


@pytest.mark.parametrize("mode", [nv.MODE_6, nv.MODE_46])
def test_power_of_two_equivariance(mode):
    x = _rand((48, 128), 2)
    base = nv.nvfp4_quantize(x, mode)
    for j in (-20, -3, 1, 7, 30):
        y = (x * np.float32(2.0 ** j)).astype(np.float32)
        q = nv.nvfp4_quantize(y, mode)
        assert np.array_equal(q["codes"], base["codes"])
        assert np.array_equal(q["sf"], base["sf"])
        assert q["ts"][0] == np.float32(base["ts"][0] * np.float32(2.0 ** j))


def test_amax_block_scale_is_448():
    # the block holding the tensor amax: u_4 = amax / (4 * amax / 1792) = 448 (4/6 mode)
    # and u_6 = amax / (6 * amax / 2688) = 448 (mode 6)
    x = _rand((16, 64), 3)
    r, c = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    S46 = nv.tensor_scale(x, nv.MODE_46)
    blk = x[r, (c // 16) * 16:(c // 16 + 1) * 16][None, :]
    _, sc4, _ = nv._encode_candidate(blk, np.float32([S46]), 4)
    assert sc4[0] == 126
    S6 = nv.tensor_scale(x, nv.MODE_6)
    _, sc6, _ = nv._encode_candidate(blk, np.float32([S6]), 6)
    assert sc6[0] == 126


def test_zero_group():
    x = np.zeros((4, 32), dtype=np.float32)
    x[1, 3] = -0.0
    q = nv.nvfp4_quantize(x, nv.MODE_46)
    assert q["ts"][0] == 1.0
    assert not q["sf"].any()
    codes = nv.unpack_codes(q["codes"])
    assert codes[1, 3] == 8 and codes.sum() == 8
    # per-group: an all-zero group next to a normal one
    y = np.concatenate([_rand((4, 32), 4), np.zeros((3, 32), np.float32)])
    qg = nv.nvfp4_quantize(y, nv.MODE_46, [0, 4, 7])
    assert qg["ts"][1] == 1.0 and not qg["sf"][4:].any()
    assert qg["ts"][0] == nv.tensor_scale(y[:4], nv.MODE_46)


def _exact_sq_err(xb, q, sc, S):
    tot = Fraction(0)
    for i in range(16):
        v = Fraction(float(xb[i])) - Fraction(float(fmt.e2m1_decode(q[i]))) * Fraction(float(fmt.e4m3_decode(sc))) * Fraction(float(S))
        tot += v * v
    return tot


def test_four_over_six_choice_exact_rational():
    """The stored candidate has the lower exact squared error, except near-ties
    that the float32 error sums cannot resolve (|e4-e6| <= 2**-18 (e4+e6))."""
    rng = np.random.default_rng(5)
    nblk = 3000
    x = rng.standard_normal((nblk, 16)).astype(np.float32) * np.exp2(rng.integers(-3, 4, (nblk, 1))).astype(np.float32)
    S = nv.tensor_scale(x, nv.MODE_46)
    Sv = np.full(nblk, S, np.float32)
    q6, sc6, _ = nv._encode_candidate(x, Sv, 6)
    q4, sc4, _ = nv._encode_candidate(x, Sv, 4)
    q, sc, m = nv.quantize_blocks(x.reshape(nblk, 16), np.full(nblk, S, np.float32), nv.MODE_46)
    n4 = 0
    close = 0
    for b in range(nblk):
        e6 = _exact_sq_err(x[b], q6[b], sc6[b], S)
        e4 = _exact_sq_err(x[b], q4[b], sc4[b], S)
        if abs(e4 - e6) <= Fraction(1, 1 << 18) * (e4 + e6):
            close += 1
            continue
        want4 = e4 < e6
        assert (m[b, 0] == 4) == want4, b
        n4 += want4
    assert 0.1 * nblk < n4 < 0.9 * nblk       # both candidates get chosen
    assert close < nblk // 50


def test_candidate_codes_are_nearest_grid_points():
    """Each code is the nearest E2M1 point to x / eff (brute force), up to the one
    rounding of the reciprocal: checked exactly whenever the margin exceeds 2**-20."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((500, 16)).astype(np.float32)
    S = nv.tensor_scale(x, nv.MODE_46)
    for m in (6, 4):
        q, sc, _ = nv._encode_candidate(x, np.full(500, S, np.float32), m)
        for b in range(0, 500, 7):
            effb = Fraction(float(fmt.e4m3_decode(sc[b]))) * Fraction(float(S))
            for i in range(16):
                t = Fraction(float(x[b, i])) / effb
                a = min(abs(t), Fraction(6))
                d = sorted((abs(a - Fraction(g)), c) for c, g in enumerate(E2M1_SET))
                if d[1][0] - d[0][0] <= Fraction(1, 1 << 20) * max(a, Fraction(1)):
                    continue
                assert (q[b, i] & 7) == d[0][1]


def test_scale_is_rne_of_amax_over_m_s():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((400, 16)).astype(np.float32)
    S = nv.tensor_scale(x, nv.MODE_46)
    for m in (4, 6):
        _, sc, _ = nv._encode_candidate(x, np.full(400, S, np.float32), m)
        grid = fmt.e4m3_decode(np.arange(127))
        for b in range(400):
            u = Fraction(float(np.float32(np.abs(x[b]).max() / np.float32(np.float32(m) * S))))
            d = sorted((abs(u - Fraction(float(g))), c % 2, c) for c, g in enumerate(grid))
            assert sc[b] == d[0][2]


def test_dequant_exact_and_fixed_scale_reencode():
    x = _rand((32, 128), 8)
    q = nv.nvfp4_quantize(x, nv.MODE_46)
    deq = nv.nvfp4_dequantize(q["codes"], q["sf"], q["ts"])
    codes = nv.unpack_codes(q["codes"])
    sc = np.repeat(q["sf"].astype(np.int64), 16, axis=1)
    S = q["ts"][0]
    # deq is the real q * sc * S rounded once to float32
    for r in range(0, 32, 5):
        for c in range(0, 128, 3):
            exact = Fraction(float(fmt.e2m1_decode(codes[r, c]))) * Fraction(float(fmt.e4m3_decode(sc[r, c]))) * Fraction(float(S))
            # q * sc * S has at most 30 significant bits, so float(exact) is exact and
            # np.float32 of it is the one correct rounding
            assert Fraction(float(deq[r, c])) == Fraction(float(np.float32(float(exact))))
    # re-encoding the dequantised values under the same block scales gives the same codes
    eff = (fmt.e4m3_decode(sc).astype(np.float32) * S).astype(np.float32)
    inv = np.where(eff > 0, np.float32(1.0) / np.where(eff > 0, eff, 1), 0).astype(np.float32)
    re = fmt.e2m1_round((deq * inv).astype(np.float32))
    nz = eff > 0
    assert np.array_equal(re[nz] & 7, codes[nz] & 7)


def test_mode6_never_uses_four():
    q = nv.nvfp4_quantize(_rand((8, 64), 9), nv.MODE_6)
    assert (q["choice"] == 6).all()


def test_bf16_input_equals_its_float32_value():
    import torch
    x = _rand((8, 64), 10)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    a = nv.nvfp4_quantize(bits, nv.MODE_46)
    b = nv.nvfp4_quantize(fmt.bf16_to_f32(bits), nv.MODE_46)
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["sf"], b["sf"])


@pytest.mark.parametrize("mode", [nv.MODE_6, nv.MODE_46])
def test_infinite_reciprocal_keeps_zero_signs(mode):
    """A group of float32 subnormals (about 2^-130): S = fl(amax / (m_max 448))
    is subnormal, eff = fl(dec(sc) S) falls below 2^-128 and fl(1 / eff)
    overflows.  By the definition every nonzero element then saturates to +-6
    (codes 7 / 15) and every zero element keeps its own sign (codes 0 / 8),
    whatever sign the platform gives the NaN of 0 * inf."""
    t = np.float32(2.0 ** -130)
    x = np.array([[t, -t / 2, 0.0, -0.0, 3 * t / 8, -5 * t / 8, 0.0, t / 4,
                   -0.0, t / 2, -t, 0.0, t / 8, -t / 8, -0.0, 7 * t / 8]], dtype=np.float32)
    assert np.signbit(x[0, 3]) and not np.signbit(x[0, 2])
    q = nv.nvfp4_quantize(x, mode)
    S = np.float32(q["ts"][0])
    assert 0 < S < np.float32(2.0 ** -126)                     # subnormal tensor scale
    sc = int(q["sf"][0, 0])
    eff = np.float32(fmt.e4m3_decode(np.array([sc]))[0]) * S
    with np.errstate(over="ignore", divide="ignore"):
        assert np.isinf(np.float32(1.0) / eff)
    want = np.where(x[0] == 0, np.where(np.signbit(x[0]), 8, 0), np.where(x[0] < 0, 15, 7))
    assert np.array_equal(nv.unpack_codes(q["codes"])[0], want)

"""Pins of the MXFP8 oracle: MX scale rule, RNE, exact SR probability, SR
unbiasedness, transposed group layout and the requantisation."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as fmt
from oracle import mxfp8 as mx
from oracle import nvfp4 as nv
from oracle import srhash

GRID = fmt.e4m3_decode(np.arange(127))          # non-negative finite E4M3 values


def test_mx_scale_least_exponent_brute_force():
    vals = []
    for E in range(-140, 128):
        for f in (1.0, 1.75, 2.0):
            b = np.float32(f * 2.0 ** E) if -149 <= E + np.log2(f) < 128 else None
            if b is None or not np.isfinite(b) or b == 0:
                continue
            bb = np.float32(b).view(np.uint32).astype(np.int64)
            for k in (-2, -1, 0, 1, 2):
                v = np.uint32(np.clip(bb + k, 1, 0x7F7FFFFF)).view(np.float32)
                vals.append(float(v))
    vals = np.array(vals + [0.0])
    got = mx.mx_scale_exponent(vals)
    for a, e in zip(vals, got):
        if a == 0:
            assert e == -127
            continue
        want = next(t for t in range(-300, 300) if Fraction(a) <= 448 * Fraction(2) ** t)
        assert e == max(-127, min(127, want)), a


def _brute_rne(w):
    s = 0x80 if np.signbit(w) else 0
    a = abs(float(w))
    best = min(((abs(Fraction(a) - Fraction(float(g))), c % 2, c) for c, g in enumerate(GRID)))
    return best[2] | s


def test_rne_codes_brute_force_and_torch():
    rng = np.random.default_rng(0)
    v = (rng.standard_normal((40, 32)) * np.exp2(rng.integers(-20, 20, (40, 1)))).astype(np.float32)
    codes, sf = mx.quantize_blocks_rows(v, mx.RNE)
    e = sf.astype(np.int64) - 127
    w = v.astype(np.float64) * np.exp2(-e)[:, None]
    assert np.abs(w).max() <= 448.0
    for b in range(40):
        for i in range(0, 32, 3):
            assert codes[b, i] == _brute_rne(w[b, i])
    # torch's cast of the exactly scaled float32 values agrees
    t = torch.from_numpy(w.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(t, codes)


def _sr_neighbours(a):
    """Largest grid value <= a and the next grid value (brute force over the grid)."""
    lo = max(float(g) for g in GRID if g <= a)
    his = [float(g) for g in GRID if g > lo]
    return lo, (min(his) if his else lo)


@pytest.mark.parametrize("w", [1.0 + 2 ** -20, 1.3, 7.77, 300.1, 447.9, 0.0005, 0.0123, 2 ** -6 + 2 ** -30, 5e-7, 260.0])
def test_sr_exact_probability(w):
    w = float(np.float32(w))
    lo, hi = _sr_neighbours(w)
    step = Fraction(hi) - Fraction(lo)
    frac = (Fraction(w) - Fraction(lo)) / step
    F = (frac * 65536).numerator // (frac * 65536).denominator
    r = np.arange(65536)
    codes = mx.round_sr(np.full(65536, w), r)
    vals = fmt.e4m3_decode(codes)
    assert set(np.unique(vals)) <= {lo, hi}
    assert int((vals == hi).sum()) == (F if hi != lo else 0)
    # negative values mirror
    neg = fmt.e4m3_decode(mx.round_sr(np.full(65536, -w), r))
    assert np.array_equal(neg, -vals)


def test_sr_grid_values_never_move():
    r = np.arange(0, 65536, 97)
    for g in GRID:
        codes = mx.round_sr(np.full(r.shape, g), r)
        assert (fmt.e4m3_decode(codes) == g).all()


def test_sr_unbiased_over_seeds():
    # lhc.media page: stochastic rounding keeps the value on average
    n = 30000
    # one fixed element index, n different seeds
    rs = np.array([srhash.random16(s, 0, np.array([12345], np.uint64))[0] for s in range(1, n + 1)])
    for w in (1.3, 0.0123, 100.7, 2 ** -8 + 2 ** -12, 6.0625):
        w = float(np.float32(w))
        vals = fmt.e4m3_decode(mx.round_sr(np.full(n, w), rs))
        lo, hi = _sr_neighbours(w)
        f = (w - lo) / (hi - lo)
        sigma = (hi - lo) * np.sqrt(f * (1 - f) / n) + 1e-30
        assert abs(vals.mean() - w) <= 5 * sigma + (hi - lo) * 2 ** -16


def test_rne_requant_bias_vs_sr():
    """lhc.media page: requantising with a rounding that always favours one
    direction biases values; stochastic rounding removes the bias on average."""
    rng = np.random.default_rng(3)
    v = (1.0 + rng.random(32 * 512) * 0.06).astype(np.float32).reshape(-1, 32)   # just above 1: RNE rounds all to 1
    exact = v.astype(np.float64).mean()
    c_rne, s_rne = mx.quantize_blocks_rows(v, mx.RNE)
    d_rne = (fmt.e4m3_decode(c_rne) * fmt.e8m0_decode(s_rne)[:, None]).mean()
    idx = np.arange(v.size, dtype=np.uint64).reshape(v.shape)
    d_sr = []
    for seed in range(1, 65):
        c, s = mx.quantize_blocks_rows(v, mx.SR, seed, 0, idx)
        d_sr.append((fmt.e4m3_decode(c) * fmt.e8m0_decode(s)[:, None]).mean())
    assert abs(d_rne - exact) > 0.02 * exact / 2
    assert abs(np.mean(d_sr) - exact) < 1e-4


def test_mx_dequant_idempotent_rne():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((16, 96)) * 3).astype(np.float32)
    c1, s1 = mx.quantize_rowwise(x)
    d1 = mx.dequant_rowwise(c1, s1).astype(np.float32)
    c2, s2 = mx.quantize_rowwise(d1)
    assert np.array_equal(mx.dequant_rowwise(c2, s2), mx.dequant_rowwise(c1, s1))


def test_transposed_layout_exact_values():
    """Values that are exact in MXFP8 survive a transposed grouped quantisation
    unchanged (RNE and SR alike), which pins the layout, padding and grouping."""
    rng = np.random.default_rng(5)
    R, C = 150, 64
    off = np.array([0, 3, 3, 40, 72, 150])          # includes an empty group and ragged tails
    # values k * 2**-3 with |k| < 16 are E4M3-exact under any block scale <= the amax's
    x = (rng.integers(-15, 16, (R, C)) * 0.125).astype(np.float32)
    for rnd, lay in ((mx.RNE, mx.SF_ROWS), (mx.SR, mx.SF_ROWS), (mx.RNE, mx.SF_BLOCKS)):
        codes, sf = mx.quantize_transposed(x, off, rnd, seed=1, stream_id=2, sf_layout=lay)
        blocks = mx.dequant_transposed(codes, sf, off, C, lay)
        offp = mx.padded_offsets(off)
        assert len(codes) == C * offp[-1]
        for g in range(len(off) - 1):
            Rg = off[g + 1] - off[g]
            assert blocks[g].shape == (C, mx.pad32(Rg))
            assert np.array_equal(blocks[g][:, :Rg], x[off[g]:off[g + 1]].T.astype(np.float64))
            assert not blocks[g][:, Rg:].any()


@pytest.mark.parametrize("sf_layout", [mx.SF_ROWS, mx.SF_BLOCKS])
def test_transposed_scale_positions(sf_layout):
    """Each (column, 32-row block) of a group gets a planted amax of
    448 * 2**k, whose scale byte must be k + 127 (the least exponent with
    amax <= 448 * 2**e), at the position the layout names: row-major
    [C][P/32] or block-major [P/32][C], after the group's C * off_pad / 32."""
    rng = np.random.default_rng(9)
    R, C = 130, 96
    off = np.array([0, 40, 40, 130])                # an empty group, ragged tails
    offp = mx.padded_offsets(off)
    x = (rng.uniform(-1.0, 1.0, (R, C)) * 2.0 ** -8).astype(np.float32)
    want = {}
    for g in range(len(off) - 1):
        for b in range((off[g + 1] - off[g] + 31) // 32):
            rows = np.arange(off[g] + 32 * b, min(off[g] + 32 * b + 32, off[g + 1]))
            for c in range(C):
                k = (c + 3 * b + g) % 7 - 3
                x[rows[(c + b) % len(rows)], c] = np.float32(448.0 * 2.0 ** k) * (1 if c % 2 else -1)
                want[(g, b, c)] = k + 127
    _, sf = mx.quantize_transposed(x, off, mx.RNE, sf_layout=sf_layout)
    assert len(sf) == C * offp[-1] // 32
    for (g, b, c), byte in want.items():
        nb = (offp[g + 1] - offp[g]) // 32
        pos = C * offp[g] // 32 + (c * nb + b if sf_layout == mx.SF_ROWS else b * C + c)
        assert sf[pos] == byte, (g, b, c)


def test_requant_sr_t_exact_grid_and_unbiased():
    rng = np.random.default_rng(6)
    R, C = 64, 96
    x = rng.standard_normal((R, C)).astype(np.float32)
    q = nv.nvfp4_quantize(x, nv.MODE_46)
    deq = nv.nvfp4_dequantize(q["codes"], q["sf"], q["ts"]).astype(np.float64)
    acc = np.zeros((C, R))
    n = 64
    for seed in range(1, n + 1):
        codes, sf = mx.requant_sr_t(q["codes"], q["sf"], q["ts"], None, True, seed, 0)
        acc += mx.dequant_transposed(codes, sf, [0, R], C)[0]
    err = acc / n - deq.T
    # per element the SR error has std <= step/2; the mean of n draws: step/(2 sqrt n)
    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(deq.T), 2.0 ** -140))) - 3)
    assert (np.abs(err) <= 6 * step / (2 * np.sqrt(n)) + 1e-30).all()
    # "does not recover all the information lost": the mean tends to deq(Q(x)), not x
    assert np.abs(acc / n - x.T).mean() > 3 * np.abs(err).mean()


def test_wgrad_unbiased_over_seeds():
    """E[dU_col^T . X_T] over SR seeds equals the product with the exact
    dequantised X (linearity): pins requant_sr_t inside a wgrad."""
    rng = np.random.default_rng(7)
    M, d, F = 40, 64, 32
    x = rng.standard_normal((M, d)).astype(np.float32)
    q = nv.nvfp4_quantize(x, nv.MODE_46)
    dU = rng.standard_normal((M, F)).astype(np.float32)
    off = np.array([0, M])
    uc, us = mx.quantize_transposed(dU, off, mx.RNE)
    U = mx.dequant_transposed(uc, us, off, F)[0]               # [F, 64]
    exact = U @ np.pad(nv.nvfp4_dequantize(q["codes"], q["sf"], q["ts"]).astype(np.float64), ((0, 24), (0, 0)))
    n = 128
    acc = np.zeros((F, d))
    for seed in range(1, n + 1):
        c, s = mx.requant_sr_t(q["codes"], q["sf"], q["ts"], off, False, seed, 0)
        acc += U @ mx.dequant_transposed(c, s, off, d)[0].T
    rel = np.linalg.norm(acc / n - exact) / np.linalg.norm(exact)
    one = np.linalg.norm(U @ mx.dequant_transposed(*mx.requant_sr_t(q["codes"], q["sf"], q["ts"], off, False, 1, 0), off, d)[0].T - exact) / np.linalg.norm(exact)
    assert rel < one / 4          # averaging 128 draws shrinks the error ~ sqrt(128) ~ 11x


def test_requant_mx_exact_values_and_unbiased():
    """MXFP8 -> transpose -> MXFP8 SR: values that are exact in both blockings
    pass unchanged; in general the requantisation is unbiased over seeds."""
    rng = np.random.default_rng(21)
    R, C = 96, 64
    off = np.array([0, 40, 96])
    x = (rng.integers(-15, 16, (R, C)) * 0.125).astype(np.float32)
    c, s = mx.quantize_rowwise(x, mx.RNE)                     # exact: k / 8 with |k| < 16
    assert np.array_equal(mx.dequant_rowwise(c, s), x.astype(np.float64))
    for lay in (mx.SF_ROWS, mx.SF_BLOCKS):
        tc, ts_ = mx.requant_mx_sr_t(c, s, off, seed=3, stream_id=1, sf_layout=lay)
        blocks = mx.dequant_transposed(tc, ts_, off, C, lay)
        for g in range(2):
            assert np.array_equal(blocks[g][:, :off[g + 1] - off[g]], x[off[g]:off[g + 1]].T.astype(np.float64))
    y = (rng.standard_normal((64, 32)) * np.exp2(rng.integers(-6, 6, (64, 1)))).astype(np.float32)
    c, s = mx.quantize_rowwise(y, mx.RNE)
    v = mx.dequant_rowwise(c, s)
    acc = np.zeros((32, 64))
    n = 400
    for seed in range(n):
        tc, ts_ = mx.requant_mx_sr_t(c, s, None, seed=seed, stream_id=0)
        acc += mx.dequant_transposed(tc, ts_, [0, 64], 32)[0]
    err = np.abs(acc / n - v.T)
    # each SR step is at most one E4M3 grid step of its block: the mean converges
    step = np.abs(v.T).max(axis=1, keepdims=True) * 2.0 ** -3
    assert np.all(err <= 4 * step / np.sqrt(n) + 1e-30)

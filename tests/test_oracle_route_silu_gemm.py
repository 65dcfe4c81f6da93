"""Pins of the routing, SiLU and GEMM oracles."""
import decimal
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as fmt
from oracle import gemm
from oracle import mxfp8 as mx
from oracle import nvfp4 as nv
from oracle import route
from oracle import silu


# ---------------------------------------------------------------- routing

def test_topk_invariants_and_tie_rule():
    rng = np.random.default_rng(0)
    T, E, k = 200, 24, 5
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:20] = np.round(logits[:20])              # many exact ties
    bias = (-1.1 * np.log(np.arange(E) + 1)).astype(np.float32)
    idx, gates = route.topk_gates(logits, k, bias)
    z = (logits + bias).astype(np.float32)
    for t in range(T):
        sel = list(idx[t])
        assert len(set(sel)) == k
        rest = [e for e in range(E) if e not in sel]
        # every selected value beats every unselected one; equal values -> lower index first
        for s in sel:
            for r in rest:
                assert z[t, s] > z[t, r] or (z[t, s] == z[t, r] and s < r)
        for a, b in zip(sel, sel[1:]):
            assert z[t, a] > z[t, b] or (z[t, a] == z[t, b] and a < b)
    # library routine: a stable sort of -z lists the same experts
    ref = np.argsort(-z, axis=1, kind="stable")[:, :k]
    assert np.array_equal(ref, idx)


def test_topk_all_ties():
    idx, gates = route.topk_gates(np.zeros((3, 10), np.float32), 4)
    assert (idx == np.arange(4)).all()
    assert (gates == np.float32(0.25)).all()


def test_gates_are_renormalised_softmax():
    rng = np.random.default_rng(1)
    logits = (rng.standard_normal((300, 16)) * 3).astype(np.float32)
    idx, gates = route.topk_gates(logits, 4)
    for t in range(300):
        z = logits[t, idx[t]].astype(np.float64)
        p = np.exp(z - z.max())
        p /= p.sum()
        assert np.allclose(gates[t], p, rtol=4e-7, atol=0)
        assert abs(float(gates[t].astype(np.float64).sum()) - 1.0) <= 4 * 2 ** -24
        assert (np.diff(gates[t]) <= 0).all()


def test_permutation_matches_stable_argsort():
    rng = np.random.default_rng(2)
    T, E, k = 300, 12, 3
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    idx[:, 0] = np.where(rng.random(T) < 0.5, 0, idx[:, 0])   # skew
    P = route.permutation(idx, E)
    flat = idx.reshape(-1)
    assert np.array_equal(P["perm"], np.argsort(flat, kind="stable"))
    assert np.array_equal(P["off"], np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert np.array_equal(P["inv_perm"][P["perm"]], np.arange(T * k))
    cnt = np.bincount(flat, minlength=E)
    assert np.array_equal(np.diff(P["off_pad"]), (cnt + 31) // 32 * 32)


# ---------------------------------------------------------------- SiLU tables

def test_silu_closed_forms():
    bits, s, d = silu.tables()
    u = fmt.bf16_to_f32(bits)
    assert s[u == 0].max() == 0 and d[u == 0].min() == 0.5
    big = u >= 100
    assert np.array_equal(s[big], u[big])            # silu(u) -> u
    neg = u <= -200
    assert (s[neg] == 0).all() and np.signbit(s[neg]).all()   # -> -0
    # silu(u) = u * sigma(u) is odd-symmetric up to u: silu(u) - silu(-u) = u
    pos = (u > 0) & (u < 20)
    ub = bits[pos]
    s_neg = silu.silu_f32(ub | np.uint16(0x8000)).astype(np.float64)
    assert np.allclose(s[pos].astype(np.float64) - s_neg, u[pos], rtol=2e-7, atol=1e-30)


def test_silu_tables_against_decimal():
    bits, s, d = silu.tables()
    u = fmt.bf16_to_f32(bits)
    rng = np.random.default_rng(3)
    ok = np.nonzero(np.abs(u) < 4000)[0]         # beyond, exp overflows Decimal's range (closed forms cover it)
    pick = rng.choice(ok, 1500, replace=False)
    with decimal.localcontext() as ctx:
        ctx.prec = 50
        for i in pick:
            x = decimal.Decimal(float(u[i]))
            sig = 1 / (1 + (-x).exp())
            want_s = silu._dec_to_f32(x * sig)
            want_d = silu._dec_to_f32(sig * (1 + x * (1 - sig)))
            assert s[i] == want_s and d[i] == want_d, float(u[i])


def test_silu_certificate_count():
    bits, s, d = silu.tables()
    u = fmt.bf16_to_f32(bits).astype(np.float64)
    # the float64 evaluation is certified (margin > 1e-13) everywhere except at tiny
    # |u| < 2**-8, where u/2 + u**2/4 (silu) and 1/2 + u/2 (silu') land on or next to
    # float32 rounding midpoints; those entries come from the Decimal evaluation
    for f in (silu._silu_f64, silu._dsilu_f64):
        bad = silu._boundary_distance(f(u)) < silu._MARGIN
        assert bad.sum() < 400
        assert (np.abs(u[bad]) < 2.0 ** -8).all()


# ---------------------------------------------------------------- GEMMs

def test_grouped_gemm_exact_rational_tiny():
    rng = np.random.default_rng(4)
    E, N, K = 3, 5, 32
    off = np.array([0, 2, 2, 7])
    x = rng.standard_normal((7, K)).astype(np.float32)
    w = rng.standard_normal((E * N, K)).astype(np.float32)
    qa = nv.nvfp4_quantize(x, nv.MODE_46)
    qb = nv.nvfp4_quantize(w, nv.MODE_6, np.arange(E + 1) * N)
    A = nv.nvfp4_exact_f64(qa["codes"], qa["sf"], qa["ts"])
    B = nv.nvfp4_exact_f64(qb["codes"], qb["sf"], qb["ts"], np.arange(E + 1) * N).reshape(E, N, K)
    C = gemm.grouped_nt(A, B, off)
    for e in range(E):
        for m in range(off[e], off[e + 1]):
            for n in range(N):
                terms = [Fraction(float(A[m, kk])) * Fraction(float(B[e, n, kk])) for kk in range(K)]
                exact = sum(terms)
                # float64 summation: |error| <= K * 2**-53 * sum |a*b|
                bound = K * Fraction(1, 1 << 53) * sum(abs(t) for t in terms)
                assert abs(Fraction(float(C[m, n])) - exact) <= bound


def test_wgrad_shapes_and_empty_expert():
    rng = np.random.default_rng(5)
    A = [rng.standard_normal((4, 32)), np.zeros((4, 0)), rng.standard_normal((4, 64))]
    B = [rng.standard_normal((3, 32)), np.zeros((3, 0)), rng.standard_normal((3, 64))]
    dw = gemm.wgrad(A, B)
    assert dw.shape == (3, 4, 3) and not dw[1].any()
    assert np.allclose(dw[2], A[2] @ B[2].T)


def test_route_backward_matches_finite_differences():
    """The router backward against central differences of a float64 softmax
    over the selected experts (the function whose derivative it is), with
    the loss L = sum_j dg_j * g_j(z)."""
    rng = np.random.default_rng(12)
    T, E, k = 20, 9, 4
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, gates = route.topk_gates(logits, k)
    dg = rng.standard_normal((T, k)).astype(np.float32)
    dz = route.route_backward(dg, gates, idx, E)
    h = 1e-6
    for t in range(T):
        sel = idx[t].astype(np.int64)
        zt = logits[t].astype(np.float64)

        def loss(z):
            w = np.exp(z[sel] - z[sel].max())
            return float(np.dot(dg[t].astype(np.float64), w / w.sum()))
        for e in range(E):
            zp, zm = zt.copy(), zt.copy()
            zp[e] += h
            zm[e] -= h
            fd = (loss(zp) - loss(zm)) / (2 * h)
            # float32 gates and sums: agreement to a few float32 ulps of the terms
            assert abs(dz[t, e] - fd) <= 1e-5 * (1 + np.abs(dg[t]).sum()), (t, e, dz[t, e], fd)
        assert not dz[t][np.setdiff1d(np.arange(E), sel)].any()       # unselected experts: exactly 0


def test_route_backward_shift_invariance_and_k1():
    """Softmax gradients sum to zero over the selected set (up to float32
    rounding); with k = 1 the single gate is 1 and its gradient is exactly 0."""
    rng = np.random.default_rng(13)
    logits = rng.standard_normal((30, 12)).astype(np.float32)
    idx, gates = route.topk_gates(logits, 5)
    dg = rng.standard_normal((30, 5)).astype(np.float32)
    dz = route.route_backward(dg, gates, idx, 12)
    assert np.all(np.abs(dz.sum(axis=1)) <= 1e-5 * (1 + np.abs(dg).sum(axis=1)))
    idx1, g1 = route.topk_gates(logits, 1)
    assert np.all(g1 == 1.0)
    assert not route.route_backward(dg[:, :1], g1, idx1, 12).any()


def test_silu_piecewise_monotone_over_bf16():
    """The NVFP4 quantiser's SiLU amax takes max |silu| over a group from three
    extremes of the bf16 inputs.  That rests on a property of the correctly
    rounded silu, checked here over every finite bf16 value: silu is
    non-decreasing on [0, inf); below zero, |silu| is non-increasing in |u| for
    u <= -1.28125 (bf16 0xBFA4) and non-decreasing in |u| for
    -1.2734375 (0xBFA3) <= u < 0, and those two ranges hold every negative."""
    from oracle import silu as osl
    bits = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    s = osl.silu_f32(bits).astype(np.float64)
    mag = (bits & 0x7FFF).astype(np.int64)
    fin = mag < 0x7F80
    pos = (bits < 0x8000) & fin
    neg = (bits >= 0x8000) & fin
    lo = neg & (mag >= 0x3FA4)
    hi = neg & (mag <= 0x3FA3)
    assert not np.any(lo & hi) and np.array_equal(lo | hi, neg)
    for sel, sign in ((pos, 1), (lo, -1), (hi, 1)):
        o = np.argsort(mag[sel], kind="stable")
        a = np.abs(s[sel][o])
        assert np.all(sign * np.diff(a) >= 0)

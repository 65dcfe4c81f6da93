"""Pins of the router oracle (oracle/router.py), each independent of its own
arithmetic: exact integer-valued cases and fractions for the BF16 GEMM, one-hot
closed forms for the fused un-permuting sum, brute-force loops for the weight
gradient, and the gradient of the gate softmax against finite differences of
the whole router (logits -> gates)."""
from fractions import Fraction

import numpy as np

from oracle import formats as fmt
from oracle import route
from oracle import router


def _bf16(a):
    return fmt.f64_to_bf16(np.asarray(a, dtype=np.float64))


def test_logits_exact_on_integer_operands():
    rng = np.random.default_rng(0)
    x = rng.integers(-8, 9, (7, 48)).astype(np.float64)
    w = rng.integers(-8, 9, (5, 48)).astype(np.float64) * 0.25
    got = router.logits(_bf16(x), _bf16(w))
    want = np.array([[sum(Fraction(x[t, c]) * Fraction(w[e, c]) for c in range(48)) for e in range(5)]
                     for t in range(7)], dtype=np.float64)
    assert np.array_equal(got.astype(np.float64), want)


def test_logits_round_once_against_fractions():
    """Random bf16 operands: the float32 result is the exact rational sum rounded
    once to nearest (checked through the two neighbouring float32 values)."""
    rng = np.random.default_rng(1)
    xb = _bf16(rng.standard_normal((3, 64)))
    wb = _bf16(rng.standard_normal((4, 64)) * 0.1)
    got = router.logits(xb, wb)
    xf, wf = fmt.bf16_to_f32(xb), fmt.bf16_to_f32(wb)
    for t in range(3):
        for e in range(4):
            s = sum(Fraction(float(xf[t, c])) * Fraction(float(wf[e, c])) for c in range(64))
            g = got[t, e]
            lo, hi = np.nextafter(g, np.float32(-np.inf)), np.nextafter(g, np.float32(np.inf))
            assert abs(Fraction(float(g)) - s) <= abs(Fraction(float(lo)) - s)
            assert abs(Fraction(float(g)) - s) <= abs(Fraction(float(hi)) - s)


def test_unpermute_sum_router_one_hot():
    """dXp rows one-hot at their row number, W_r rows one-hot at d-1-e, dz a
    power of two per (token, slot): every output column holds one term."""
    rng = np.random.default_rng(2)
    T, k, E = 12, 3, 9
    A = T * k
    d = 64
    inv = rng.permutation(A).astype(np.int32)
    dXp = np.zeros((A, d), dtype=np.float32)
    dXp[np.arange(A), np.arange(A)] = np.arange(A) + 1.0
    w = np.zeros((E, d))
    w[np.arange(E), d - 1 - np.arange(E)] = 1.0 + np.arange(E) / 8.0
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    dl = np.zeros((T, E), dtype=np.float32)
    for t in range(T):
        for j in range(k):
            dl[t, idx[t, j]] = 2.0 ** -(t % 4 + j)
    got = fmt.bf16_to_f32(router.unpermute_sum_router(dXp, inv, T, k, dl, idx, _bf16(w))).astype(np.float64)
    want = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            want[t, inv[t * k + j]] += inv[t * k + j] + 1.0
            e = idx[t, j]
            want[t, d - 1 - e] += 2.0 ** -(t % 4 + j) * (1.0 + e / 8.0)
    assert np.array_equal(got, fmt.bf16_to_f32(_bf16(want)).astype(np.float64))


def test_weight_grad_brute_force():
    rng = np.random.default_rng(3)
    T, E, k, d = 20, 6, 2, 16
    xb = _bf16(rng.standard_normal((T, d)))
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    dl = np.zeros((T, E), dtype=np.float32)
    for t in range(T):
        dl[t, idx[t]] = rng.standard_normal(k)
    got = router.weight_grad(xb, dl, idx)
    xf = fmt.bf16_to_f32(xb)
    for e in range(E):
        for c in range(d):
            s = 0.0
            for t in range(T):
                if e in idx[t]:
                    s += float(dl[t, e]) * float(xf[t, c])
            assert abs(got[e, c] - s) <= 1e-12 * (1 + abs(s))


def test_router_chain_matches_finite_differences():
    """loss = sum_t sum_j c[t, j] * g[t, j] with gates from logits = x W^T:
    dL/dW = dz^T x and dL/dx = dz W from the oracle's softmax backward and
    router gradients, against central finite differences in float64 of the
    same loss (top-k set fixed by the unperturbed logits)."""
    rng = np.random.default_rng(4)
    T, E, k, d = 5, 7, 3, 8
    x = fmt.bf16_to_f32(_bf16(rng.standard_normal((T, d)))).astype(np.float64)    # bf16-valued
    w = rng.standard_normal((E, d)) * 0.3
    c = rng.standard_normal((T, k))
    z = x @ w.T
    idx, _ = route.topk_gates(z.astype(np.float32), k)

    def loss(xv, wv):
        zz = xv @ wv.T
        L = 0.0
        for t in range(T):
            sel = zz[t, idx[t]]
            g = np.exp(sel - sel.max())
            g /= g.sum()
            L += float(c[t] @ g)
        return L
    zz = x @ w.T
    gates = np.zeros((T, k))
    for t in range(T):
        sel = zz[t, idx[t]]
        g = np.exp(sel - sel.max())
        gates[t] = g / g.sum()
    dz = route.route_backward(c.astype(np.float32), gates.astype(np.float32), idx, E).astype(np.float64)
    dW = router.weight_grad(_bf16(x), dz, idx)
    xb = x
    h = 1e-6
    for (e, col) in [(idx[0, 0], 1), (idx[2, 1], 5), (idx[4, 2], 0)]:
        wp, wm = w.copy(), w.copy()
        wp[e, col] += h
        wm[e, col] -= h
        fd = (loss(xb, wp) - loss(xb, wm)) / (2 * h)
        assert abs(dW[e, col] - fd) <= 1e-4 * (1 + abs(fd))
    dxr = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            dxr[t] += dz[t, idx[t, j]] * w[idx[t, j]]
    for (t, col) in [(0, 2), (3, 7)]:
        xp, xm = xb.copy(), xb.copy()
        xp[t, col] += h
        xm[t, col] -= h
        fd = (loss(xp, w) - loss(xm, w)) / (2 * h)
        assert abs(dxr[t, col] - fd) <= 1e-4 * (1 + abs(fd))
    # the fused un-permuting sum adds exactly this term (dXp = 0, W in bf16)
    wb = _bf16(w)
    got = fmt.bf16_to_f32(router.unpermute_sum_router(np.zeros((T * k, d), np.float32), np.arange(T * k), T, k,
                                                       dz.astype(np.float32), idx, wb)).astype(np.float64)
    ref = np.zeros((T, d))
    wf = fmt.bf16_to_f32(wb).astype(np.float64)
    for t in range(T):
        for j in range(k):
            ref[t] += float(np.float32(dz[t, idx[t, j]])) * wf[idx[t, j]]
    assert np.allclose(got, ref, rtol=2 ** -7, atol=1e-30)

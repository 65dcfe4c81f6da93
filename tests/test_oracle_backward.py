"""Pins of the oracle's backward chain that do not reuse the chain's own arithmetic.

* Closed forms with one-hot rows and distinct gates: the gated gradient rows
  (dYp[row] = g[t, j] * dy[t] for the assignment t*k + j of the row), the
  un-permuting sum and the gate-weighted combine.
* One-hot probes through the whole backward: with one-hot upstream gradient
  rows dy[t] = +-2**p_t * e_(i_t) (distinct columns i_t) and down-projection
  weights whose rows are one-hot at an injective column map, every value of
  dH, dXp, dx, dW_down and dW_up is a single product of two quantised
  operands.  MXFP8 rounding (nearest or stochastic) returns one of the two
  values of the block's E4M3 grid around its input (the input itself when it
  lies on the grid), so each output must be a product of such neighbours of
  values the definitions give directly (the forward's dequantised operands,
  the gates, dy).  A transposed operand, a wrong expert, a wrong token index
  or gate slot, or a misrouted row lands outside those sets.
* An independent float64 backward of the unquantised layer (plain loops over
  tokens and slots), which the oracle must track at the NVFP4/MXFP8 error level.
* Planted mistakes, monkeypatched into the oracle on the CPU, that the pins
  above must catch.

The pages fix the chain's steps (lhc.media page, the paragraphs on the backward
transposition and on stochastic rounding; agihunt.info page, "Confirmed": MXFP8
backpropagation with requantisation) but print no values for it.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import formats as fmt
from oracle import layer
from oracle import mxfp8 as mx
from oracle import nvfp4 as nv
from oracle import silu

# positive finite E4M3 magnitudes in increasing order (codes 0x00 .. 0x7E)
_GRID = fmt.e4m3_decode(np.arange(0, 127, dtype=np.int64))
assert np.all(np.diff(_GRID) > 0) and _GRID[-1] == 448.0


def _block_exp(amax):
    """Least integer e with amax <= 448 * 2**e (e = -127 for amax = 0), by search."""
    a = np.asarray(amax, dtype=np.float64)
    out = np.full(a.shape, -127, dtype=np.int64)
    for idx in zip(*np.nonzero(a > 0)):
        v = float(a[idx])
        e = int(np.floor(np.log2(v / 448.0))) - 2
        while v > 448.0 * 2.0 ** e:
            e += 1
        out[idx] = max(-127, min(127, e))
    return out


def _nbrs(v, e):
    """(lo, hi): the values of the grid 2**e * E4M3 around each v (signed, float64);
    lo == hi where v lies on the grid."""
    v = np.asarray(v, dtype=np.float64)
    s = np.exp2(np.asarray(e, dtype=np.float64))
    a = np.abs(v) / s
    assert np.all(a <= 448.0)
    i = np.searchsorted(_GRID, a, side="right") - 1
    lo = _GRID[i]
    hi = np.where(lo == a, lo, _GRID[np.minimum(i + 1, len(_GRID) - 1)])
    sg = np.where(np.signbit(v), -1.0, 1.0)
    return sg * lo * s, sg * hi * s


def _products(a_pair, b_pair):
    """The four products of the neighbours of two factors: [4, ...]."""
    (al, ah), (bl, bh) = a_pair, b_pair
    return np.stack([al * bl, al * bh, ah * bl, ah * bh])


def _in_set(got, cands):
    got = np.asarray(got, dtype=np.float64)
    return np.any(cands == got[None], axis=0)


# ------------------------------------------------------------ closed forms

def _random_assignment(rng, T, k):
    A = T * k
    inv = rng.permutation(A).astype(np.int32)       # assignment -> row
    perm = np.empty(A, dtype=np.int32)
    perm[inv] = np.arange(A, dtype=np.int32)        # row -> assignment
    return perm, inv


def _one_hot_probe_gated_rows(T=40, d=16, k=3, seed=0):
    rng = np.random.default_rng(seed)
    perm, inv = _random_assignment(rng, T, k)
    # dy[t] = (t + 1) e_(t mod d): exact in bf16 (t + 1 <= 256)
    dyf = np.zeros((T, d), dtype=np.float32)
    dyf[np.arange(T), np.arange(T) % d] = np.arange(T) + 1.0
    dy = fmt.bf16_round(dyf)
    # distinct gates with 9 significant bits, so g * (t + 1) is exact in float32
    gates = (1.0 + np.arange(T * k).reshape(T, k) / 256.0).astype(np.float32) / 4.0
    got = layer.gated_grad_rows(dy, gates, perm, k)
    want = np.zeros((T * k, d), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            want[inv[t * k + j], t % d] = float(gates[t, j]) * (t + 1)
    return got, want


def test_gated_grad_rows_one_hot_distinct_gates():
    got, want = _one_hot_probe_gated_rows()
    assert got.dtype == np.float32
    assert np.array_equal(got.astype(np.float64), want)


def test_unpermute_sum_one_hot_rows():
    """dXp[row] = (row + 1) e_row (d > A: no two rows share a column), so
    dx[t] holds row + 1 at column row for exactly the k rows of token t."""
    rng = np.random.default_rng(1)
    T, k = 30, 4
    A = T * k
    d = 128
    perm, inv = _random_assignment(rng, T, k)
    dXp = np.zeros((A, d), dtype=np.float32)
    dXp[np.arange(A), np.arange(A)] = np.arange(A) + 1.0
    got = fmt.bf16_to_f32(layer.unpermute_sum(dXp, inv, T, k)).astype(np.float64)
    want = np.zeros((T, d))
    for row in range(A):
        want[perm[row] // k, row] = row + 1.0      # row holds assignment perm[row] of token perm[row] // k
    assert np.array_equal(got, want)


def test_combine_one_hot_rows_distinct_gates():
    """Yp[row] = (row + 1) e_row and gates 2**-(j + 1 + t mod 3): y[t] holds
    g[t, j] * (row + 1) at column row = inv[t*k + j] (exact in bf16)."""
    rng = np.random.default_rng(2)
    T, k = 25, 3
    A = T * k
    d = 96
    perm, inv = _random_assignment(rng, T, k)
    Yp = np.zeros((A, d), dtype=np.float32)
    Yp[np.arange(A), np.arange(A)] = np.arange(A) + 1.0
    gates = np.exp2(-(np.arange(k)[None, :] + 1.0 + (np.arange(T) % 3)[:, None])).astype(np.float32)
    got = fmt.bf16_to_f32(layer.combine(Yp, gates, inv, k)).astype(np.float64)
    want = np.zeros((T, d))
    for row in range(A):
        t, j = divmod(int(perm[row]), k)
        want[t, row] = float(gates[t, j]) * (row + 1)
    assert np.array_equal(got, want)


# --------------------------------------------------- one-hot probe backward

def _probe_inputs(k, seed, T=64, d=64, F=96, E=4):
    rng = np.random.default_rng(seed)
    x = synth.bf16_bits(torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16))
    w_up = (rng.standard_normal((E, F, d)) * 0.02).astype(np.float32)
    # W_down[e] row i is one-hot at column fmap[e][i] (injective per expert)
    fmap = np.array([[(5 * i + 3 * e) % F for i in range(d)] for e in range(E)])
    w_down = np.zeros((E, d, F), dtype=np.float32)
    for e in range(E):
        w = (rng.standard_normal(d) * 0.05).astype(np.float32)
        w[w == 0] = 0.01
        w_down[e, np.arange(d), fmap[e]] = w
    # dy[t] = +-2**p e_(i_t), distinct columns i_t
    cols = rng.permutation(d)[:T]
    p = rng.integers(-12, -5, T)
    sgn = rng.choice([-1.0, 1.0], T)
    dyf = np.zeros((T, d), dtype=np.float32)
    dyf[np.arange(T), cols] = sgn * np.exp2(p)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    return dict(x=x, w_up=w_up, w_down=w_down, fmap=fmap, cols=cols, dyf=dyf, dy=fmt.bf16_round(dyf),
                logits=logits, k=k, dims=(T, d, F, E))


def _rows_of(off, e):
    return np.arange(off[e], off[e + 1])


def _check_probe_backward(inp, fw, bw):
    """Asserts every output of the backward is the product of neighbours the
    definitions give (see the module docstring); returns the number of
    non-zero values checked."""
    T, d, F, E = inp["dims"]
    k = inp["k"]
    P = fw["perm"]
    off, perm, inv = np.asarray(P["off"], np.int64), np.asarray(P["perm"], np.int64), np.asarray(P["inv_perm"], np.int64)
    gates = fw["gates"]
    cols, fmap, dyf = inp["cols"], inp["fmap"], inp["dyf"]
    A = T * k
    tok = perm // k
    slot = perm % k
    exp_of = np.searchsorted(off, np.arange(A), side="right") - 1      # expert of each row
    n_checked = 0

    # 1. dYp[row] = g[t, j] * dy[t]: one-hot at i_t, exact (power-of-two dy)
    dyp_val = gates[tok, slot].astype(np.float64) * dyf[tok, cols[tok]].astype(np.float64)
    want = np.zeros((A, d))
    want[np.arange(A), cols[tok]] = dyp_val
    assert np.array_equal(bw["dYp"].astype(np.float64), want), "dYp"
    # neighbours of each row's single non-zero (its MX block holds it alone, row-wise and per column)
    dyp_n = _nbrs(dyp_val, _block_exp(np.abs(dyp_val)))

    # 2. dH[row] is one-hot at f* = fmap[e][i_t]: q(dYp) * q(W_down^T value), the
    #    transposed requantised weight's block along d holding one non-zero
    wd_deq = nv.nvfp4_dequantize(fw["wd"]["codes"], fw["wd"]["sf"], fw["wd"]["ts"],
                                 np.arange(E + 1) * d).astype(np.float64).reshape(E, d, F)
    fstar = fmap[exp_of, cols[tok]]
    wv = wd_deq[exp_of, cols[tok], fstar]
    assert np.all(wv != 0)
    cands = _products(dyp_n, _nbrs(wv, _block_exp(np.abs(wv))))
    dH = bw["dH"].astype(np.float64)
    assert _in_set(dH[np.arange(A), fstar], cands).all(), "dH value"
    dH_off = dH.copy()
    dH_off[np.arange(A), fstar] = 0
    assert not dH_off.any(), "dH outside the probed column"
    n_checked += A

    # 3. dU = fl(dH * silu'(U)) at f*, and its neighbours
    dsil = silu.dsilu_f32(fw["U"][np.arange(A), fstar])
    du_val = (bw["dH"][np.arange(A), fstar] * dsil).astype(np.float32).astype(np.float64)
    assert np.array_equal(bw["dU"][np.arange(A), fstar].astype(np.float64), du_val), "dU"
    du_n = _nbrs(du_val, _block_exp(np.abs(du_val)))

    # 4. dXp[row, i'] = q(dU) * q(W_up value at (f*, i')), the block of 32 f's of column i'
    wu_deq = nv.nvfp4_dequantize(fw["wu"]["codes"], fw["wu"]["sf"], fw["wu"]["ts"],
                                 np.arange(E + 1) * F).astype(np.float64).reshape(E, F, d)
    blk_amax = np.abs(wu_deq).reshape(E, F // 32, 32, d).max(axis=2)        # [E, F/32, d]
    wv = wu_deq[exp_of, fstar, :]                                            # [A, d]
    we = _block_exp(blk_amax[exp_of, fstar // 32, :])
    cands = _products((du_n[0][:, None], du_n[1][:, None]), _nbrs(wv, we))
    assert _in_set(bw["dXp"].astype(np.float64), cands).all(), "dXp"
    n_checked += int(np.count_nonzero(bw["dXp"]))

    # 5. dx[t] = bf16(sum_j dXp[row(t, j)]): over every choice of neighbours
    dx = fmt.bf16_to_f32(bw["dx"]).astype(np.float64)
    rows = inv.reshape(T, k)
    sums = np.zeros((1, T, d), dtype=np.float32)
    for j in range(k):
        c = cands[:, rows[:, j], :].astype(np.float32)                       # [4, T, d], exact
        sums = (sums[:, None] + c[None]).reshape(-1, T, d)                   # float32 adds in slot order
    ok = np.zeros((T, d), dtype=bool)
    for s in sums:
        ok |= fmt.bf16_to_f32(fmt.bf16_round(s)).astype(np.float64) == dx
    assert ok.all(), "dx"

    # 6. dW_down[e][i, f] = q(dYp_col) * q(H_T value) for the one row of e with
    #    i_t = i (blocks of 32 of e's rows along each column of H), else 0
    h_deq = nv.nvfp4_dequantize(fw["hq"]["codes"], fw["hq"]["sf"], fw["hq"]["ts"], off).astype(np.float64)
    dWd = bw["dW_down"].astype(np.float64)
    dWu = bw["dW_up"].astype(np.float64)
    x_deq = nv.nvfp4_dequantize(fw["xq_perm"]["codes"], fw["xq_perm"]["sf"], fw["xq_perm"]["ts"]).astype(np.float64)
    for e in range(E):
        r = _rows_of(off, e)
        hit_d = np.zeros(d, dtype=bool)
        hit_f = np.zeros(F, dtype=bool)
        if r.size:
            loc = r - off[e]
            pad = mx.pad32(r.size)
            hb = np.zeros((pad, F))
            hb[:r.size] = np.abs(h_deq[r])
            hamax = hb.reshape(pad // 32, 32, F).max(axis=1)                 # [blocks, F]
            xb = np.zeros((pad, d))
            xb[:r.size] = np.abs(x_deq[r])
            xamax = xb.reshape(pad // 32, 32, d).max(axis=1)
            i_r = cols[tok[r]]
            hn = _nbrs(h_deq[r], _block_exp(hamax[loc // 32]))
            cd = _products((dyp_n[0][r][:, None], dyp_n[1][r][:, None]), hn)  # [4, |r|, F]
            assert _in_set(dWd[e][i_r], cd).all(), f"dW_down expert {e}"
            hit_d[i_r] = True
            f_r = fstar[r]
            xn = _nbrs(x_deq[r], _block_exp(xamax[loc // 32]))
            cu = _products((du_n[0][r][:, None], du_n[1][r][:, None]), xn)
            assert _in_set(dWu[e][f_r], cu).all(), f"dW_up expert {e}"
            hit_f[f_r] = True
            n_checked += int(np.count_nonzero(dWd[e][i_r]) + np.count_nonzero(dWu[e][f_r]))
        assert not dWd[e][~hit_d].any(), f"dW_down expert {e}: rows without a token"
        assert not dWu[e][~hit_f].any(), f"dW_up expert {e}: rows without a token"

    # 7. dg[t, j] = <dy[t], Yp[row]> = dy[t, i_t] * Yp[row, i_t] (one term, exact)
    want = dyf[tok, cols[tok]].astype(np.float64) * fw["Yp"][np.arange(A), cols[tok]].astype(np.float64)
    got = bw["dg"][tok, slot]
    assert np.array_equal(got, want), "dg"
    return n_checked


def _probe(k, seed):
    inp = _probe_inputs(k, seed)
    fw = layer.forward(inp["x"], inp["w_up"], inp["w_down"], inp["logits"], k)
    bw = layer.backward(fw, inp["dy"], seed=3 + seed)
    return inp, fw, bw


@pytest.mark.parametrize("k,seed", [(1, 0), (2, 1), (3, 2)])
def test_backward_one_hot_probe(k, seed):
    inp, fw, bw = _probe(k, seed)
    n = _check_probe_backward(inp, fw, bw)
    T, d, F, E = inp["dims"]
    assert n > T * k * (d // 2)        # most checked values are non-zero


def test_backward_one_hot_probe_rejects_planted_mistakes(monkeypatch):
    """Each planted mistake (in a copy of the oracle's step, on the CPU) fails the probe."""
    inp = _probe_inputs(2, 5)
    fw = layer.forward(inp["x"], inp["w_up"], inp["w_down"], inp["logits"], 2)
    good = layer.gated_grad_rows

    def wrong_slot(dy_bf16, gates, perm, k):
        a = np.asarray(perm, dtype=np.int64)
        a2 = (a // k) * k + (a % k + 1) % k       # the token's next slot's gate
        g = np.asarray(gates, np.float32).reshape(-1)[a2]
        return (g[:, None] * fmt.bf16_to_f32(dy_bf16)[a // k]).astype(np.float32)

    def wrong_token(dy_bf16, gates, perm, k):
        a = np.asarray(perm, dtype=np.int64)
        T = dy_bf16.shape[0]
        g = np.asarray(gates, np.float32).reshape(-1)[a]
        return (g[:, None] * fmt.bf16_to_f32(dy_bf16)[(a // k + 1) % T]).astype(np.float32)

    for bad in (wrong_slot, wrong_token):
        monkeypatch.setattr(layer, "gated_grad_rows", bad)
        bw = layer.backward(fw, inp["dy"])
        with pytest.raises(AssertionError):
            _check_probe_backward(inp, fw, bw)
    monkeypatch.setattr(layer, "gated_grad_rows", good)

    good_un = layer.unpermute_sum

    def misrouted(dXp, inv, T, k):
        inv = np.asarray(inv).copy()
        inv[[0, k]] = inv[[k, 0]]                 # two tokens' first assignments swap rows
        return good_un(dXp, inv, T, k)
    monkeypatch.setattr(layer, "unpermute_sum", misrouted)
    bw = layer.backward(fw, inp["dy"])
    with pytest.raises(AssertionError):
        _check_probe_backward(inp, fw, bw)


# ---------------------------------------------- float64 unquantised backward

def _f64_backward(x_bits, w_up, w_down, idx, gates, dy_bits):
    """Backward of the unquantised layer y[t] = sum_j g_j W_down[e_j] silu(W_up[e_j] x_t),
    token by token and slot by slot, in float64."""
    x = fmt.bf16_to_f32(x_bits).astype(np.float64)
    dy = fmt.bf16_to_f32(dy_bits).astype(np.float64)
    T, k = idx.shape
    E = w_up.shape[0]
    Wu = w_up.astype(np.float64)
    Wd = w_down.astype(np.float64)
    dx = np.zeros_like(x)
    dWu = np.zeros_like(Wu)
    dWd = np.zeros_like(Wd)
    dg = np.zeros((T, k))
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            g = float(gates[t, j])
            u = Wu[e] @ x[t]
            s = 1.0 / (1.0 + np.exp(-u))
            h = u * s
            dg[t, j] = dy[t] @ (Wd[e] @ h)
            dye = g * dy[t]
            dh = Wd[e].T @ dye
            du = dh * s * (1.0 + u * (1.0 - s))
            dx[t] += Wu[e].T @ du
            dWd[e] += np.outer(dye, h)
            dWu[e] += np.outer(du, x[t])
    dz = np.zeros((T, E))
    for t in range(T):
        sm = sum(float(gates[t, i]) * dg[t, i] for i in range(k))
        for j in range(k):
            dz[t, idx[t, j]] = float(gates[t, j]) * (dg[t, j] - sm)
    return dict(dx=dx, dW_up=dWu, dW_down=dWd, dg=dg, dlogits=dz)


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def _f64_case(seed=4):
    inp = synth.layer_inputs(128, 128, 128, 4, 2, device="cpu", seed=seed, outlier_p=0.001, outlier_mul=20.0)
    x = synth.bf16_bits(inp["x"])
    wu, wd = synth.f32_np(inp["w_up"]), synth.f32_np(inp["w_down"])
    dy = synth.bf16_bits(inp["dy"])
    fw = layer.forward(x, wu, wd, synth.f32_np(inp["logits"]), 2)
    ref = _f64_backward(x, wu, wd, fw["idx"], fw["gates"], dy)
    return fw, dy, ref


def _f64_errors(bw, ref, E=4):
    errs = dict(dx=_rel(fmt.bf16_to_f32(bw["dx"]), ref["dx"]), dg=_rel(bw["dg"], ref["dg"]),
                dlogits=_rel(bw["dlogits"], ref["dlogits"]))
    for e in range(E):
        errs[f"dW_up[{e}]"] = _rel(bw["dW_up"][e], ref["dW_up"][e])
        errs[f"dW_down[{e}]"] = _rel(bw["dW_down"][e], ref["dW_down"][e])
    return errs


# NVFP4 (4/6 activations, mode-6 weights) forward and MXFP8 backward: each
# NVFP4 operand carries about 9% relative (RMS) error, and the forward output
# that dg and the backward's dU depend on passes through four of them; measured
# here 0.15-0.20.  The planted mistakes give 0.6-1.5.
F64_TOL = 0.28


def test_backward_tracks_unquantised_float64():
    fw, dy, ref = _f64_case()
    bw = layer.backward(fw, dy)
    errs = _f64_errors(bw, ref)
    print({k_: round(v, 4) for k_, v in errs.items()})
    for key, v in errs.items():
        assert v < F64_TOL, (key, v)


def test_float64_backward_rejects_planted_mistakes(monkeypatch):
    """A wrong token or gate slot in the gated rows, or a misrouted un-permuting
    sum, moves the oracle far from the float64 backward."""
    fw, dy, ref = _f64_case()
    good = layer.gated_grad_rows

    def wrong_slot(dy_bf16, gates, perm, k):
        a = np.asarray(perm, dtype=np.int64)
        g = np.asarray(gates, np.float32).reshape(-1)[(a // k) * k + (a % k + 1) % k]
        return (g[:, None] * fmt.bf16_to_f32(dy_bf16)[a // k]).astype(np.float32)

    def wrong_token(dy_bf16, gates, perm, k):
        a = np.asarray(perm, dtype=np.int64)
        T = dy_bf16.shape[0]
        g = np.asarray(gates, np.float32).reshape(-1)[a]
        return (g[:, None] * fmt.bf16_to_f32(dy_bf16)[(a // k + 1) % T]).astype(np.float32)
    for bad in (wrong_token, wrong_slot):
        monkeypatch.setattr(layer, "gated_grad_rows", bad)
        errs = _f64_errors(layer.backward(fw, dy), ref)
        assert errs["dx"] > 2 * F64_TOL and max(errs.values()) > 2 * F64_TOL, (bad.__name__, errs)
    monkeypatch.setattr(layer, "gated_grad_rows", good)

    good_un = layer.unpermute_sum

    def misrouted(dXp, inv, T, k):
        return good_un(dXp, np.roll(np.asarray(inv), 1), T, k)
    monkeypatch.setattr(layer, "unpermute_sum", misrouted)
    errs = _f64_errors(layer.backward(fw, dy), ref)
    assert errs["dx"] > 2 * F64_TOL, errs

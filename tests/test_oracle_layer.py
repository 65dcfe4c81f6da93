"""Invariants of the whole-layer oracle (small shapes)."""
import numpy as np
import pytest
import torch

import synth
from oracle import formats as fmt
from oracle import gemm
from oracle import mxfp8 as mx
from oracle import layer
from oracle import nvfp4 as nv
from oracle import silu


def _inputs(T=64, d=64, F=96, E=4, k=2, seed=0, zipf=None):
    inp = synth.layer_inputs(T, d, F, E, k, device="cpu", seed=seed, outlier_p=0.001, outlier_mul=20.0, zipf=zipf)
    return dict(x=synth.bf16_bits(inp["x"]), w_up=synth.f32_np(inp["w_up"]), w_down=synth.f32_np(inp["w_down"]),
                logits=synth.f32_np(inp["logits"]), dy=synth.bf16_bits(inp["dy"]),
                bias=None if inp["bias"] is None else synth.f32_np(inp["bias"]), k=k)


def test_single_expert_top1_is_dense_nvfp4_mlp():
    i = _inputs(E=1, k=1)
    fw = layer.forward(i["x"], i["w_up"], i["w_down"], i["logits"], 1)
    assert (fw["gates"] == 1).all()
    assert np.array_equal(fw["perm"]["perm"], np.arange(64))
    xq = nv.nvfp4_quantize(i["x"], nv.MODE_46)
    wu = nv.nvfp4_quantize(i["w_up"][0], nv.MODE_6)
    U = fmt.f64_to_bf16(nv.nvfp4_exact_f64(xq["codes"], xq["sf"], xq["ts"]) @
                        nv.nvfp4_exact_f64(wu["codes"], wu["sf"], wu["ts"]).T)
    assert np.array_equal(U, fw["U"])
    hq = nv.nvfp4_quantize(silu.silu_f32(U), nv.MODE_46)
    wd = nv.nvfp4_quantize(i["w_down"][0], nv.MODE_6)
    Y = (nv.nvfp4_exact_f64(hq["codes"], hq["sf"], hq["ts"]) @ nv.nvfp4_exact_f64(wd["codes"], wd["sf"], wd["ts"]).T).astype(np.float32)
    assert np.array_equal(fmt.bf16_round(Y), fw["y"])


def test_token_permutation_equivariance():
    i = _inputs(seed=1)
    fw = layer.forward(i["x"], i["w_up"], i["w_down"], i["logits"], 2)
    bw = layer.backward(fw, i["dy"])
    p = np.random.default_rng(0).permutation(64)
    fw2 = layer.forward(i["x"][p], i["w_up"], i["w_down"], i["logits"][p], 2)
    assert np.array_equal(fw2["y"], fw["y"][p])
    bw2 = layer.backward(fw2, i["dy"][p])
    assert np.array_equal(bw2["dx"], bw["dx"][p])


def test_zero_input_gives_zero_output():
    i = _inputs(seed=2)
    x = np.zeros_like(i["x"])
    fw = layer.forward(x, i["w_up"], i["w_down"], i["logits"], 2)
    assert not (fw["y"] & 0x7FFF).any()
    bw = layer.backward(fw, np.zeros_like(i["dy"]))
    assert not (bw["dx"] & 0x7FFF).any()
    assert not bw["dW_up"].any() and not bw["dW_down"].any()


def test_expert_relabelling_equivariance():
    i = _inputs(seed=3, E=4)
    fw = layer.forward(i["x"], i["w_up"], i["w_down"], i["logits"], 2)
    p = np.array([2, 0, 3, 1])
    fw2 = layer.forward(i["x"], i["w_up"][p], i["w_down"][p], i["logits"][:, p], 2)
    assert np.array_equal(fw2["y"], fw["y"])


def test_layer_close_to_float64_reference():
    """The quantised layer tracks the unquantised float64 MLP (NVFP4 error level)."""
    i = _inputs(seed=4, T=128, d=128, F=128, E=4, k=2)
    fw = layer.forward(i["x"], i["w_up"], i["w_down"], i["logits"], 2)
    x = fmt.bf16_to_f32(i["x"]).astype(np.float64)
    y = np.zeros((128, 128))
    for t in range(128):
        for j in range(2):
            e = fw["idx"][t, j]
            u = i["w_up"][e].astype(np.float64) @ x[t]
            h = u / (1 + np.exp(-u))
            y[t] += fw["gates"][t, j] * (i["w_down"][e].astype(np.float64) @ h)
    got = fmt.bf16_to_f32(fw["y"]).astype(np.float64)
    rel = np.linalg.norm(got - y) / np.linalg.norm(y)
    assert rel < 0.2, rel


def test_backward_shapes_and_wgrad_reference():
    i = _inputs(seed=5)
    fw = layer.forward(i["x"], i["w_up"], i["w_down"], i["logits"], 2)
    bw = layer.backward(fw, i["dy"])
    T, d, F, E, k = fw["dims"]
    assert bw["dW_up"].shape == (E, F, d) and bw["dW_down"].shape == (E, d, F)
    assert bw["dx"].shape == (T, d)
    # dW_down tracks the float64 product of the unquantised operands
    off = fw["perm"]["off"]
    H = silu.silu_f32(fw["U"]).astype(np.float64)
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        ref = bw["dYp"][r0:r1].astype(np.float64).T @ H[r0:r1]
        rel = np.linalg.norm(bw["dW_down"][e] - ref) / max(np.linalg.norm(ref), 1e-30)
        assert rel < 0.2


def test_dgates_one_hot_rows():
    """Rows of Yp that are (row + 1) times the unit vector e_(row mod d) make
    dg[t, j] = (row + 1) * dy[t, row mod d], row = inv[t*k + j]: pins the
    row mapping and the sum without the oracle's own dot product."""
    rng = np.random.default_rng(3)
    T, d, k = 50, 24, 3
    A = T * k
    inv = rng.permutation(A).astype(np.int32)
    Yp = np.zeros((A, d), dtype=np.float32)
    Yp[np.arange(A), np.arange(A) % d] = np.arange(A) + 1.0
    dy = synth.bf16_bits(torch.randn(T, d).to(torch.bfloat16))
    dg = layer.dgates(dy, Yp, inv, k)
    dyf = fmt.bf16_to_f32(dy)
    rows = inv.reshape(T, k)
    want = (rows + 1.0) * dyf[np.arange(T)[:, None], rows % d]
    assert np.array_equal(dg, want.astype(np.float64))


def test_dgates_brute_force_and_combine_link():
    """Plain loops on a tiny case, and sum_j g * dg = <dy, sum_j g * Yp[row]>
    (the combine's weighted sum before rounding)."""
    rng = np.random.default_rng(4)
    T, d, k = 6, 5, 2
    inv = rng.permutation(T * k).astype(np.int32)
    Yp = rng.standard_normal((T * k, d)).astype(np.float32)
    dy = synth.bf16_bits(torch.randn(T, d).to(torch.bfloat16))
    dyf = fmt.bf16_to_f32(dy)
    dg = layer.dgates(dy, Yp, inv, k)
    for t in range(T):
        for j in range(k):
            s = 0.0
            for c in range(d):
                s += float(dyf[t, c]) * float(Yp[inv[t * k + j], c])
            assert abs(dg[t, j] - s) <= 1e-12 * (1 + abs(s))
    g = rng.random((T, k))
    lhs = (g * dg).sum(axis=1)
    comb = np.stack([sum(g[t, j] * Yp[inv[t * k + j]].astype(np.float64) for j in range(k)) for t in range(T)])
    rhs = (dyf.astype(np.float64) * comb).sum(axis=1)
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_mxfp8_forward_dense_reduction():
    """E = 1, k = 1 and operands exact in MXFP8: U = bf16(x @ W_up^T) exactly,
    Yp = deq(MXFP8(silu(U))) @ W_down^T, y = bf16(Yp)."""
    rng = np.random.default_rng(31)
    T, d, F = 40, 64, 96
    x = (rng.integers(-3, 4, (T, d)) * 0.5).astype(np.float32)
    wu = (rng.integers(-3, 4, (1, F, d)) * 0.25).astype(np.float32)
    wd = (rng.integers(-3, 4, (1, d, F)) * 0.25).astype(np.float32)
    xb = fmt.f64_to_bf16(x.astype(np.float64))
    fw = layer.forward_mx(xb, wu, wd, np.zeros((T, 1), np.float32), 1)
    U = fmt.f64_to_bf16(x.astype(np.float64) @ wu[0].T.astype(np.float64))
    assert np.array_equal(fw["U"], U)
    hc, hs = fw["hq"]["codes"], fw["hq"]["sf"]
    Yp = (mx.dequant_rowwise(hc, hs) @ wd[0].T.astype(np.float64)).astype(np.float32)
    assert np.array_equal(fw["Yp"], Yp)
    assert np.array_equal(fw["y"], fmt.bf16_round(Yp))


def test_mxfp8_backward_tracks_float64():
    i = _inputs(seed=7)
    fw = layer.forward_mx(i["x"], i["w_up"], i["w_down"], i["logits"], 2)
    bw = layer.backward_mx(fw, i["dy"])
    T, d, F, E, k = fw["dims"]
    assert bw["dW_up"].shape == (E, F, d) and bw["dW_down"].shape == (E, d, F) and bw["dx"].shape == (T, d)
    off = fw["perm"]["off"]
    H = silu.silu_f32(fw["U"]).astype(np.float64)
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        ref = bw["dYp"][r0:r1].astype(np.float64).T @ H[r0:r1]
        rel = np.linalg.norm(bw["dW_down"][e] - ref) / max(np.linalg.norm(ref), 1e-30)
        assert rel < 0.1

"""Stage-wise, teacher-forced parity of the whole expert layer (GPU).

Each step of the HIP path is compared with the oracle fed the GPU's own inputs
to that step (copied back to the host):
* byte for byte: routing, every quantiser (X, weights, H with the SiLU amax
  folded into the up GEMM's epilogue, the transposed SR requantisations of
  W_down, H, W_up and X with their stream ids, both MXFP8 copies of g*dY and
  of dU = dH * silu'(U)), the combine, the un-permuting sum, the router
  backward;
* per element, |C - C_exact| <= 1e-3 * sum|a*b| + half an ulp of the output
  type, C_exact the float64 product of the exact dequantised operands: every
  GEMM (U, Yp, dH, dW_down, dXp, dW_up) and the gate gradient.

Also: the RL-rollout-shaped forward (512 tokens, 384 experts of 4096 -> 1536
-> 4096, top-8 of unbiased logits, about 10 rows per expert) on sampled
experts and tokens, and the combined dgrad + wgrad call moe_grouped_gemm_bwd.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import assert_bytes_equal, cuda_i32, gemm_tol_check, to_np
from oracle import formats as fmt
from oracle import gemm as og
from oracle import layer as olayer
from oracle import mxfp8 as mx
from oracle import nvfp4 as nv
from oracle import route
from oracle import silu

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import precision_moe_numerics_quant_amd as m4
    from precision_moe_numerics_quant_amd import layer


def _nv(q):
    return dict(codes=to_np(q[0]), sf=to_np(q[1]), ts=to_np(q[2]))


def _check_nv(got, want, what):
    assert_bytes_equal(got["codes"], want["codes"], what + " codes")
    assert_bytes_equal(got["sf"], want["sf"], what + " scales")
    assert_bytes_equal(np.asarray(got["ts"], np.float32).view(np.uint32),
                       np.asarray(want["ts"], np.float32).view(np.uint32), what + " tensor scales")


def _check_t(got_pair, want_pair, what):
    """A transposed group-major MXFP8 pair; the GPU's buffers are sized by the
    padded upper bound, so only the written extent is compared."""
    n = len(want_pair[0])
    assert_bytes_equal(to_np(got_pair[0])[:n], want_pair[0], what + " codes")
    assert_bytes_equal(to_np(got_pair[1])[:n // 32], want_pair[1], what + " scales")


def _wgrad_check(got, a_list, b_list, what):
    exact = og.wgrad(a_list, b_list)
    bound = og.wgrad([np.abs(a) for a in a_list], [np.abs(b) for b in b_list])
    gemm_tol_check(got.astype(np.float64), exact, bound, what)


def test_layer_config1_stagewise_teacher_forced():
    inp = synth.config_inputs(1, device="cpu")
    c = synth.CONFIGS[1]
    T, d, F, E, k = c["T"], c["d"], c["F"], c["E"], c["k"]
    seed, lay = synth.SR_SEED, 0
    sid = lambda role: 16 * lay + role
    dev = {kk: (v.cuda() if torch.is_tensor(v) else v) for kk, v in inp.items()}
    fw = layer.forward(dev["x"], dev["w_up"], dev["w_down"], dev["logits"], k, seed=seed, layer=lay)
    bw = layer.backward(fw, dev["dy"], seed=seed, layer=lay)
    torch.cuda.synchronize()
    x = synth.bf16_bits(inp["x"])
    dy = synth.bf16_bits(inp["dy"])
    w_up, w_down = synth.f32_np(inp["w_up"]), synth.f32_np(inp["w_down"])

    # routing (identical inputs): bit-exact
    idx, gates = route.topk_gates(synth.f32_np(inp["logits"]), k)
    P = route.permutation(idx, E)
    r = fw["route"]
    assert_bytes_equal(to_np(r["idx"]), idx, "idx")
    assert_bytes_equal(to_np(r["gates"]).view(np.uint32), gates.view(np.uint32), "gates")
    for key in ("off", "off_pad", "perm", "inv_perm"):
        assert_bytes_equal(to_np(r[key]), P[key], key)
    off, perm, inv = P["off"], P["perm"], P["inv_perm"]

    # F1: weights, and their transposed SR copies (roles 2, 3)
    wu, wd = olayer.quantize_weights(w_up, w_down)
    _check_nv(_nv(fw["wq"]["wu"]), wu, "W_up")
    _check_nv(_nv(fw["wq"]["wd"]), wd, "W_down")
    wdT = mx.requant_sr_t(wd["codes"], wd["sf"], wd["ts"], np.arange(E + 1) * d, True, seed, sid(3), mx.SF_ROWS)
    wuT = mx.requant_sr_t(wu["codes"], wu["sf"], wu["ts"], np.arange(E + 1) * F, True, seed, sid(2), mx.SF_ROWS)
    _check_t(bw["wdT"], wdT, "W_down^T requant")
    _check_t(bw["wuT"], wuT, "W_up^T requant")

    # F4, F5: X quant and the dispatch gather
    xq = nv.nvfp4_quantize(x, nv.MODE_46)
    _check_nv(_nv(fw["xq"]), xq, "X")
    src = perm.astype(np.int64) // k
    assert_bytes_equal(to_np(fw["xq_perm"][0]), xq["codes"][src], "X gathered codes")
    assert_bytes_equal(to_np(fw["xq_perm"][1]), xq["sf"][src], "X gathered scales")

    # F6: U per element (bf16 out)
    A64 = nv.nvfp4_exact_f64(xq["codes"][src], xq["sf"][src], xq["ts"])
    Bup = nv.nvfp4_exact_f64(wu["codes"], wu["sf"], wu["ts"], np.arange(E + 1) * F).reshape(E, F, d)
    U = to_np(fw["U"])
    gemm_tol_check(fmt.bf16_to_f32(U).astype(np.float64), og.grouped_nt(A64, Bup, off),
                   og.abs_bound_nt(A64, Bup, off), "U", out_bf16=True)

    # F7: H = silu(U) of the GPU's U -> NVFP4 4/6 per expert (the amax came from F6's epilogue)
    hq = nv.nvfp4_quantize(silu.silu_f32(U), nv.MODE_46, off)
    _check_nv(_nv(fw["hq"]), hq, "H")

    # F8: Yp per element (float32 out)
    H64 = nv.nvfp4_exact_f64(hq["codes"], hq["sf"], hq["ts"], off)
    Bdn = nv.nvfp4_exact_f64(wd["codes"], wd["sf"], wd["ts"], np.arange(E + 1) * d).reshape(E, d, F)
    Yp = to_np(fw["Yp"])
    gemm_tol_check(Yp.astype(np.float64), og.grouped_nt(H64, Bdn, off), og.abs_bound_nt(H64, Bdn, off), "Yp")

    # F9: combine of the GPU's Yp, bit-exact
    assert_bytes_equal(to_np(fw["y"]), olayer.combine(Yp, gates, inv, k), "y")

    # B1: g * dY gathered -> MXFP8 RNE row-wise and transposed (block-major scales)
    dYp = olayer.gated_grad_rows(dy, gates, perm, k)
    dy_row = mx.quantize_rowwise(dYp, mx.RNE)
    dy_col = mx.quantize_transposed(dYp, off, mx.RNE, sf_layout=mx.SF_BLOCKS)
    assert_bytes_equal(to_np(bw["dy_row"][0]), dy_row[0], "dY row codes")
    assert_bytes_equal(to_np(bw["dy_row"][1]), dy_row[1], "dY row scales")
    _check_t(bw["dy_col"], dy_col, "dY transposed")

    # B3: dH per element
    WdT = np.stack(mx.dequant_transposed(wdT[0], wdT[1], np.arange(E + 1) * d, F))
    dYr = mx.dequant_rowwise(*dy_row)
    dH = to_np(bw["dH"])
    gemm_tol_check(dH.astype(np.float64), og.grouped_nt(dYr, WdT, off), og.abs_bound_nt(dYr, WdT, off), "dH")

    # B4: H requantised (role 1) from the GPU's Hq
    hT = mx.requant_sr_t(hq["codes"], hq["sf"], hq["ts"], off, True, seed, sid(1), mx.SF_BLOCKS)
    _check_t(bw["hT"], hT, "H^T requant")

    # B5: dW_down per element
    _wgrad_check(to_np(bw["dW_down"]), mx.dequant_transposed(dy_col[0], dy_col[1], off, d, mx.SF_BLOCKS),
                 mx.dequant_transposed(hT[0], hT[1], off, F, mx.SF_BLOCKS), "dW_down")

    # B6: dU = fl(dH * silu'(U)) from the GPU's dH and U -> both MXFP8 copies
    dU = (dH * silu.dsilu_f32(U)).astype(np.float32)
    du_row = mx.quantize_rowwise(dU, mx.RNE)
    du_col = mx.quantize_transposed(dU, off, mx.RNE, sf_layout=mx.SF_BLOCKS)
    assert_bytes_equal(to_np(bw["du_row"][0]), du_row[0], "dU row codes")
    assert_bytes_equal(to_np(bw["du_row"][1]), du_row[1], "dU row scales")
    _check_t(bw["du_col"], du_col, "dU transposed")

    # B8: dXp per element
    WuT = np.stack(mx.dequant_transposed(wuT[0], wuT[1], np.arange(E + 1) * F, d))
    dUr = mx.dequant_rowwise(*du_row)
    dXp = to_np(bw["dXp"])
    gemm_tol_check(dXp.astype(np.float64), og.grouped_nt(dUr, WuT, off), og.abs_bound_nt(dUr, WuT, off), "dXp")

    # B9: X requantised (role 0, the single tensor scale)
    xT = mx.requant_sr_t(xq["codes"][src], xq["sf"][src], xq["ts"], off, False, seed, sid(0), mx.SF_BLOCKS)
    _check_t(bw["xT"], xT, "X^T requant")

    # B10: dW_up per element
    _wgrad_check(to_np(bw["dW_up"]), mx.dequant_transposed(du_col[0], du_col[1], off, F, mx.SF_BLOCKS),
                 mx.dequant_transposed(xT[0], xT[1], off, d, mx.SF_BLOCKS), "dW_up")

    # B11: un-permuting sum of the GPU's dXp, bit-exact
    assert_bytes_equal(to_np(bw["dx"]), olayer.unpermute_sum(dXp, inv, T, k), "dx")

    # B12: gate gradient per element; B13: router backward of the GPU's dg, bit-exact
    dg = to_np(bw["dg"])
    gemm_tol_check(dg.astype(np.float64), olayer.dgates(dy, Yp, inv, k),
                   olayer.dgates(dy & 0x7FFF, np.abs(Yp), inv, k), "dg")
    assert_bytes_equal(to_np(bw["dlogits"]).view(np.uint32),
                       route.route_backward(dg, gates, idx, E).view(np.uint32), "dlogits")


# ------------------------------------------------- RL-rollout-shaped forward

def test_rl_rollout_forward_config5_sampled():
    """T = 512, d = 4096, F = 1536, E = 384, top-8 of unbiased N(0,1) logits
    (about 10 rows per expert), forward only, in the launches the benchmark
    times: routing and X in full, sampled experts' weights, U, H, Yp, and
    sampled tokens' y, each teacher-forced against the oracle."""
    c = synth.CONFIGS[5]
    T, d, F, E, k = c["T"], c["d"], c["F"], c["E"], c["k"]
    inp = synth.layer_inputs(T, d, F, E, k, device="cuda", seed=0, zipf=None, with_dy=False)
    print("config 5: weights + forward on the GPU", flush=True)
    wq = layer.quantize_weights(inp["w_up"], inp["w_down"])
    fw = layer.forward(inp["x"], inp["w_up"], inp["w_down"], inp["logits"], k, wq=wq)
    torch.cuda.synchronize()
    idx, gates = route.topk_gates(synth.f32_np(inp["logits"]), k)
    P = route.permutation(idx, E)
    r = fw["route"]
    for key in ("off", "off_pad", "perm", "inv_perm"):
        assert_bytes_equal(to_np(r[key]), P[key], key)
    assert_bytes_equal(to_np(r["gates"]).view(np.uint32), gates.view(np.uint32), "gates")
    off, perm, inv = P["off"].astype(np.int64), P["perm"], P["inv_perm"]
    cnt = np.diff(off)
    assert cnt.min() >= 1 and cnt.max() <= 32                 # every expert has a few rows
    x = synth.bf16_bits(inp["x"])
    xq = nv.nvfp4_quantize(x, nv.MODE_46)
    _check_nv(_nv(fw["xq"]), xq, "X")
    src = perm.astype(np.int64) // k
    U = to_np(fw["U"])
    Yp = to_np(fw["Yp"])
    hq_gpu = _nv(fw["hq"])
    wu_c, wu_s, wu_t = (to_np(t) for t in wq["wu"])
    wd_c, wd_s, wd_t = (to_np(t) for t in wq["wd"])
    rng = np.random.default_rng(1)
    experts = sorted({0, E - 1, int(np.argmax(cnt)), int(np.argmin(cnt)), *rng.choice(E, 3, replace=False).tolist()})
    for e in experts:
        rows = np.arange(off[e], off[e + 1])
        # this expert's weights (mode 6, one tensor scale), bit-exact
        qu = nv.nvfp4_quantize(synth.f32_np(inp["w_up"][e]), nv.MODE_6)
        qd = nv.nvfp4_quantize(synth.f32_np(inp["w_down"][e]), nv.MODE_6)
        _check_nv(dict(codes=wu_c[e * F:(e + 1) * F], sf=wu_s[e * F:(e + 1) * F], ts=wu_t[e:e + 1]), qu, f"W_up[{e}]")
        _check_nv(dict(codes=wd_c[e * d:(e + 1) * d], sf=wd_s[e * d:(e + 1) * d], ts=wd_t[e:e + 1]), qd, f"W_down[{e}]")
        a64 = nv.nvfp4_exact_f64(xq["codes"][src[rows]], xq["sf"][src[rows]], xq["ts"])
        b64 = nv.nvfp4_exact_f64(qu["codes"], qu["sf"], qu["ts"])
        gemm_tol_check(fmt.bf16_to_f32(U[rows]).astype(np.float64), a64 @ b64.T, np.abs(a64) @ np.abs(b64).T,
                       f"U expert {e}", out_bf16=True)
        # H of this expert from the GPU's U: one tensor scale for the expert's rows
        hq = nv.nvfp4_quantize(silu.silu_f32(U[rows]), nv.MODE_46)
        _check_nv(dict(codes=hq_gpu["codes"][rows], sf=hq_gpu["sf"][rows], ts=hq_gpu["ts"][e:e + 1]), hq, f"H[{e}]")
        h64 = nv.nvfp4_exact_f64(hq["codes"], hq["sf"], hq["ts"])
        bd = nv.nvfp4_exact_f64(qd["codes"], qd["sf"], qd["ts"])
        gemm_tol_check(Yp[rows].astype(np.float64), h64 @ bd.T, np.abs(h64) @ np.abs(bd).T, f"Yp expert {e}")
    toks = np.unique(np.r_[rng.choice(T, 24, replace=False), 0, T - 1])
    y = to_np(fw["y"])
    local_inv = np.arange(len(toks) * k, dtype=np.int32)
    yp_s = Yp[inv.reshape(T, k)[toks].reshape(-1)]
    assert_bytes_equal(y[toks], olayer.combine(yp_s, gates[toks], local_inv, k), "y sampled tokens")


# ------------------------------------------------ combined backward call

@pytest.mark.parametrize("M_list,Nout,Nin", [([0, 37, 130, 1, 300], 256, 512), ([64, 0, 200], 1536, 1024)])
def test_grouped_gemm_bwd_combined_call(M_list, Nout, Nin):
    """moe_grouped_gemm_bwd (dgrad and wgrad of one expert linear in one call)
    against the oracle: dx per element from dy row-wise and W^T requantised,
    dW per element from the transposed dy and x (beta = 0, empty experts
    zero)."""
    E = len(M_list)
    off = np.concatenate([[0], np.cumsum(M_list)]).astype(np.int64)
    M = int(off[-1])
    offp = mx.padded_offsets(off)
    rng = np.random.default_rng(M + Nout)
    dyf = (rng.standard_normal((M, Nout)) * 1e-3).astype(np.float32)
    xf = rng.standard_normal((M, Nin)).astype(np.float32)
    wT = (rng.standard_normal((E * Nin, Nout)) * 0.02).astype(np.float32)   # W^T [E][Nin][Nout]
    dy_row = mx.quantize_rowwise(dyf, mx.RNE)
    dy_col = mx.quantize_transposed(dyf, off, mx.RNE, sf_layout=mx.SF_BLOCKS)
    x_col = mx.quantize_transposed(xf, off, mx.SR, seed=3, stream_id=0, sf_layout=mx.SF_BLOCKS)
    w_row = mx.quantize_rowwise(wT, mx.SR, seed=3, stream_id=2)
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    dx, dw = m4.moe_grouped_gemm_bwd(g(dy_row[0]), g(dy_row[1]), g(w_row[0]), g(w_row[1]), g(dy_col[0]),
                                     g(dy_col[1]), g(x_col[0]), g(x_col[1]), cuda_i32(off), cuda_i32(offp),
                                     Nin, Nout)
    torch.cuda.synchronize()
    a = mx.dequant_rowwise(*dy_row)
    b = mx.dequant_rowwise(*w_row).reshape(E, Nin, Nout)
    gemm_tol_check(to_np(dx).astype(np.float64), og.grouped_nt(a, b, off), og.abs_bound_nt(a, b, off), "dx")
    _wgrad_check(to_np(dw), mx.dequant_transposed(dy_col[0], dy_col[1], off, Nout, mx.SF_BLOCKS),
                 mx.dequant_transposed(x_col[0], x_col[1], off, Nin, mx.SF_BLOCKS), "dW")

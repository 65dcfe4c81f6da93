"""The NVFP4-forward / MXFP8-backward expert layer, end to end (test infrastructure).

Pages: agihunt.info page, "Confirmed" (expert layers' forward in NVFP4,
backpropagation in MXFP8 with requantisation and stochastic rounding; 4/6
activation quantisation); lhc.media page, the paragraphs on precisions (FP32
master weights, some BF16 activations), on the backward transposition and
stochastic rounding, and on dispatching NVFP4 inputs to the experts;
fourweekmba.com page, "Update" (a token goes to 8 of 384 experts).

Forward (readings where the pages are silent: weights use the plain
amax->6 scale with one tensor scale per expert matrix; X is quantised once,
before dispatch, with one tensor scale; H gets one tensor scale per expert):

 1. Wq_up[e] = NVFP4(W_up[e] [F, d], mode 6); Wq_down[e] = NVFP4(W_down[e] [d, F], mode 6)
 2. route: top-k indices and gates; stable permutation by expert
 3. Xq = NVFP4(x [T, d], 4/6, one tensor scale)
 4. Xq_perm = rows of Xq in expert order (codes and block scales; S_x shared)
 5. U = bf16(exact Xq_perm_e . Wq_up[e]^T)
 6. H = silu(U) (correctly rounded float32); Hq = NVFP4(H, 4/6, one group per expert)
 7. Yp = float32(exact Hq_e . Wq_down[e]^T)
 8. y[t] = bf16(acc), acc = 0; for j = 0..k-1: acc = fl(acc + fl(g[t, j] * Yp[row(t, j)]))

Backward (gradients dY, dU in MXFP8 with RNE; forward operands requantised with
stochastic rounding, stream id 16 * layer + role, role 0 = X_T, 1 = H_T,
2 = W_up_T, 3 = W_down_T):

 1. dYp[row(t, j)] = fl(g[t, j] * dy[t]); MXFP8 row-wise [A, d] and transposed per expert
 2. Wd_T = requant_sr_t(Wq_down, groups of d rows) -> [E][F][d]
 3. dH = float32(exact dYp_row . Wd_T[e]^T)                 [A, F]
 4. H_T = requant_sr_t(Hq, groups = experts)                -> [E][F][pad32 M_e]
 5. dW_down[e] = float32(exact dYp_col[e] . H_T[e]^T)        [E, d, F]
 6. dU = fl(dH * dsilu(U)); MXFP8 row-wise and transposed per expert
 7. Wu_T = requant_sr_t(Wq_up, groups of F rows)             -> [E][d][F]
 8. dXp = float32(exact dU_row . Wu_T[e]^T)                   [A, d]
 9. X_T = requant_sr_t(Xq_perm, groups = experts, S_x)       -> [E][d][pad32 M_e]
10. dW_up[e] = float32(exact dU_col[e] . X_T[e]^T)          [E, F, d]
11. dx[t] = bf16(acc), acc = 0; for j: acc = fl(acc + dXp[row(t, j)])
12. dg[t, j] = <dy[t], Yp[row(t, j)]>: the gate gradient, the derivative of the
    combine's weighted sum in g[t, j] (exact here; a float32 sum of d products
    in the library)
13. dlogits = route_backward(fl32(dg), g, idx): the softmax backward over each
    token's selected experts (route.py)

The transposed operands of the weight-gradient products (dYp_col, H_T, dU_col,
X_T) keep their scales block-major (SF_BLOCKS), the requantised weights
row-major (SF_ROWS): storage only, the values are the same either way.
"""
import numpy as np

from . import formats as fmt
from . import gemm
from . import mxfp8 as mx
from . import nvfp4 as nv
from . import route
from . import silu

ROLE_X, ROLE_H, ROLE_WUP, ROLE_WDOWN = 0, 1, 2, 3


def quantize_weights(W_up, W_down):
    E, F, d = W_up.shape
    wu = nv.nvfp4_quantize(W_up.reshape(E * F, d), nv.MODE_6, np.arange(E + 1) * F)
    wd = nv.nvfp4_quantize(W_down.reshape(E * d, F), nv.MODE_6, np.arange(E + 1) * d)
    return wu, wd


def forward(x_bf16, W_up, W_down, logits, k, bias=None, weights_q=None):
    """x_bf16 [T, d] uint16 bf16 bits; W_up [E, F, d], W_down [E, d, F] float32."""
    T, d = x_bf16.shape
    E, F, _ = W_up.shape
    wu, wd = quantize_weights(W_up, W_down) if weights_q is None else weights_q
    idx, gates = route.topk_gates(logits, k, bias)
    P = route.permutation(idx, E)
    off, perm, inv = P["off"], P["perm"], P["inv_perm"]
    xq = nv.nvfp4_quantize(x_bf16, nv.MODE_46)
    src = perm.astype(np.int64) // k
    xq_perm = dict(codes=xq["codes"][src], sf=xq["sf"][src], ts=xq["ts"])
    A64 = nv.nvfp4_exact_f64(xq_perm["codes"], xq_perm["sf"], xq_perm["ts"])
    Bup = nv.nvfp4_exact_f64(wu["codes"], wu["sf"], wu["ts"], np.arange(E + 1) * F).reshape(E, F, d)
    U = fmt.f64_to_bf16(gemm.grouped_nt(A64, Bup, off))
    H = silu.silu_f32(U)
    hq = nv.nvfp4_quantize(H, nv.MODE_46, off)
    H64 = nv.nvfp4_exact_f64(hq["codes"], hq["sf"], hq["ts"], off)
    Bdn = nv.nvfp4_exact_f64(wd["codes"], wd["sf"], wd["ts"], np.arange(E + 1) * d).reshape(E, d, F)
    Yp = gemm.grouped_nt(H64, Bdn, off).astype(np.float32)
    y = combine(Yp, gates, inv, k)
    return dict(wu=wu, wd=wd, idx=idx, gates=gates, perm=P, xq=xq, xq_perm=xq_perm,
                U=U, hq=hq, Yp=Yp, y=y, dims=(T, d, F, E, k))


def combine(Yp, gates, inv, k):
    """y[t] = bf16(sum_j fl(g[t,j] * Yp[row(t,j)])) in order j = 0..k-1."""
    T = gates.shape[0]
    d = Yp.shape[1]
    acc = np.zeros((T, d), dtype=np.float32)
    inv = np.asarray(inv, dtype=np.int64).reshape(T, k)
    for j in range(k):
        acc = (acc + (gates[:, j:j + 1] * Yp[inv[:, j]]).astype(np.float32)).astype(np.float32)
    return fmt.bf16_round(acc)


def unpermute_sum(dXp, inv, T, k):
    """dx[t] = bf16(sum_j dXp[row(t,j)]) in order j = 0..k-1."""
    d = dXp.shape[1]
    acc = np.zeros((T, d), dtype=np.float32)
    inv = np.asarray(inv, dtype=np.int64).reshape(T, k)
    for j in range(k):
        acc = (acc + dXp[inv[:, j]]).astype(np.float32)
    return fmt.bf16_round(acc)


def dgates(dy_bf16, Yp, inv, k):
    """dg[t, j] = sum_c dy[t, c] * Yp[row(t, j), c], row(t, j) = inv[t*k + j]
    (float64: every product of a bf16 and a float32 is exact)."""
    dy = fmt.bf16_to_f32(dy_bf16).astype(np.float64)
    T = dy.shape[0]
    rows = np.asarray(inv, dtype=np.int64).reshape(T, k)
    Y = np.asarray(Yp, dtype=np.float64)
    return np.stack([np.einsum("tc,tc->t", dy, Y[rows[:, j]]) for j in range(k)], axis=1)


def gated_grad_rows(dy_bf16, gates, perm, k):
    """dYp[row] = fl(g[t, j] * dy[t]) for the assignment a = perm[row] = t*k + j."""
    dy = fmt.bf16_to_f32(dy_bf16)
    a = np.asarray(perm, dtype=np.int64)
    g = np.asarray(gates, dtype=np.float32).reshape(-1)[a]
    return (g[:, None] * dy[a // k]).astype(np.float32)


def backward(fw, dy_bf16, seed=1, layer=0):
    """The backward of ``forward`` (steps 1-13 above)."""
    def req(q, off, ts_per_group, role, layout):
        return mx.requant_sr_t(q["codes"], q["sf"], q["ts"], off, ts_per_group, seed, 16 * layer + role, layout)
    return _backward(fw, dy_bf16, req)


def _backward(fw, dy_bf16, req):
    """Backward steps; req(q, group offsets, ts per group, role, scale layout)
    is the transposed SR requantisation of the forward operand q."""
    T, d, F, E, k = fw["dims"]
    P = fw["perm"]
    off, perm, inv = P["off"], P["perm"], P["inv_perm"]
    dYp = gated_grad_rows(dy_bf16, fw["gates"], perm, k)
    dy_row_c, dy_row_s = mx.quantize_rowwise(dYp, mx.RNE)
    dy_col_c, dy_col_s = mx.quantize_transposed(dYp, off, mx.RNE, sf_layout=mx.SF_BLOCKS)
    wd = fw["wd"]
    wdT_c, wdT_s = req(wd, np.arange(E + 1) * d, True, ROLE_WDOWN, mx.SF_ROWS)
    WdT = np.stack(mx.dequant_transposed(wdT_c, wdT_s, np.arange(E + 1) * d, F))   # [E, F, d]
    dH = gemm.grouped_nt(mx.dequant_rowwise(dy_row_c, dy_row_s), WdT, off).astype(np.float32)
    hq = fw["hq"]
    hT_c, hT_s = req(hq, off, True, ROLE_H, mx.SF_BLOCKS)
    HT = mx.dequant_transposed(hT_c, hT_s, off, F, mx.SF_BLOCKS)
    dYc = mx.dequant_transposed(dy_col_c, dy_col_s, off, d, mx.SF_BLOCKS)
    dW_down = gemm.wgrad(dYc, HT).astype(np.float32)
    dU = (dH * silu.dsilu_f32(fw["U"])).astype(np.float32)
    du_row_c, du_row_s = mx.quantize_rowwise(dU, mx.RNE)
    du_col_c, du_col_s = mx.quantize_transposed(dU, off, mx.RNE, sf_layout=mx.SF_BLOCKS)
    wu = fw["wu"]
    wuT_c, wuT_s = req(wu, np.arange(E + 1) * F, True, ROLE_WUP, mx.SF_ROWS)
    WuT = np.stack(mx.dequant_transposed(wuT_c, wuT_s, np.arange(E + 1) * F, d))   # [E, d, F]
    dXp = gemm.grouped_nt(mx.dequant_rowwise(du_row_c, du_row_s), WuT, off).astype(np.float32)
    xp = fw["xq_perm"]
    xT_c, xT_s = req(xp, off, False, ROLE_X, mx.SF_BLOCKS)
    XT = mx.dequant_transposed(xT_c, xT_s, off, d, mx.SF_BLOCKS)
    dUc = mx.dequant_transposed(du_col_c, du_col_s, off, F, mx.SF_BLOCKS)
    dW_up = gemm.wgrad(dUc, XT).astype(np.float32)
    dx = unpermute_sum(dXp, inv, T, k)
    dg = dgates(dy_bf16, fw["Yp"], inv, k)
    dlogits = route.route_backward(dg.astype(np.float32), fw["gates"], fw["idx"], E)
    return dict(dg=dg, dlogits=dlogits, dYp=dYp, dy_row=(dy_row_c, dy_row_s), dy_col=(dy_col_c, dy_col_s),
                wdT=(wdT_c, wdT_s), dH=dH, hT=(hT_c, hT_s), dW_down=dW_down, dU=dU,
                du_row=(du_row_c, du_row_s), du_col=(du_col_c, du_col_s), wuT=(wuT_c, wuT_s),
                dXp=dXp, xT=(xT_c, xT_s), dW_up=dW_up, dx=dx)


# ------------------------------------------------ MXFP8-forward variant
#
# The layers the pages keep at higher precision run their forward in MXFP8
# (agihunt.info page, "Confirmed": the last 16.6% of layers in MXFP8;
# lhc.media page: the final sixth of the layers), and full MXFP8 training is
# the pages' baseline (fourweekmba.com page, "Why the Gain Is 8%, Not 3x").
# Readings: x, the weights and H are quantised to MXFP8 with round to nearest
# even along the forward contraction (blocks of 32, no tensor scale); U is
# stored in bf16 as in the NVFP4 forward; the backward is the same, except
# that the requantisations read the MXFP8 forward operands.

def forward_mx(x_bf16, W_up, W_down, logits, k, bias=None):
    T, d = x_bf16.shape
    E, F, _ = W_up.shape
    wu_c, wu_s = mx.quantize_rowwise(W_up.reshape(E * F, d).astype(np.float32), mx.RNE)
    wd_c, wd_s = mx.quantize_rowwise(W_down.reshape(E * d, F).astype(np.float32), mx.RNE)
    idx, gates = route.topk_gates(logits, k, bias)
    P = route.permutation(idx, E)
    off, perm, inv = P["off"], P["perm"], P["inv_perm"]
    xf = fmt.bf16_to_f32(x_bf16)
    xp_c, xp_s = mx.quantize_rowwise(xf[perm.astype(np.int64) // k], mx.RNE)
    A64 = mx.dequant_rowwise(xp_c, xp_s)
    Bup = mx.dequant_rowwise(wu_c, wu_s).reshape(E, F, d)
    U = fmt.f64_to_bf16(gemm.grouped_nt(A64, Bup, off))
    H = silu.silu_f32(U)
    h_c, h_s = mx.quantize_rowwise(H, mx.RNE)
    Bdn = mx.dequant_rowwise(wd_c, wd_s).reshape(E, d, F)
    Yp = gemm.grouped_nt(mx.dequant_rowwise(h_c, h_s), Bdn, off).astype(np.float32)
    y = combine(Yp, gates, inv, k)
    mxq = lambda c, s_: dict(codes=c, sf=s_)
    return dict(wu=mxq(wu_c, wu_s), wd=mxq(wd_c, wd_s), idx=idx, gates=gates, perm=P, xq_perm=mxq(xp_c, xp_s),
                U=U, hq=mxq(h_c, h_s), Yp=Yp, y=y, dims=(T, d, F, E, k))


def backward_mx(fw, dy_bf16, seed=1, layer=0):
    """The backward of ``forward_mx``: as ``backward``, with the transposed
    SR requantisations reading MXFP8 forward operands."""
    def req(q, off, ts_per_group, role, layout):
        return mx.requant_mx_sr_t(q["codes"], q["sf"], off, seed, 16 * layer + role, layout)
    return _backward(fw, dy_bf16, req)

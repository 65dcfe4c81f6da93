"""The router in front of the expert layer: its BF16 GEMM and backward (test infrastructure).

The pages describe a mixture-of-experts model whose tokens each go to 8 of 384
experts (fourweekmba.com page, "Update") and keep some activations in BF16
(lhc.media page, paragraph on the precisions that remain); how the router
scores are made is not on the pages.  The plain reading taken here: a linear
router in BF16, logits = x . W_r^T with x [T, d] and W_r [E, d] both bf16 and
float32 results, whose gradients follow from the softmax backward of the gates
(route.route_backward), dz = dlogits [T, E] with non-zero entries only at each
token's k selected experts:

* forward: logits[t, e] = RN32(sum_c x[t, c] * W_r[e, c]), the exact sum of
  the bf16 products rounded once to float32 (the GPU accumulates in float32;
  the tolerance is the GEMM rule);
* input gradient: dx_r[t] = sum over the token's k selected experts e_j of
  dz[t, e_j] * W_r[e_j]; it joins the expert path's input gradient in the
  un-permuting sum, which in float32, one operation at a time, is
    acc = 0; for j = 0..k-1: acc = fl(acc + dXp[row(t, j)]);
    for j = 0..k-1: acc = fl(acc + fl(dz[t, e_j] * W_r[e_j, c]));
    dx[t, c] = bf16(acc)
  (bit-exact against the GPU);
* weight gradient: dW_r[e] = sum over the tokens routed to e of dz[t, e] * x[t]
  (float32 output of an exact sum; the GEMM tolerance rule).
"""
import numpy as np

from . import formats as fmt

F32 = np.float32


def logits(x_bf16, w_bf16):
    """[T, E] float32: RN32 of the exact sum of bf16 products."""
    x = fmt.bf16_to_f32(x_bf16).astype(np.float64)
    w = fmt.bf16_to_f32(w_bf16).astype(np.float64)
    return (x @ w.T).astype(np.float32)


def logits_abs_bound(x_bf16, w_bf16):
    """sum_c |x * w| per logit (the tolerance's scale)."""
    x = np.abs(fmt.bf16_to_f32(x_bf16).astype(np.float64))
    w = np.abs(fmt.bf16_to_f32(w_bf16).astype(np.float64))
    return x @ w.T


def unpermute_sum_router(dXp, inv, T, k, dlogits, idx, w_bf16):
    """dx[t] = bf16(sum_j dXp[row(t, j)] + sum_j dz[t, e_j] * W_r[e_j]) in the
    float32 order stated in the module docstring."""
    d = dXp.shape[1]
    inv = np.asarray(inv, dtype=np.int64).reshape(T, k)
    idx = np.asarray(idx, dtype=np.int64)
    w = fmt.bf16_to_f32(w_bf16)
    dl = np.asarray(dlogits, dtype=np.float32)
    acc = np.zeros((T, d), dtype=np.float32)
    for j in range(k):
        acc = (acc + dXp[inv[:, j]]).astype(np.float32)
    for j in range(k):
        dz = dl[np.arange(T), idx[:, j]][:, None]
        acc = (acc + (dz * w[idx[:, j]]).astype(np.float32)).astype(np.float32)
    return fmt.bf16_round(acc)


def weight_grad(x_bf16, dlogits, idx):
    """dW_r [E, d] float64: sum over the tokens routed to e of dz[t, e] * x[t]
    (exact: every product of a float32 and a bf16 is exact in float64, and the
    sums stay far inside its precision at these sizes)."""
    x = fmt.bf16_to_f32(x_bf16).astype(np.float64)
    dl = np.asarray(dlogits, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    E = dl.shape[1]
    out = np.zeros((E, x.shape[1]))
    for j in range(k):
        e = idx[:, j]
        np.add.at(out, e, dl[np.arange(T), e][:, None] * x)
    return out


def weight_grad_abs_bound(x_bf16, dlogits, idx):
    return weight_grad(np.asarray(x_bf16) & np.uint16(0x7FFF), np.abs(np.asarray(dlogits, np.float64)), idx)

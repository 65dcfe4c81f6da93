"""Top-k routing, gates and the stable expert permutation (test infrastructure).

The pages name the model's routing (fourweekmba.com page, "Update": each token
goes to 8 of 384 experts) and the dispatch of inputs to the experts that hold
them (lhc.media page, paragraph on communication).  The routing arithmetic is
not on the pages; the plain reading used here (Mixtral-style):

* z = fl(logit + bias) per expert (bias 0 when absent);
* the top-k set is the k largest z, listed in descending order, equal values
  ordered by the lower expert index;
* gates: w_j = RN32(exp(fl(z_j - z_0))) with the exponential evaluated in
  float64 and rounded once to float32; s = w_0 + w_1 + ... in float32, in
  order j = 0..k-1; g_j = fl(w_j / s).

Permutation: assignment a = t * k + j (token t, slot j).  Rows of the
expert-grouped matrices are ordered by (expert ascending, token ascending),
i.e. a stable counting sort of the assignments by expert.  off[e] is the
number of assignments to experts below e; off_pad[e] sums pad32 of the counts;
perm[row] = a and inv_perm[a] = row.

Router backward (not on the pages either; the derivative of the gates above):
the gates are a softmax of z over the selected set, so with dg[t, j] the
gradient of the loss in g[t, j], dz[t, e_j] = g_j * (dg_j - sum_i g_i * dg_i)
for the k selected experts e_j and 0 for the others (the top-k selection has
no gradient).  In float32, one operation at a time: s = 0; for i = 0..k-1:
s = fl(s + fl(g_i * dg_i)); dz_j = fl(g_j * fl(dg_j - s)).  Since z = logit +
bias, this is also the gradient in the logits.
"""
import numpy as np

F32 = np.float32


def topk_gates(logits, k, bias=None):
    """Returns (idx [T, k] int32, gates [T, k] float32) for logits [T, E] float32."""
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    z = logits if bias is None else (logits + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    idx = np.zeros((T, k), dtype=np.int32)
    gates = np.zeros((T, k), dtype=np.float32)
    for t in range(T):
        zt = z[t]
        order = sorted(range(E), key=lambda e: (-float(zt[e]), e))[:k]
        idx[t] = order
        zs = zt[order]
        w = np.array([F32(np.exp(np.float64(F32(zs[j] - zs[0])))) for j in range(k)], dtype=np.float32)
        s = F32(0.0)
        for j in range(k):
            s = F32(s + w[j])
        gates[t] = [F32(w[j] / s) for j in range(k)]
    return idx, gates


def permutation(idx, E):
    """Stable counting sort of assignments by expert.

    Returns dict(off [E+1], off_pad [E+1], perm [A], inv_perm [A]) as int32.
    """
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    A = T * k
    flat = idx.reshape(A)
    counts = np.zeros(E, dtype=np.int64)
    for a in range(A):
        counts[flat[a]] += 1
    off = np.zeros(E + 1, dtype=np.int64)
    off_pad = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        off[e + 1] = off[e] + counts[e]
        off_pad[e + 1] = off_pad[e] + (counts[e] + 31) // 32 * 32
    fill = off[:-1].copy()
    perm = np.zeros(A, dtype=np.int64)
    inv = np.zeros(A, dtype=np.int64)
    for a in range(A):
        e = flat[a]
        row = fill[e]
        fill[e] += 1
        perm[row] = a
        inv[a] = row
    return dict(off=off.astype(np.int32), off_pad=off_pad.astype(np.int32),
                perm=perm.astype(np.int32), inv_perm=inv.astype(np.int32))


def route_backward(dg, gates, idx, E):
    """dlogits [T, E] float32 from dg [T, k] (gradient in the gates), the
    forward's gates [T, k] and top-k indices idx [T, k]."""
    dg = np.asarray(dg, dtype=np.float32)
    gates = np.asarray(gates, dtype=np.float32)
    idx = np.asarray(idx, dtype=np.int64)
    T, k = gates.shape
    out = np.zeros((T, E), dtype=np.float32)
    for t in range(T):
        s = F32(0.0)
        for i in range(k):
            s = F32(s + F32(gates[t, i] * dg[t, i]))
        for j in range(k):
            out[t, idx[t, j]] = F32(gates[t, j] * F32(dg[t, j] - s))
    return out

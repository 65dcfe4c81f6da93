"""Expert-grouped GEMMs on exactly dequantised operands (test infrastructure).

Pages: agihunt.info page, "Confirmed" (NVFP4 in the expert layers' forward pass
with a dedicated kernel, MXFP8 in backpropagation); fourweekmba.com page, "Why
the Gain Is 8%, Not 3x" (the NVFP4 matrix multiplications of the
mixture-of-experts layers).

All GEMMs are "NT": both operands are stored with the contraction dimension
contiguous, C[m, n] = sum_k A[m, k] * B[n, k].  Operands are the exact real
values of the quantised codes (NVFP4: q * sc * S, MXFP8: code * 2**e), which
float64 holds exactly; the product is a float64 matmul, whose rounding
(about K * 2**-53 relative to sum |a*b|) is negligible at the 1e-3 tolerance.

* fwd:   C[rows of e] = A[rows of e] @ B[e].T         (rows grouped by off)
* dgrad: same shape rule as fwd (A rows grouped by off, B per expert)
* wgrad: dW[e] = A_e @ B_e.T where A_e [N1, P_e], B_e [N2, P_e] are expert e's
         transposed, padded operands (P_e = pad32(M_e)); empty experts give 0.
"""
import numpy as np


def grouped_nt(A64, B64_per_expert, off):
    """C [M_total, N] float64 for A [M_total, K] and B [E, N, K] float64."""
    off = np.asarray(off, dtype=np.int64)
    E = len(off) - 1
    M = A64.shape[0]
    N = B64_per_expert.shape[1]
    C = np.zeros((M, N), dtype=np.float64)
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        if r1 > r0:
            C[r0:r1] = A64[r0:r1] @ B64_per_expert[e].T
    return C


def wgrad(A_list, B_list):
    """dW [E, N1, N2] float64 from per-expert A_e [N1, P_e] and B_e [N2, P_e]."""
    E = len(A_list)
    N1 = A_list[0].shape[0]
    N2 = B_list[0].shape[0]
    out = np.zeros((E, N1, N2), dtype=np.float64)
    for e in range(E):
        if A_list[e].shape[1] > 0:
            out[e] = A_list[e] @ B_list[e].T
    return out


def abs_bound_nt(A64, B64_per_expert, off):
    """sum_k |A[m,k] * B[n,k]| per output element (the tolerance's scale)."""
    return grouped_nt(np.abs(A64), np.abs(B64_per_expert), off)

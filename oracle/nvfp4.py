"""Two-level NVFP4 quantisation with the Four-Over-Six choice (test infrastructure).

Pages: lhc.media page, paragraph on NVFP4 (4-bit values, one scale per sixteen
values, about 4.5 bits per value); agihunt.info page, "Confirmed" (activation
quantisation chooses between two scaling factors, "Four Over Six"); agihunt.info
post list ("per-expert scales").  The pages give no formulas; the steps below
are the plainest reading, with the choice rule fixed as: per 16-value block,
try the scale that maps the block's largest magnitude to 6 and the one that
maps it to 4, keep whichever leaves the lower squared error.

Layout: codes [R, C/2] uint8, element 2j of a row in the low nibble of byte j;
block scales [R, C/16] uint8 (E4M3); one float32 tensor scale per row group.

Steps (float32 arithmetic, one rounding per operation, written fl(.)):

1. tensor scale of a group: amax_g = max|x| over the group (exact);
   S = fl(amax_g / (m_max * 448)) with m_max = 4 in 4/6 mode, 6 in mode 6.
   If S == 0 the group is a zero group and S := 1.
2. per 16-block: amax_b = max|x_i|; for each candidate m (6, and 4 in 4/6 mode):
   d = fl(m * S); u = fl(amax_b / d); sc = e4m3(u).
3. encode under m: if sc == 0 or eff = fl(dec(sc) * S) == 0, every code is a
   signed zero; otherwise inv = fl(1 / eff) and q_i = e2m1(fl(x_i * inv)),
   where a zero x_i stays a zero of its own sign also when inv is infinite
   (eff below 2**-128; every nonzero x_i then saturates to +-6).
4. dequant: deq(q, sc, S) = fl(fl(dec(q) * dec(sc)) * S)  (the inner product
   is exact).
5. error: err = 0; for i = 0..15: t = fl(x_i - deq_i); err = fl(err + fl(t * t)).
6. choose m = 4 iff err_4 < err_6 (ties keep 6); mode 6 always takes m = 6.
"""
import numpy as np

from . import formats as fmt

F32 = np.float32
MODE_6 = 6
MODE_46 = 46
BLOCK = 16


def _as_f32(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:          # bf16 bit patterns
        return fmt.bf16_to_f32(x)
    return x.astype(np.float32)


def tensor_scale(x32, mode):
    """Step 1 for one group: returns the float32 tensor scale S."""
    amax = F32(np.max(np.abs(x32))) if x32.size else F32(0.0)
    m_max = F32(4.0) if mode == MODE_46 else F32(6.0)
    S = F32(amax / F32(m_max * F32(448.0)))
    if S == F32(0.0):
        S = F32(1.0)
    return S


def _encode_candidate(xb, S, m):
    """Steps 2-5 for candidate m on blocks xb [nb, 16] with per-block S [nb]."""
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        amax_b = np.max(np.abs(xb), axis=1).astype(np.float32)
        d = (F32(m) * S).astype(np.float32)
        u = (amax_b / d).astype(np.float32)
        sc = fmt.e4m3_round_mag(u.astype(np.float64))
        scv = fmt.e4m3_decode(sc).astype(np.float32)          # exact
        eff = (scv * S).astype(np.float32)
        zero = (sc == 0) | (eff == F32(0.0))
        safe_eff = np.where(zero, F32(1.0), eff).astype(np.float32)
        inv = (F32(1.0) / safe_eff).astype(np.float32)
        y = (xb * inv[:, None]).astype(np.float32)
        # an effective scale below 2**-128 has an infinite reciprocal: a zero
        # element then stays that zero, with its own sign (0 * inf is a NaN
        # whose sign the platform picks)
        y = np.where(xb == F32(0.0), xb, y).astype(np.float32)
        q = fmt.e2m1_round(y)
        sign_only = ((xb.view(np.uint32) >> 31).astype(np.int64)) << 3
        q = np.where(zero[:, None], sign_only, q)
        deq = dequant_values(q, sc[:, None], S[:, None])
        err = np.zeros(xb.shape[0], dtype=np.float32)
        for i in range(BLOCK):
            t = (xb[:, i] - deq[:, i]).astype(np.float32)
            err = (err + (t * t).astype(np.float32)).astype(np.float32)
    return q, sc, err


def dequant_values(q, sc, S):
    """Step 4: fl(fl(dec(q) * dec(sc)) * S) as float32 (broadcasting)."""
    p = (fmt.e2m1_decode(q) * fmt.e4m3_decode(sc)).astype(np.float32)   # exact
    return (p * np.asarray(S, dtype=np.float32)).astype(np.float32)


def quantize_blocks(x32, S_rows, mode):
    """Steps 2-6 on a float32 matrix [R, C] with per-row tensor scale S_rows [R].

    Returns (codes [R, C] int 0..15, block scales [R, C/16] int 0..126,
    chosen m per block [R, C/16]).
    """
    R, C = x32.shape
    assert C % BLOCK == 0
    nb = C // BLOCK
    xb = x32.reshape(R * nb, BLOCK)
    S = np.repeat(np.asarray(S_rows, dtype=np.float32), nb)
    q6, sc6, err6 = _encode_candidate(xb, S, 6)
    if mode == MODE_6:
        q, sc, m = q6, sc6, np.full(R * nb, 6)
    elif mode == MODE_46:
        q4, sc4, err4 = _encode_candidate(xb, S, 4)
        take4 = err4 < err6
        q = np.where(take4[:, None], q4, q6)
        sc = np.where(take4, sc4, sc6)
        m = np.where(take4, 4, 6)
    else:
        raise ValueError("mode must be 6 or 46")
    return q.reshape(R, C), sc.reshape(R, nb), m.reshape(R, nb)


def pack_codes(q):
    """[R, C] codes -> [R, C/2] bytes, element 2j in the low nibble of byte j."""
    q = np.asarray(q, dtype=np.int64)
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed):
    """[R, C/2] bytes -> [R, C] codes."""
    p = np.asarray(packed, dtype=np.int64)
    R, H = p.shape
    q = np.empty((R, 2 * H), dtype=np.int64)
    q[:, 0::2] = p & 15
    q[:, 1::2] = p >> 4
    return q


def group_rows(group_row_off, R):
    """Group index of every row for offsets [G+1] (None = one group)."""
    if group_row_off is None:
        return np.zeros(R, dtype=np.int64), 1
    off = np.asarray(group_row_off, dtype=np.int64)
    g = np.zeros(R, dtype=np.int64)
    for gi in range(len(off) - 1):
        g[off[gi]:off[gi + 1]] = gi
    return g, len(off) - 1


def nvfp4_quantize(x, mode, group_row_off=None):
    """NVFP4 quantisation of x [R, C] (float32 values or bf16 bit patterns).

    group_row_off: None (one group) or row offsets [G+1]; each group gets its
    own tensor scale.  Returns dict(codes [R, C/2] u8, sf [R, C/16] u8,
    ts [G] f32, choice [R, C/16] (4 or 6)).
    """
    x32 = _as_f32(x)
    R, C = x32.shape
    g, G = group_rows(group_row_off, R)
    ts = np.zeros(G, dtype=np.float32)
    off = [0, R] if group_row_off is None else list(np.asarray(group_row_off, dtype=np.int64))
    for gi in range(G):
        ts[gi] = tensor_scale(x32[off[gi]:off[gi + 1]], mode)
    q, sc, m = quantize_blocks(x32, ts[g], mode)
    return dict(codes=pack_codes(q), sf=sc.astype(np.uint8), ts=ts, choice=m)


def nvfp4_dequantize(codes, sf, ts, group_row_off=None):
    """Step 4 on a whole tensor: float32 [R, C]."""
    q = unpack_codes(codes)
    R, C = q.shape
    g, _ = group_rows(group_row_off, R)
    sc = np.repeat(np.asarray(sf, dtype=np.int64), BLOCK, axis=1)
    S = np.asarray(ts, dtype=np.float32)[g][:, None]
    return dequant_values(q, sc, S)


def nvfp4_exact_f64(codes, sf, ts, group_row_off=None):
    """Exact real value q * sc * S of every element, as float64 (GEMM operands)."""
    q = unpack_codes(codes)
    R, C = q.shape
    g, _ = group_rows(group_row_off, R)
    sc = np.repeat(np.asarray(sf, dtype=np.int64), BLOCK, axis=1)
    S = np.asarray(ts, dtype=np.float32).astype(np.float64)[g][:, None]
    return fmt.e2m1_decode(q) * fmt.e4m3_decode(sc) * S

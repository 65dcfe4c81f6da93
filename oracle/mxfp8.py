"""MXFP8 quantisation and the transposed stochastic-rounding requantisation.

Test infrastructure (see the package docstring).

Pages: lhc.media page, the paragraph on transposition (transposing regroups the
values that share a scale factor, and quantising again can change values and
bias gradients) and the paragraph after it (dequantise the forward values,
transpose at higher precision, requantise into MXFP8 with stochastic rounding
that picks the upper or lower neighbour according to distance, so that the
value is preserved on average); fourweekmba.com page, "What Thinking Machines
Changed" (MXFP8 backward with re-quantisation and stochastic rounding).
MXFP8 itself is taken as E4M3 elements with one E8M0 scale per 32 values.

MX block of 32 values v_i:
* scale exponent e: amax = max|v_i|; e = -127 if amax == 0, otherwise the least
  integer with amax <= 448 * 2**e, clamped to [-127, 127]; stored byte e + 127.
* w_i = v_i * 2**-e (an exact real, |w_i| <= 448).
* RNE: code = sign(w_i) | e4m3(|w_i|).
* SR: a = |w_i|; step = 2**-9 if a < 2**-6 else 2**(floor(log2 a) - 3);
  lo = floor(a / step) * step (the largest grid value <= a);
  F = floor((a - lo) / step * 2**16); round up to lo + step iff
  F + r_i >= 2**16, with r_i the element's 16-bit random word (srhash).

Transposed, grouped layout ("group-major padded"): for a source matrix [R, C]
whose rows are cut into groups by offsets off[G+1], group g contributes a block
[C][pad32(R_g)] (rows of the block run along the source rows), padded with
zeros that do not change amax and encode as 0x00.  Its scales are stored
either row-major, [C][pad32(R_g)/32] (SF_ROWS: a row of the block with its
blocks in order), or block-major, [pad32(R_g)/32][C] (SF_BLOCKS: for each
32-row block of the group, the scales of all C columns in column order).
Blocks of 32 run along the source rows and never straddle a group.  The groups
are stored one after another in group order, the scales of group g starting at
C * off_pad[g] / 32 in both arrangements.  The arrangement is storage only:
which scale belongs to which 32 values does not depend on it.
"""
import numpy as np

from . import formats as fmt
from . import nvfp4 as nv
from . import srhash

MX_BLOCK = 32
RNE = 0
SR = 1
SF_ROWS = "rows"
SF_BLOCKS = "blocks"


def mx_scale_exponent(amax):
    """Scale exponent e (int) of blocks with maximum magnitudes ``amax`` (float64)."""
    amax = np.asarray(amax, dtype=np.float64)
    e = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    mant, ex = np.frexp(amax[nz])          # amax = mant * 2**ex, mant in [0.5, 1)
    E = ex - 1                             # floor(log2 amax)
    frac = mant * 2.0                      # amax / 2**E in [1, 2)
    e_nz = np.where(frac <= 1.75, E - 8, E - 7)
    e[nz] = e_nz
    return np.clip(e, -127, 127)


def round_rne(w):
    """E4M3 codes of the exact scaled values w (float64, |w| <= 448)."""
    return fmt.e4m3_round_signed(w)


def round_sr(w, r16):
    """E4M3 codes of w (float64) under stochastic rounding with 16-bit words r16."""
    w = np.asarray(w, dtype=np.float64)
    a = np.abs(w)
    sign = np.signbit(w).astype(np.int64)
    step = np.empty(a.shape, dtype=np.float64)
    small = a < 2.0 ** -6
    step[small] = 2.0 ** -9
    mant, ex = np.frexp(a[~small])
    step[~small] = np.exp2((ex - 1) - 3.0)
    t = a / step
    lo = np.floor(t)
    F = np.floor((t - lo) * 65536.0).astype(np.int64)
    up = (F + np.asarray(r16, dtype=np.int64)) >= 65536
    mag = (lo + up) * step                  # an exact grid value <= 448
    return fmt.e4m3_round_mag(mag) | (sign << 7)


def quantize_blocks_rows(v, rnd, seed=0, stream_id=0, index=None):
    """MXFP8 of float32 values v [N, 32] (each row one block).

    ``index`` [N, 32] holds the 64-bit source element index of every value
    (needed for SR only; padding entries may hold anything).
    Returns (codes [N, 32] u8, scale bytes [N] u8).
    """
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    amax = np.max(np.abs(v), axis=1)
    e = mx_scale_exponent(amax)
    w = v * np.exp2(-e.astype(np.float64))[:, None]       # exact
    if rnd == RNE:
        codes = round_rne(w)
    elif rnd == SR:
        r16 = srhash.random16(seed, stream_id, index)
        codes = round_sr(w, r16)
    else:
        raise ValueError("rnd must be RNE (0) or SR (1)")
    return codes.astype(np.uint8), (e + 127).astype(np.uint8)


def quantize_rowwise(x32, rnd=RNE, seed=0, stream_id=0):
    """MXFP8 with blocks along the columns: x [R, C] -> codes [R, C], sf [R, C/32]."""
    x32 = np.asarray(x32, dtype=np.float32)
    R, C = x32.shape
    assert C % MX_BLOCK == 0
    nb = C // MX_BLOCK
    idx = np.arange(R * C, dtype=np.uint64).reshape(R * nb, MX_BLOCK)
    codes, sf = quantize_blocks_rows(x32.reshape(R * nb, MX_BLOCK), rnd, seed, stream_id, idx)
    return codes.reshape(R, C), sf.reshape(R, nb)


def pad32(n):
    return (int(n) + MX_BLOCK - 1) // MX_BLOCK * MX_BLOCK


def padded_offsets(group_row_off):
    off = np.asarray(group_row_off, dtype=np.int64)
    sizes = off[1:] - off[:-1]
    pads = np.array([pad32(s) for s in sizes], dtype=np.int64)
    return np.concatenate([[0], np.cumsum(pads)]).astype(np.int64)


def quantize_transposed(x32, group_row_off=None, rnd=RNE, seed=0, stream_id=0, sf_layout=SF_ROWS):
    """MXFP8 of x [R, C] with blocks along the rows, group-major padded layout.

    Returns codes (1-D, length C * off_pad[G]) and sf (1-D, length
    C * off_pad[G] / 32), group g's block starting at C * off_pad[g] (codes)
    and C * off_pad[g] / 32 (scales); codes row-major [C][pad32(R_g)], scales
    [C][pad32(R_g)/32] (SF_ROWS) or [pad32(R_g)/32][C] (SF_BLOCKS).
    """
    if sf_layout not in (SF_ROWS, SF_BLOCKS):
        raise ValueError("sf_layout must be SF_ROWS or SF_BLOCKS")
    x32 = np.asarray(x32, dtype=np.float32)
    R, C = x32.shape
    off = np.array([0, R], dtype=np.int64) if group_row_off is None else np.asarray(group_row_off, dtype=np.int64)
    offp = padded_offsets(off)
    codes = np.zeros(C * offp[-1], dtype=np.uint8)
    sf = np.zeros(C * offp[-1] // MX_BLOCK, dtype=np.uint8)
    for g in range(len(off) - 1):
        r0, r1 = off[g], off[g + 1]
        Rg = r1 - r0
        P = pad32(Rg)
        if P == 0:
            continue
        blk = np.zeros((C, P), dtype=np.float32)
        blk[:, :Rg] = x32[r0:r1].T
        # source index of element (r, c) is r * C + c; padding gets index 0 (unused: it is 0)
        rows = np.arange(P, dtype=np.uint64)
        src = (np.uint64(r0) + rows)[None, :] * np.uint64(C) + np.arange(C, dtype=np.uint64)[:, None]
        nb = P // MX_BLOCK
        c_, s_ = quantize_blocks_rows(blk.reshape(C * nb, MX_BLOCK), rnd, seed, stream_id,
                                      src.reshape(C * nb, MX_BLOCK))
        codes[C * offp[g]: C * offp[g + 1]] = c_.reshape(-1)
        s_ = s_.reshape(C, nb)
        sf[C * offp[g] // MX_BLOCK: C * offp[g + 1] // MX_BLOCK] = (s_ if sf_layout == SF_ROWS else s_.T).reshape(-1)
    return codes, sf


def requant_sr_t(codes, sf, ts, group_row_off=None, ts_per_group=True, seed=1, stream_id=0, sf_layout=SF_ROWS):
    """NVFP4 [R, C] -> dequantise (float32) -> transpose -> MXFP8 SR.

    ts: tensor scales, one per group if ``ts_per_group`` else one for all rows.
    Output layout as ``quantize_transposed`` (``sf_layout`` likewise).
    """
    q = nv.unpack_codes(codes)
    R, C = q.shape
    off = np.array([0, R], dtype=np.int64) if group_row_off is None else np.asarray(group_row_off, dtype=np.int64)
    G = len(off) - 1
    ts = np.asarray(ts, dtype=np.float32)
    ts_rows = np.empty(R, dtype=np.float32)
    for g in range(G):
        ts_rows[off[g]:off[g + 1]] = ts[g] if ts_per_group else ts[0]
    sc = np.repeat(np.asarray(sf, dtype=np.int64), nv.BLOCK, axis=1)
    v = nv.dequant_values(q, sc, ts_rows[:, None])
    return quantize_transposed(v, off, SR, seed, stream_id, sf_layout)


def requant_mx_sr_t(codes, sf, group_row_off=None, seed=1, stream_id=0, sf_layout=SF_ROWS):
    """MXFP8 row-wise [R, C] (codes, scales [R, C/32]) -> exact values ->
    transpose -> MXFP8 SR: the same requantisation for a forward operand that
    is itself MXFP8 (no tensor scale).  Output layout as ``quantize_transposed``."""
    v = dequant_rowwise(codes, sf).astype(np.float32)       # exact: E4M3 times a power of two
    R = v.shape[0]
    off = np.array([0, R], dtype=np.int64) if group_row_off is None else np.asarray(group_row_off, dtype=np.int64)
    return quantize_transposed(v, off, SR, seed, stream_id, sf_layout)


def dequant_rowwise(codes, sf):
    """Exact float64 values of row-wise MXFP8 [R, C]."""
    c = np.asarray(codes)
    R, C = c.shape
    s = np.repeat(fmt.e8m0_decode(sf), MX_BLOCK, axis=1)
    return fmt.e4m3_decode(c) * s


def dequant_transposed(codes, sf, group_row_off, C, sf_layout=SF_ROWS):
    """Exact float64 values of a group-major padded tensor: list of [C, pad32(R_g)]."""
    off = np.asarray(group_row_off, dtype=np.int64)
    offp = padded_offsets(off)
    out = []
    for g in range(len(off) - 1):
        P = offp[g + 1] - offp[g]
        c_ = np.asarray(codes[C * offp[g]: C * offp[g + 1]]).reshape(C, P)
        s_ = np.asarray(sf[C * offp[g] // MX_BLOCK: C * offp[g + 1] // MX_BLOCK])
        s_ = s_.reshape(C, P // MX_BLOCK) if sf_layout == SF_ROWS else s_.reshape(P // MX_BLOCK, C).T
        out.append(fmt.e4m3_decode(c_) * np.repeat(fmt.e8m0_decode(s_), MX_BLOCK, axis=1))
    return out

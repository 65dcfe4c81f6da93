"""Combine-path quantiser: block Hadamard transform + 8-bit fixed-point MX format.

Test infrastructure (see the package docstring).

Page: lhc.media page, the paragraph on communication between GPUs.  Expert
results travelling back for the combine first go through a Hadamard transform,
which spreads extreme values over the block.  They are then quantised to an
8-bit element format ("S2F6") with scale factors, for 8.25 bits per value
instead of 16.

Readings (the page gives only the name of the format and the bit count):
* Element.  "S2F6" is read as signed two's-complement fixed point with 2
  integer bits (sign included) and 6 fraction bits: value = c * 2**-6 for an
  int8 code c.  The grid is kept symmetric, c in [-127, 127] (-128 unused).
  This is the element of the OCP MX format MXINT8.
* Scale.  One E8M0 byte per 32 consecutive values of a row, which gives
  8 + 8/32 = 8.25 bits per value.  amax = max |y_i| over the block; the
  exponent is e = floor(log2 amax) (the element's largest power of two is
  2**0), e = -127 when amax == 0, clamped to [-127, 127].  The stored byte is
  e + 127.
* Codes.  c_i = clamp(rne(y_i * 2**(6 - e)), -127, 127), with rne = round to
  nearest, ties to even.  y_i * 2**(6 - e) is computed exactly.
* Transform.  The unnormalised 32-point Walsh-Hadamard transform in natural
  (Sylvester) order, H_32 with entries +-1, over the same 32-value blocks as
  the scale.  H_32 H_32 = 32 I, so the receiver applies H_32 once more and
  multiplies by 2**-5.
* Precision.  The sender's transform runs in float32 as five butterfly
  stages (a, b) -> (a + b, a - b), partner distance 1, 2, 4, 8, 16 in that
  order.  The rounding of these sums decides the codes, so both
  implementations take them the same way.  Decoding is exact: within a block
  every c * 2**(e - 6) shares one power of two, and every partial sum of the
  inverse transform is an integer below 2**12 times it.
* Combine.  The receiver decodes each row exactly, then sums the gated rows
  in slot order, as the plain combine does.
* Backward.  The backward treats the quantisation as the identity
  (straight-through): the gate gradient keeps using the float32 expert
  outputs.
* Inputs.  Finite values with |x| <= 2**122, so that the 32-term float32
  sums stay finite.
"""
import numpy as np

BLOCK = 32
CODE_MAX = 127
FRAC_BITS = 6


def fwht32_f32(x32):
    """Butterfly Walsh-Hadamard transform of every 32-value block of the last
    axis, float32, stages h = 1, 2, 4, 8, 16 (the order that fixes rounding)."""
    y = np.array(x32, dtype=np.float32, copy=True)
    assert y.shape[-1] % BLOCK == 0
    shp = y.shape
    y = y.reshape(-1, BLOCK)
    h = 1
    while h < BLOCK:
        for i in range(BLOCK):
            if i & h:
                continue
            a = y[:, i].copy()
            b = y[:, i + h].copy()
            y[:, i] = (a + b).astype(np.float32)
            y[:, i + h] = (a - b).astype(np.float32)
        h *= 2
    return y.reshape(shp)


def scale_exponent(amax):
    """e = floor(log2 amax), -127 for amax == 0, clamped to [-127, 127]."""
    amax = np.asarray(amax, dtype=np.float64)
    e = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    _, ex = np.frexp(amax[nz])  # amax = m * 2**ex, m in [0.5, 1)
    e[nz] = ex - 1
    return np.clip(e, -127, 127)


def quantize(x32):
    """x [R, C] float32, C % 32 == 0 -> (codes int8 [R, C], scales uint8 [R, C/32])."""
    x32 = np.asarray(x32, dtype=np.float32)
    R, C = x32.shape
    assert C % BLOCK == 0
    y = fwht32_f32(x32).reshape(R, C // BLOCK, BLOCK).astype(np.float64)
    e = scale_exponent(np.abs(y).max(axis=2))
    w = np.ldexp(y, (FRAC_BITS - e)[:, :, None])  # exact: scaling by a power of two
    c = np.clip(np.rint(w), -CODE_MAX, CODE_MAX).astype(np.int8)
    return c.reshape(R, C), (e + 127).astype(np.uint8)


def dequantize(codes, scales):
    """Exact decode: H_32 (c * 2**(e - 6)) * 2**-5 per block, float32 [R, C]."""
    c = np.asarray(codes, dtype=np.int8).astype(np.int64)
    R, C = c.shape
    e = np.asarray(scales, dtype=np.int64).reshape(R, C // BLOCK) - 127
    H = hadamard_matrix()
    blocks = c.reshape(R, C // BLOCK, BLOCK) @ H  # H symmetric; integer sums
    v = np.ldexp(blocks.astype(np.float64), (e - FRAC_BITS - 5)[:, :, None])
    out = v.astype(np.float32)
    assert np.array_equal(out.astype(np.float64), v)  # the decode is exact in float32
    return out.reshape(R, C)


def hadamard_matrix(n=BLOCK):
    """Sylvester H_n (entries +-1, int64): H_1 = [1], H_2m = [[H, H], [H, -H]]."""
    H = np.ones((1, 1), dtype=np.int64)
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def combine_payload(codes, scales, gates, inv, k):
    """y[t] = bf16(sum_j fl(g[t,j] * Yhat[row(t,j)])) in order j = 0..k-1, with
    Yhat the exact decode of the payload."""
    from .layer import combine
    return combine(dequantize(codes, scales), np.asarray(gates, dtype=np.float32), inv, k)


def payload_bits_per_value(C):
    """Bits sent per value for a row of C values: C code bytes + C/32 scale bytes."""
    return 8.0 * (C + C // BLOCK) / C


__all__ = ["fwht32_f32", "scale_exponent", "quantize", "dequantize", "hadamard_matrix", "combine_payload",
           "payload_bits_per_value"]

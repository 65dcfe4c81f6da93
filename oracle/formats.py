"""Element and scale codecs (test infrastructure; see the package docstring).

Formats named on the pages (lhc.media page, paragraph on NVFP4's 4-bit values
sharing one scale per sixteen values; agentbuildlog.com page, "What 4-bit
training means here", for NVFP4 and MXFP8) and fixed here by their public
definitions:

* E2M1 (FP4): sign, 2 exponent bits (bias 1), 1 mantissa bit.  Magnitudes of
  codes 0..7 are {0, 0.5, 1, 1.5, 2, 3, 4, 6}; code 8 is -0.
* E4M3 (FN variant): sign, 4 exponent bits (bias 7), 3 mantissa bits;
  subnormals m * 2**-9; largest finite 448 (code 0x7E); 0x7F / 0xFF are NaN and
  never produced; no infinities.
* E8M0: an unsigned exponent, value 2**(c - 127) for c in 0..254; 255 is NaN
  and never produced.
* BF16: binary32 rounded to 8 significant bits, ties to even.

Rounding rules (readings, since the pages name the formats without defining
their rounding):

* ``e2m1_round``: round to nearest, ties to the even code, saturate at 6; the
  sign bit of the result is the sign bit of the input (so small negatives give
  -0, code 8); +-inf saturates to +-6, and a NaN input encodes as a zero
  with the NaN's sign bit (the NVFP4 encoder passes none: a zero element
  under an infinite reciprocal scale stays that zero).
* ``e4m3_round_mag``: for u >= 0, round to nearest on the E4M3 grid, ties to the
  even code, values above 448 clamp to 448.
"""
import numpy as np

F32 = np.float32

E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def e2m1_decode(codes):
    """Exact value of 4-bit E2M1 codes (array of ints 0..15) as float64."""
    c = np.asarray(codes).astype(np.int64)
    mag = E2M1_MAG[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def e4m3_decode(codes):
    """Exact value of E4M3FN byte codes as float64 (NaN for 0x7F/0xFF)."""
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e8m0_decode(codes):
    """Exact value of E8M0 byte codes as float64 (NaN for 255)."""
    c = np.asarray(codes).astype(np.int64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def _sign_bit(x32):
    return (np.asarray(x32, dtype=np.float32).view(np.uint32) >> 31).astype(np.int64)


def e2m1_round(v):
    """E2M1 code (0..15) of float32 values ``v``: RNE, saturate at 6, keep sign.

    Grid spacing is 0.5 on [0, 2), 1 on [2, 4) and 2 on [4, 6]; on each piece
    the nearest grid point is taken and an exact half-way value goes to the
    neighbour with the even code.
    """
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v).astype(np.float64)            # exact
    sign = _sign_bit(v)
    # +-inf saturates to +-6; a NaN encodes as a zero with its sign bit
    a = np.where(np.isnan(a), 0.0, np.minimum(a, 6.0))
    step = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    base = np.where(a < 2.0, 0.0, np.where(a < 4.0, 2.0, 4.0))
    base_code = np.where(a < 2.0, 0, np.where(a < 4.0, 4, 6))
    t = (a - base) / step                       # exact: power-of-two step
    lo = np.floor(t)
    rem = t - lo
    code = base_code + lo.astype(np.int64)
    up = (rem > 0.5) | ((rem == 0.5) & ((code & 1) == 1))
    code = code + up.astype(np.int64)
    code = np.minimum(code, 7)                  # a >= 6 (and 5 < a < 6 rounding up) -> 6
    return (code | (sign << 3)).astype(np.int64)


def e4m3_round_mag(u):
    """E4M3 code (0..126) of non-negative float32 ``u``: RNE, clamp to 448.

    Below 2**-6 the grid is the subnormal grid m * 2**-9; from 2**-6 upward a
    value in [2**E, 2**(E+1)) sits on a grid of step 2**(E-3).  Ties go to the
    even code (the even mantissa).
    """
    u = np.asarray(u, dtype=np.float64)
    if np.any(u < 0) or np.any(np.isnan(u)):
        raise ValueError("e4m3_round_mag takes non-negative finite values")
    out = np.empty(u.shape, dtype=np.int64)
    big = u >= 448.0
    out[big] = 126
    small = u < 2.0 ** -6
    # subnormal region: value = m * 2**-9, m in 0..8 (m = 8 is the first normal)
    t = u[small] * 2.0 ** 9
    lo = np.floor(t)
    rem = t - lo
    m = lo.astype(np.int64) + ((rem > 0.5) | ((rem == 0.5) & ((lo.astype(np.int64) & 1) == 1)))
    out[small] = m                               # m = 8 is code 8 = 2**-6, consistent
    mid = ~big & ~small
    um = u[mid]
    mant, ex = np.frexp(um)                      # um = mant * 2**ex, mant in [0.5, 1)
    E = ex - 1                                   # um in [2**E, 2**(E+1))
    t = um / np.exp2(E - 3.0)                    # in [8, 16), exact
    lo = np.floor(t)
    rem = t - lo
    lo_i = lo.astype(np.int64)
    up = (rem > 0.5) | ((rem == 0.5) & ((lo_i & 1) == 1))
    sig = lo_i + up                              # 8..16
    E2 = np.where(sig == 16, E + 1, E)
    sig = np.where(sig == 16, 8, sig)
    code = ((E2 + 7) << 3) | (sig - 8)
    out[mid] = np.minimum(code, 126)
    return out


def e4m3_round_signed(v):
    """E4M3 code of signed float values: sign bit | e4m3_round_mag(|v|)."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.int64)
    return e4m3_round_mag(np.abs(v)) | (sign << 7)


def bf16_round(x32):
    """Round float32 values to bfloat16 (ties to even); returns uint16 bit patterns."""
    b = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = (b + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(bits16):
    """Exact float32 value of bfloat16 bit patterns."""
    return (np.asarray(bits16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f64_to_bf16(x64):
    """Round float64 values to bfloat16 once (ties to even); returns uint16 bits.

    Used where the method rounds an exact (float64) result straight to bf16,
    e.g. a GEMM output; rounding through float32 first could double-round.
    """
    x = np.asarray(x64, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.uint16)
    sign = np.signbit(x)
    a = np.abs(x)
    nz = a > 0
    mant, ex = np.frexp(a[nz])                    # a = mant * 2**ex, mant in [0.5, 1)
    E = ex - 1
    E = np.maximum(E, -126)                       # bf16 subnormals share the 2**-126 grid
    step = np.exp2(E - 7.0)
    t = a[nz] / step
    lo = np.floor(t)
    rem = t - lo
    lo_i = lo.astype(np.int64)
    up = (rem > 0.5) | ((rem == 0.5) & ((lo_i & 1) == 1))
    val = (lo_i + up) * step                      # exact in float64
    val32 = val.astype(np.float32)                # exact: val is a bf16 value
    bits = (val32.view(np.uint32) >> 16).astype(np.uint16)
    out[nz] = bits
    out = np.where(sign, out | np.uint16(0x8000), out)
    return out.astype(np.uint16)

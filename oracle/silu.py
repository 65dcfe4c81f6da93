"""Correctly rounded SiLU and SiLU' over every bf16 input (test infrastructure).

The pages keep some activations in BF16 (lhc.media page, paragraph on the
precisions that remain); the expert MLP's activation is SiLU (a reading: the
pages do not name it).  The up-projection output U is stored as bf16, and the
activation is evaluated from it as correctly rounded float32 values:

    silu(u)  = RN32(u / (1 + exp(-u)))
    dsilu(u) = RN32(s * (1 + u * (1 - s)))   with s = 1 / (1 + exp(-u))

Each entry is evaluated in float64 and certified: if the float64 value lies
closer than 1e-13 (relative) to a float32 rounding boundary, the entry is
re-evaluated with ``decimal`` at 60 digits.
"""
import decimal

import numpy as np

from . import formats as fmt

_MARGIN = 1e-13


def _silu_f64(u):
    with np.errstate(over="ignore"):
        return u / (1.0 + np.exp(-u))


def _dsilu_f64(u):
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-u))
    return s * (1.0 + u * (1.0 - s))


def _boundary_distance(x64):
    """Relative distance of x64 to the nearest float32 rounding boundary."""
    x = np.asarray(x64, dtype=np.float64)
    a = np.abs(x)
    out = np.full(x.shape, np.inf)
    nz = (a > 0) & np.isfinite(a)
    mant, ex = np.frexp(a[nz])
    E = np.maximum(ex - 1, -126)
    ulp = np.exp2(E - 23.0)
    t = a[nz] / ulp
    dist = np.abs(t - np.floor(t) - 0.5) * ulp
    out[nz] = dist / a[nz]
    return out


def _dec_silu(u, prec=60):
    with decimal.localcontext() as ctx:
        ctx.prec = prec
        d = decimal.Decimal(float(u))
        return d / (1 + (-d).exp())


def _dec_dsilu(u, prec=60):
    with decimal.localcontext() as ctx:
        ctx.prec = prec
        d = decimal.Decimal(float(u))
        s = 1 / (1 + (-d).exp())
        return s * (1 + d * (1 - s))


def _dec_to_f32(dval):
    """Round a Decimal to float32 (ties to even) via exact rational arithmetic."""
    from fractions import Fraction
    fr = Fraction(dval)
    if fr == 0:
        return np.float32(0.0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    E = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** E > a:
        E -= 1
    E = max(E, -126)
    ulp = Fraction(2) ** (E - 23)
    t = a / ulp
    lo = t.numerator // t.denominator
    rem = t - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return np.float32(sign * float(lo * ulp))


_TABLES = None


def tables():
    """(u_bits [n] uint16, silu [n] float32, dsilu [n] float32) over finite bf16 u."""
    global _TABLES
    if _TABLES is None:
        bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        u32 = fmt.bf16_to_f32(bits)
        fin = np.isfinite(u32)
        bits = bits[fin]
        u = u32[fin].astype(np.float64)
        s64 = _silu_f64(u)
        d64 = _dsilu_f64(u)
        s32 = s64.astype(np.float32)
        d32 = d64.astype(np.float32)
        for arr64, arr32, dec in ((s64, s32, _dec_silu), (d64, d32, _dec_dsilu)):
            bad = np.nonzero(_boundary_distance(arr64) < _MARGIN)[0]
            for i in bad:
                arr32[i] = _dec_to_f32(dec(u[i]))
        _TABLES = (bits, s32, d32)
    return _TABLES


def silu_f32(u_bits):
    """Correctly rounded silu of bf16 bit patterns -> float32."""
    bits, s32, _ = tables()
    lut = np.zeros(65536, dtype=np.float32)
    lut[bits] = s32
    return lut[np.asarray(u_bits, dtype=np.uint16)]


def dsilu_f32(u_bits):
    """Correctly rounded silu' of bf16 bit patterns -> float32."""
    bits, _, d32 = tables()
    lut = np.zeros(65536, dtype=np.float32)
    lut[bits] = d32
    return lut[np.asarray(u_bits, dtype=np.uint16)]

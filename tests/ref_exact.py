"""Exact re-derivation of the method on tiny inputs, for pinning the oracle.

Written independently of ``oracle/``: values are Python ``Fraction``s, the
square root is a 60-digit ``decimal``, and every rounding is a nearest-point
search over the target format's code points (all of them for e4m3fn and
e2m1, the handful of neighbours of a float estimate for bf16 and fp32) with
ties going to the code whose last bit is 0 (the even mantissa).
"""
from __future__ import annotations

import decimal
import struct
from fractions import Fraction as F

import numpy as np

decimal.getcontext().prec = 60


# ------------------------------------------------------------ code points --
def bf16_value(bits: int) -> F:
    """Exact value of a finite bf16 bit pattern (sign, 8-bit exponent, 7-bit mantissa)."""
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    assert e != 0xFF
    if e == 0:
        return sign * F(m, 1) * F(2) ** (-126 - 7)
    return sign * F(128 + m) * F(2) ** (e - 127 - 7)


def f32_value(bits: int) -> F:
    sign = -1 if bits & 0x80000000 else 1
    e = (bits >> 23) & 0xFF
    m = bits & 0x7FFFFF
    assert e != 0xFF
    if e == 0:
        return sign * F(m) * F(2) ** (-126 - 23)
    return sign * F((1 << 23) + m) * F(2) ** (e - 127 - 23)


def _e4m3_magnitudes():
    out = []
    for c in range(0x7F):                    # 0x7F is NaN
        e, m = c >> 3, c & 7
        out.append(F(m, 8) * F(2) ** -6 if e == 0 else F(8 + m, 8) * F(2) ** (e - 7))
    return out


E4M3_MAG = _e4m3_magnitudes()                # codes 0x00..0x7E, increasing
E2M1_MAG = [F(0), F(1, 2), F(1), F(3, 2), F(2), F(3), F(4), F(6)]


def nearest_code(a: F, mags) -> int:
    """Index of the magnitude nearest to a >= 0; ties to the even index.
    Beyond the largest magnitude the largest wins (saturation)."""
    best, bestd = None, None
    for i, g in enumerate(mags):
        d = abs(a - g)
        if bestd is None or d < bestd or (d == bestd and i % 2 == 0):
            best, bestd = i, d
    return best


def _nearest_by_neighbours(a: F, est_bits: int, value_of, lo: int, hi: int) -> int:
    best, bestd = None, None
    for b in range(max(lo, est_bits - 3), min(hi, est_bits + 3) + 1):
        d = abs(a - value_of(b))
        if bestd is None or d < bestd or (d == bestd and b % 2 == 0):
            best, bestd = b, d
    return best


def bf16_round(v: F, negative_zero: bool = False) -> int:
    """bf16 bits nearest to the exact value v (finite range assumed)."""
    sign = 0x8000 if (v < 0 or (v == 0 and negative_zero)) else 0
    a = abs(v)
    est = struct.unpack("<I", struct.pack("<f", float(a)))[0] >> 16
    return sign | _nearest_by_neighbours(a, est, bf16_value, 0, 0x7F7F)


def f32_round(v: F) -> int:
    a = abs(v)
    est = struct.unpack("<I", struct.pack("<f", float(a)))[0]
    return (0x80000000 if v < 0 else 0) | _nearest_by_neighbours(a, est, f32_value, 0, 0x7F7FFFFF)


def f32_from_bits(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", bits))[0]


# --------------------------------------------------------------- pipeline --
def _sqrt_fraction(d: F) -> decimal.Decimal:
    return (decimal.Decimal(d.numerator) / decimal.Decimal(d.denominator)).sqrt()


def _dec_to_fraction(x: decimal.Decimal) -> F:
    return F(x)


def reference_row(x_bits, r_bits, g_bits, eps: float, group: int, fmt: int):
    """Exact result for one row. Returns (h_bits | None, yb_bits, scales, codes)
    where scales are fp32 bit patterns (FP8) or e8m0 bytes (MXFP4) and codes
    are one code per element (unpacked). Raises if the decimal evaluation
    cannot decide a bf16 rounding (a value within 1e-45 of a midpoint)."""
    N = len(x_bits)
    h_bits = []
    hv = []
    for j in range(N):
        xv = bf16_value(int(x_bits[j]))
        if r_bits is None:
            h_bits.append(int(x_bits[j]))
            hv.append(xv)
        else:
            s = xv + bf16_value(int(r_bits[j]))
            negz = s == 0 and (x_bits[j] & 0x8000) and (r_bits[j] & 0x8000)
            b = bf16_round(s, bool(negz))
            h_bits.append(b)
            hv.append(bf16_value(b))
    ss = sum((v * v for v in hv), F(0))
    eps_exact = F(float(np.float32(eps)))
    d = ss / N + eps_exact
    inv = decimal.Decimal(1) / _sqrt_fraction(d) if d > 0 else decimal.Decimal(0)
    yb = []
    for j in range(N):
        g = bf16_value(int(g_bits[j]))
        yd = (decimal.Decimal(hv[j].numerator) / decimal.Decimal(hv[j].denominator)) \
            * (decimal.Decimal(g.numerator) / decimal.Decimal(g.denominator)) * inv
        y = _dec_to_fraction(yd)
        b = bf16_round(y, negative_zero=(y == 0 and ((h_bits[j] ^ int(g_bits[j])) & 0x8000) != 0))
        # decidability: the decimal value must not sit on a rounding midpoint
        if y != 0:
            lo = bf16_value(b & 0x7FFF)
            for nb in ((b & 0x7FFF) - 1, (b & 0x7FFF) + 1):
                if 0 <= nb <= 0x7F7F:
                    mid = (lo + bf16_value(nb)) / 2
                    assert abs(abs(y) - mid) > abs(y) * F(1, 10 ** 45), "undecidable bf16 rounding"
        yb.append(b)
    scales, codes = [], []
    for g0 in range(0, N, group):
        vals = [bf16_value(b) for b in yb[g0:g0 + group]]
        amax = max(abs(v) for v in vals)
        if fmt == 0:
            sbits = 0x3F800000 if amax == 0 else f32_round(amax / 448)
            s = f32_value(sbits)
            scales.append(sbits)
            for b, v in zip(yb[g0:g0 + group], vals):
                c = nearest_code(abs(v) / s, E4M3_MAG)
                codes.append(c | (0x80 if b & 0x8000 else 0))
        else:
            if amax == 0:
                e = 0
            else:
                e = -200
                while not (F(2) ** (e + 2) <= amax < F(2) ** (e + 3)):
                    e += 1
                e = max(-127, min(127, e))
            scales.append(e + 127)
            for b, v in zip(yb[g0:g0 + group], vals):
                c = nearest_code(abs(v) / F(2) ** e, E2M1_MAG)
                codes.append(c | (0x8 if b & 0x8000 else 0))
    return (h_bits if r_bits is not None else None), yb, scales, codes

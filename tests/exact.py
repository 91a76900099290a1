"""Exact-arithmetic references for pinning the oracle's floating point.

Rational arithmetic (``fractions.Fraction``) plus an explicit round-to-nearest-even into
the IEEE binary32 / binary64 grids.  Nothing here uses the host's float operations for the
quantities it checks, so it pins the oracle's fp32/fp64 operation order independently of
the C compiler (a reciprocal instead of a division, a fused multiply-add, a single- instead
of double-precision scale, a different rounding mode would all show up).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def _rne(q: Fraction, mant_bits: int, emin: int) -> Fraction:
    """Round q to the nearest value with ``mant_bits`` significand bits (ties to even)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = -q if q < 0 else q
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)                     # subnormal range keeps the minimum exponent
    ulp = Fraction(2) ** (e - (mant_bits - 1))
    scaled = a / ulp
    fl = scaled.numerator // scaled.denominator
    rem = scaled - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def rne32(q: Fraction) -> Fraction:
    return _rne(q, 24, -126)


def rne64(q: Fraction) -> Fraction:
    return _rne(q, 53, -1022)


def fr(v) -> Fraction:
    """Exact rational value of a float (fp32 or fp64)."""
    return Fraction(float(v))


def round_half_even_int(q: Fraction) -> int:
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return int(fl)


def absmean_exact(w: np.ndarray) -> Fraction:
    """alpha = mean|W| computed exactly, then rounded once to fp32."""
    s = sum((abs(fr(v)) for v in np.asarray(w, np.float32).reshape(-1)), Fraction(0))
    return rne32(s / w.size)


def codes_exact(w: np.ndarray, alpha: Fraction) -> np.ndarray:
    """clip(round_half_even(fp32(W / alpha)), -1, 1) with an exact fp32 division."""
    out = np.zeros(np.asarray(w).shape, np.int8).reshape(-1)
    for i, v in enumerate(np.asarray(w, np.float32).reshape(-1)):
        if alpha == 0:
            out[i] = 0
            continue
        q = rne32(fr(v) / alpha)
        out[i] = max(-1, min(1, round_half_even_int(q)))
    return out.reshape(np.asarray(w).shape)


def quantize_act_exact(x: np.ndarray):
    """Per-token beta = fp32(max|x| + fp32(1e-8)); x_q = clip(rne(fp32(fp32(127*x)/beta)))."""
    x = np.asarray(x, np.float32)
    eps = rne32(Fraction(1, 10 ** 8))
    xq = np.zeros(x.shape, np.int8)
    beta = []
    for m in range(x.shape[0]):
        mx = max(abs(fr(v)) for v in x[m])
        b = rne32(mx + eps)
        beta.append(b)
        for j, v in enumerate(x[m]):
            t = rne32(rne32(fr(v) * 127) / b)
            xq[m, j] = max(-127, min(127, round_half_even_int(t)))
    return xq, beta


def dequant_scale_exact(alpha: Fraction, beta: Fraction) -> Fraction:
    """fp32(fp64(fp64(alpha*beta) / 127))."""
    return rne32(rne64(rne64(alpha * beta) / 127))


def dequant_exact(acc: np.ndarray, beta, alpha: Fraction) -> np.ndarray:
    y = np.zeros(acc.shape, np.float32)
    for m in range(acc.shape[0]):
        s = dequant_scale_exact(alpha, beta[m])
        for n in range(acc.shape[1]):
            y[m, n] = float(rne32(Fraction(int(acc[m, n])) * s))
    return y

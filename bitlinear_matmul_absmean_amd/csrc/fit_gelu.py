"""Coefficients of the fast fp64 GELU in common.hpp (gelu_approx), and its measured error.

erfcx(y) = exp(y^2) erfc(y) is interpolated at 17 Chebyshev points of t = 2 / (2 + y) over
y in [0, 5.7] (t in [2 / 7.7, 1]), in long double with the C library's erfcl and expl, and the
interpolant is written as a polynomial in u = S t + O, u in [-1, 1].  The script then evaluates
the fp64 path the kernels take (u clamped at -1, erfc = exp(-v^2 / 2) erfcx, Phi from erfc,
GELU = v Phi) over a dense grid and random fp32 inputs with v >= -4 and prints the largest
relative error against GELU in long double; the kernels' rounding test assumes it stays below
6e-14.

    python bitlinear_matmul_absmean_amd/csrc/fit_gelu.py
"""
import ctypes

import numpy as np

LD = np.longdouble
DEGREE = 16
Y_MAX = 5.7

_m = ctypes.CDLL("libm.so.6")
for _name in ("erfcl", "expl"):
    getattr(_m, _name).restype = ctypes.c_longdouble
    getattr(_m, _name).argtypes = [ctypes.c_longdouble]


def erfcx_ld(y):
    return np.array([_m.expl(LD(v) * LD(v)) * _m.erfcl(LD(v)) for v in np.atleast_1d(y)], dtype=LD)


def fit(degree=DEGREE, y_max=Y_MAX):
    """Monomial coefficients in u (constant first), and S, O with u = S t + O."""
    t0 = LD(2) / (LD(2) + LD(y_max))
    c, h = (t0 + 1) / 2, (1 - t0) / 2
    n = degree + 1
    k = np.arange(n, dtype=LD)
    theta = LD(np.pi) * (k + LD(0.5)) / n
    u = np.cos(theta)
    t = c + h * u
    f = erfcx_ld(LD(2) / t - LD(2))
    cheb = np.array([LD(2) / n * np.sum(f * np.cos(j * theta)) for j in range(n)], dtype=LD)
    cheb[0] /= 2
    # Chebyshev series -> monomials in u, by the recurrence T_{j+1} = 2 u T_j - T_{j-1}
    mono = np.zeros(n, dtype=LD)
    t_prev, t_cur = np.zeros(n, dtype=LD), np.zeros(n, dtype=LD)
    t_prev[0], t_cur[1] = 1, 1
    mono += cheb[0] * t_prev + cheb[1] * t_cur
    for j in range(2, n):
        t_next = np.zeros(n, dtype=LD)
        t_next[1:] = 2 * t_cur[:-1]
        t_next -= t_prev
        mono += cheb[j] * t_next
        t_prev, t_cur = t_cur, t_next
    return mono.astype(np.float64), float(1 / h), float(-c / h)


def gelu_fast(v, coef, s, o):
    """The kernels' fp64 evaluation (a division stands in for rcp + two Newton steps)."""
    v = v.astype(np.float64)
    y = np.abs(v) * 0.70710678118654752440
    u = np.maximum((2.0 / (2.0 + y)) * s + o, -1.0)
    e = np.full_like(u, coef[-1])
    for c in coef[-2::-1]:
        e = e * u + c
    q = np.exp(-0.5 * v * v) * e
    return v * np.where(v < 0, 0.5 * q, 1.0 - 0.5 * q)


def gelu_ld(v):
    return np.array([LD(0.5) * LD(x) * _m.erfcl(-LD(x) / np.sqrt(LD(2))) for x in v], dtype=LD)


def main():
    coef, s, o = fit()
    print(f"S2 = 2 * {s!r}, O = {o!r}")
    for c in coef:
        print(f"    {float(c)!r},")
    rng = np.random.default_rng(0)
    v = np.concatenate([np.linspace(-4.0, 12.0, 200_001), rng.uniform(-4.0, 12.0, 200_000),
                        rng.normal(0.0, 1.0, 100_000)]).astype(np.float32)
    v = v[(v >= -4.0) & (v != 0.0)]
    exact = gelu_ld(v)
    rel = np.abs((gelu_fast(v, coef, s, o).astype(LD) - exact) / exact).astype(np.float64)
    print(f"max relative error over {v.size} inputs in [-4, 12]: {rel.max():.3e} at v = {v[rel.argmax()]!r}")


if __name__ == "__main__":
    main()

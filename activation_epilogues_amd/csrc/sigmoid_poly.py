"""Coefficients of the polynomial the softmax+sigmoid epilogues use for
sigmoid(p) = 1 / (1 + exp(-p)) on p in [0, 1] (p is a softmax probability).

sigmoid(p) - 1/2 is odd in p, so on [-1, 1] it is approximated by an odd
polynomial, p * (r0 + r1 p^2 + r2 p^4 + r3 p^6).  Method: the Chebyshev
series of sigmoid(p) - 1/2 on [-1, 1] (coefficients from a high-degree
Chebyshev interpolant), truncated after T7 (its even terms are zero),
converted to the monomial basis and rounded to float32.  The kernels evaluate
1/2 + p * R(p^2) with Horner's rule in p^2: one multiply and four FMAs.  This
prints r0 .. r3 and the largest error of that float32 evaluation on a dense
grid of [0, 1] against the float64 definition (about 1.1e-7, two units in the
last place of results in [0.5, 0.74]):

    python activation_epilogues_amd/csrc/sigmoid_poly.py
"""
import numpy as np
from numpy.polynomial import chebyshev as cheb

TERMS = 4  # odd monomials p, p^3, p^5, p^7


def sigmoid(p):
    return 1.0 / (1.0 + np.exp(-p))


def coefficients(terms: int = TERMS) -> np.ndarray:
    series = cheb.chebinterpolate(lambda t: sigmoid(t) - 0.5, 64)  # Chebyshev series, to rounding
    kept = series[: 2 * terms].copy()
    kept[0::2] = 0.0                       # an odd function: the even terms vanish
    mono = cheb.cheb2poly(kept)            # coefficients of p^0 .. p^(2 terms - 1)
    return mono[1::2].astype(np.float32)   # r_k multiplies p^(2k + 1)


def eval32(r: np.ndarray, p: np.ndarray) -> np.ndarray:
    """1/2 + p * R(p^2) in float32, as the kernels compute it."""
    u = (p * p).astype(np.float32)
    acc = np.full_like(p, r[-1])
    for a in r[-2::-1]:
        acc = (acc * u + a).astype(np.float32)
    return (acc * p + np.float32(0.5)).astype(np.float32)


if __name__ == "__main__":
    r = coefficients()
    grid = np.linspace(0.0, 1.0, 400001).astype(np.float32)
    err = np.abs(eval32(r, grid).astype(np.float64) - sigmoid(grid.astype(np.float64))).max()
    for i, a in enumerate(r):
        print(f"r{i} = {float(a):.9e}f")
    print(f"max |error| of the float32 evaluation on [0, 1]: {err:.3e}")

"""Coefficients of the polynomial the softmax+sigmoid epilogue uses for
sigmoid(p) = 1 / (1 + exp(-p)) on p in [0, 1] (p is a softmax probability).

Method: Chebyshev interpolation of degree 6 at the 7 Chebyshev points of
[0, 1], converted to the monomial basis in p and rounded to float32; the
kernel evaluates it with Horner's rule.  This prints the coefficients (c0 ..
c6) and the largest error of a float32 Horner evaluation on a dense grid of
[0, 1] against the float64 definition (about 7e-8):

    python activation_epilogues_amd/csrc/sigmoid_poly.py
"""
import numpy as np
from numpy.polynomial import chebyshev as cheb
from numpy.polynomial import polynomial as poly

DEG = 6


def sigmoid(p):
    return 1.0 / (1.0 + np.exp(-p))


def coefficients(deg: int = DEG) -> np.ndarray:
    k = np.arange(deg + 1)
    t = np.cos((2 * k + 1) * np.pi / (2 * (deg + 1)))  # Chebyshev points of [-1, 1]
    c = cheb.chebfit(t, sigmoid((t + 1) / 2), deg)      # interpolant in t = 2p - 1
    in_t = cheb.cheb2poly(c)
    in_p = np.zeros(deg + 1)
    for i, a in enumerate(in_t):
        in_p[: i + 1] += a * poly.polypow([-1.0, 2.0], i)
    return in_p.astype(np.float32)


def horner32(c: np.ndarray, p: np.ndarray) -> np.ndarray:
    acc = np.full_like(p, c[-1])
    for a in c[-2::-1]:
        acc = (acc * p + a).astype(np.float32)
    return acc


if __name__ == "__main__":
    c = coefficients()
    grid = np.linspace(0.0, 1.0, 400001).astype(np.float32)
    err = np.abs(horner32(c, grid).astype(np.float64) - sigmoid(grid.astype(np.float64))).max()
    for i, a in enumerate(c):
        print(f"c{i} = {float(a):.9e}f")
    print(f"max |error| of float32 Horner on [0, 1]: {err:.3e}")

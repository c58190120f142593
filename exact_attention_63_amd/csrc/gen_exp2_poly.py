"""Coefficients of the polynomial that approximates 2^f on [0, 1] in the
software exp2 of the forward kernel (fa2_fwd_kernel.hpp, sw_exp2).

A least-squares fit of the relative error at Chebyshev nodes (close to the
minimax polynomial), degree 4, with the constant term pinned to 1 so that
2^0 is exact.  Prints the coefficients (c1..c4 for f, f^2, f^3, f^4) and the
largest relative error on a dense grid, in double and after rounding the
coefficients to float32.

    python gen_exp2_poly.py
"""

import numpy as np


def fit(degree: int = 4, nodes: int = 64):
    k = np.arange(nodes)
    f = 0.5 - 0.5 * np.cos(np.pi * (k + 0.5) / nodes)      # Chebyshev nodes on [0, 1]
    target = np.exp2(f)
    # 2^f ~ 1 + sum_i c_i f^i; weight rows by 1/2^f to fit the relative error
    a = np.stack([f ** i for i in range(1, degree + 1)], axis=1) / target[:, None]
    b = (target - 1.0) / target
    c, *_ = np.linalg.lstsq(a, b, rcond=None)
    return c


def rel_error(c):
    f = np.linspace(0.0, 1.0, 200001)
    p = 1.0 + sum(ci * f ** (i + 1) for i, ci in enumerate(c))
    return np.abs(p / np.exp2(f) - 1.0).max()


if __name__ == "__main__":
    c = fit()
    c32 = c.astype(np.float32).astype(np.float64)
    for i, ci in enumerate(c.astype(np.float32)):
        print(f"c{i + 1} = {float(ci)!r}f")
    print(f"max relative error: {rel_error(c):.3e} (double), {rel_error(c32):.3e} (float32 coefficients)")

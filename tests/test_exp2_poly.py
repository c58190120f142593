"""The polynomial of the forward kernel's software exp2 (sw_exp2 in
fa2_fwd_kernel.hpp): its coefficients are the ones gen_exp2_poly.py fits, and
2^x = 2^n * p(f) built from them stays within 3.5e-6 relative error of the
exact power of its float32 argument (the fit's 2.94e-6 plus float32
rounding), with masked (-inf) arguments giving exactly 0."""

import os
import re
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_63_amd", "csrc")


def kernel_coefficients():
    src = open(os.path.join(CSRC, "fa2_fwd_kernel.hpp")).read()
    body = src[src.index("float sw_exp2(float x)"):]
    body = body[:body.index("\n}\n")]
    return [float(x) for x in re.findall(r"(-?\d+\.\d+(?:e-?\d+)?)f", body) if abs(float(x)) < 1.0]


def sw_exp2(x, c):
    """The kernel's steps in float32: clamp, floor, fraction, Horner, ldexp, zero below -126."""
    x = np.asarray(x, dtype=np.float32)
    xc = np.maximum(x, np.float32(-127.0))
    n = np.floor(xc)
    f = (xc - n).astype(np.float32)
    c1, c2, c3, c4 = (np.float32(v) for v in c)
    p = np.float32(c4) * f + c3
    p = (p * f + c2).astype(np.float32)
    p = (p * f + c1).astype(np.float32)
    p = (p * f + np.float32(1.0)).astype(np.float32)
    r = np.ldexp(p, n.astype(np.int32)).astype(np.float32)
    return np.where(x < -126.0, np.float32(0.0), r)


def test_coefficients_match_the_fit():
    sys.path.insert(0, CSRC)
    import gen_exp2_poly
    fitted = gen_exp2_poly.fit().astype(np.float32)
    got = kernel_coefficients()
    # the constants appear in Horner order: c4, c3, c2, c1
    assert np.allclose(got, fitted[::-1], rtol=0, atol=0), (got, fitted)


def test_relative_error_and_masking():
    c = kernel_coefficients()[::-1]           # c1..c4
    # float32 arguments, as the kernel sees them; the exact power of each
    x = np.concatenate([np.linspace(-30.0, 8.0, 400001), np.arange(-30, 9, dtype=np.float64)])
    x = x.astype(np.float32).astype(np.float64)
    got = sw_exp2(x, c).astype(np.float64)
    rel = np.abs(got / np.exp2(x) - 1.0).max()
    # the fit's 2.94e-6 plus float32 rounding in the fraction and Horner steps
    assert rel <= 3.5e-6, rel
    assert sw_exp2(np.array([-np.inf, -126.5, -1000.0]), c).tolist() == [0.0, 0.0, 0.0]
    assert sw_exp2(np.array([0.0]), c)[0] == 1.0

"""Elementwise error bounds for the backward pass (shared by the GPU parity
test and the CPU test that pins the bound itself).

The kernels recompute P in fp32 from the saved LSE (relative error ~1e-6),
round P to the input dtype for dV = P^T dO, take D from the O the forward
pass stored (rounded to the dtype), round dS = P (dP - D) to the dtype for
dQ = scale dS K and dK = scale dS^T Q, accumulate in fp32 and round the
results to the dtype.  With u the unit roundoff of the dtype (bf16 2^-8,
fp16 2^-11) and a_i = sum_t |dO_it| |O_it|:

  E_ij   = u (|dS_ij| + P_ij a_i)          rounding of dS, and of O inside D
  |dV| <= u P^T |dO| + u |dV|
  |dK| <= |scale| E^T |Q| + u |dK|
  |dQ| <= |scale| E |K| + u |dQ|
  |D|  <= (u + 1e-5) a

An element passes when |got - ref| <= 2 * bound + 1e-5 * max|ref| (the
factor 2 covers second-order terms and fp32 accumulation, ~d 2^-24
relative).
"""

import numpy as np

import oracle

UNIT = {"fp16": 2.0 ** -11, "bf16": 2.0 ** -8}


def head_bounds(q, k, v, o_r, do, causal, scale, dtype, ref):
    """Bounds for one head (fp64 arrays [N, d]); ref = oracle (dq, dk, dv, delta)."""
    u = UNIT[dtype]
    n = q.shape[0]
    vis = oracle.visible_mask(np.arange(n), n, causal)
    s = np.where(vis, scale * (q @ k.T), -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(axis=1, keepdims=True)
    dq, dk, dv, delta = ref
    ds = p * ((do @ v.T) - delta[:, None])
    a = (np.abs(do) * np.abs(o_r)).sum(axis=1)
    E = u * (np.abs(ds) + p * a[:, None])
    b_dv = u * (p.T @ np.abs(do)) + u * np.abs(dv)
    b_dk = abs(scale) * (E.T @ np.abs(q)) + u * np.abs(dk)
    b_dq = abs(scale) * (E @ np.abs(k)) + u * np.abs(dq)
    b_delta = (u + 1e-5) * a
    return b_dq, b_dk, b_dv, b_delta


def allowance(bound, ref):
    return 2.0 * bound + 1e-5 * max(np.abs(ref).max(), 1e-30)


def worst_ratio(got, ref, bound):
    """max |got - ref| / allowance over all elements (<= 1 passes)."""
    err = np.abs(got - ref)
    return float((err / allowance(bound, ref)).max()) if err.size else 0.0

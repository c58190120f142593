"""CPU oracle for the exact-attention backward pass: dQ, dK, dV.

TEST INFRASTRUCTURE ONLY.  This module checks the HIP backward kernels.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import or call it.  It shares no code with the HIP
library or its Python binding and imports neither.

The pages name the backward pass as the step after the forward one: the
"FlashAttention v4 Blackwell pipeline co-design" diagram (its list of v4
directions, the backward note under its pseudo-code panel and its
"Backward 2-CTA" item) aims to cut dQ atomic accumulation, and a snippet of
the search-result page for "flash attention v2 论文" lists backward support
in a fused-attention implementation.  None of them prints the gradient
formulas.  This module therefore takes the derivative of the forward
definition (reading B1).  With S = scale * Q K^T (masked), P = softmax
rows of S, O = P V, and an upstream gradient dO:

  dV = P^T dO
  dP = dO V^T
  D_i = sum_j P_ij dP_ij          (equal to sum_d dO_id O_id)
  dS = P * (dP - D)               (elementwise, D broadcast along rows)
  dQ = scale * dS K
  dK = scale * dS^T Q

Masked entries have P = 0, hence dS = 0.  Everything is float64; library
matmuls serve as single steps.

READINGS
  B1  The gradients are those of the forward definition (the pages give
      none).
  B2  The upstream gradient dO has the shape and dtype of O.  The
      rounded-dtype dO is upcast exactly, like Q, K and V.
  B3  D is taken from P and dP (the definition).  The identity
      D_i = dO_i . O_i holds for the exact O, and the tests check it.

Pins (tests/test_oracle_backward.py): central finite differences of the
forward oracle, the fp64 CPU autograd of PyTorch's
scaled_dot_product_attention, the two column-sum identities
(sum_j dK_j = 0, sum_j dV_j = sum_i dO_i), and planted mistakes.
"""

from __future__ import annotations

import numpy as np

from .attention import visible_mask

__all__ = ["attention_backward"]


def _head_backward(q, k, v, do, causal, scale):
    n = q.shape[0]
    rows = np.arange(n, dtype=np.int64)
    s = scale * (q @ k.T)
    vis = visible_mask(rows, k.shape[0], causal)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    p = e / e.sum(axis=1)[:, None]
    dv = p.T @ do
    dp = do @ v.T
    delta = (p * dp).sum(axis=1)
    ds = p * (dp - delta[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv, delta


def attention_backward(q, k, v, do, causal: bool, scale: float):
    """Gradients of O = attention(q, k, v) against the upstream gradient do.

    q, k, v, do: float64 [..., N, d] (any number of leading batch/head dims).
    Returns (dq, dk, dv, delta) with delta[..., N] = rowsum(P * dP).
    """
    arrs = []
    for x in (q, k, v, do):
        x = np.asarray(x)
        if x.dtype != np.float64:
            raise TypeError("oracle inputs must be float64 (exact upcasts of the rounded inputs)")
        arrs.append(x)
    q, k, v, do = arrs
    if q.ndim < 2 or any(x.shape != q.shape for x in (k, v, do)):
        raise ValueError("q, k, v, do must share one shape [..., N, d]")
    n, d = q.shape[-2:]
    lead = q.shape[:-2]
    qf, kf, vf, df = (x.reshape(-1, n, d) for x in (q, k, v, do))
    dq = np.empty_like(qf)
    dk = np.empty_like(qf)
    dv = np.empty_like(qf)
    delta = np.empty(qf.shape[:2])
    for h in range(qf.shape[0]):
        dq[h], dk[h], dv[h], delta[h] = _head_backward(qf[h], kf[h], vf[h], df[h], causal, scale)
    return (dq.reshape(*lead, n, d), dk.reshape(*lead, n, d), dv.reshape(*lead, n, d),
            delta.reshape(*lead, n))

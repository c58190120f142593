"""CPU oracle for exact attention forward: O = softmax(scale * Q K^T) V and LSE.

TEST INFRASTRUCTURE ONLY.  This module is the independent checker of the HIP
path.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import or call it.  It shares no code with the HIP
library or its Python binding and imports neither.

Everything is float64 NumPy.  The caller hands in arrays that already hold the
fp16/bf16-rounded inputs, upcast exactly to float64, so that both sides see the
same numbers.  Library matmuls serve as single steps (the score product Q K^T
and the product P V); there is no blocking or fusion beyond what each
definition below states.

Sources (web pages on the subject):
  * search-result page for "flash attention v2 论文", snippet headed
    "0x01 Standard Self-Attention / 0x02 (Safe) Softmax: 3-pass": the standard
    attention definition (S = Q K^T, P = softmax(S), O = P V) and the
    three-pass safe softmax (row max; sum of exp(s - max); normalise).
  * same page, snippet on the FlashAttention paper title: the tiled method is
    exact, its output equals standard attention.
  * "FlashAttention v2 better parallelism + work partitioning" diagram,
    concept pseudo-code panel: per-row running state (m, l, acc) updated by an
    online softmax step per key tile, acc += P V, one output write per row.
  * "FlashAttention v4 Blackwell pipeline co-design" diagram, pseudo-code
    panel: the rescale of acc and l by exp(m - m_new), P = exp(S - m_new), and
    the final normalisation O = acc / l.  That panel omits adding rowsum(P) to l
    and the assignment m = m_new; both are restored here (see READINGS).

READINGS where the pages are silent, garbled or ambiguous:
  R1  l accumulates rowsum(P) and m takes m_new after each tile (both steps are
      missing from the v4 pseudo-code panel; without them O = acc / l is wrong).
  R2  LSE is the natural-log log-sum-exp of the scaled, masked scores of a row:
      LSE_i = ln sum_{j visible} exp(scale * q_i . k_j) = m_i + ln l_i.  The
      pages never define it; the forward pass is specified to return it.
  R3  Causal: key j is visible to query i iff j <= i (the diagonal is visible).
      Query and key lengths are equal, so top-left and bottom-right alignment
      coincide.
  R4  The scale multiplies the scores after the product (Q is never pre-scaled).
  R5  A tile with no visible key for a row leaves that row's state unchanged
      (exp offsets are guarded so that -inf - (-inf) never occurs).
  R6  The conditional rescale of the v4 diagram ("skip the rescale when the
      max changes little") is taken in its exact form: the reference max may
      lag the true running max by at most a threshold; the final O and LSE
      are unchanged in exact arithmetic.

Pins that tie this module to something other than itself live in
``tests/test_oracle_pins.py``: brute-force sums on tiny inputs, the worked
example in ``tests/golden/``, closed forms (constant V, scale = 0, causal row
0), invariants (shift and permutation), and the fp64 CPU
``scaled_dot_product_attention`` of PyTorch as a library special case.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "visible_mask",
    "softmax_probs",
    "attention_3pass",
    "attention_online",
]


def visible_mask(rows: np.ndarray, n_keys: int, causal: bool) -> np.ndarray:
    """Boolean [len(rows), n_keys]: True where key j is visible to query row i.

    Reading R3: causal visibility is j <= i.
    """
    rows = np.asarray(rows, dtype=np.int64)
    if not causal:
        return np.ones((rows.shape[0], n_keys), dtype=bool)
    return np.arange(n_keys, dtype=np.int64)[None, :] <= rows[:, None]


def _head_3pass(q, k, v, causal, scale, rows):
    """Standard attention with the 3-pass safe softmax for one head.

    q: [N, d], k: [N, d], v: [N, d] float64; rows: query indices to produce.
    Returns (O [len(rows), d], LSE [len(rows)], P [len(rows), N]).
    """
    s = scale * (q[rows] @ k.T)                      # scores of the requested rows
    vis = visible_mask(rows, k.shape[0], causal)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)                                # pass 1: row max
    e = np.exp(s - m[:, None])                       # masked entries give exp(-inf) = 0
    l = e.sum(axis=1)                                # pass 2: row sum of exp(s - m)
    p = e / l[:, None]                               # pass 3: normalise
    o = p @ v
    lse = m + np.log(l)                              # reading R2
    return o, lse, p


def _as_f64(x):
    x = np.asarray(x)
    if x.dtype != np.float64:
        raise TypeError("oracle inputs must be float64 (exact upcasts of the rounded inputs)")
    return x


def _check_shapes(q, k, v):
    if q.ndim < 2 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError(f"q, k, v must share one shape [..., N, d]; got {q.shape}, {k.shape}, {v.shape}")


def softmax_probs(q, k, causal: bool, scale: float, rows=None) -> np.ndarray:
    """The attention probabilities P = softmax(scale * q K^T) of one head.

    q, k: [N, d] float64.  Returns [len(rows), N]; masked entries are 0.
    Exposed so that tests can check that every row of P sums to one.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    n = q.shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    _, _, p = _head_3pass(q, k, k, causal, scale, rows)
    return p


def attention_3pass(q, k, v, causal: bool, scale: float, rows=None, chunk: int = 1024):
    """Exact attention forward, 3-pass safe softmax, float64.

    q, k, v: float64 [..., N, d] (any number of leading batch/head dims).
    rows: optional 1-D array of query indices; when given, only those rows of
      every head are produced (rows are independent of each other, so this is
      the same definition evaluated on fewer rows).
    chunk: rows per step, to bound the [chunk, N] score buffer; it changes
      memory use only, not arithmetic.
    Returns (O [..., R, d], LSE [..., R]) with R = N or len(rows).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    _check_shapes(q, k, v)
    n, d = q.shape[-2:]
    lead = q.shape[:-2]
    rows = np.arange(n, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= n):
        raise IndexError("row index out of range")
    qf = q.reshape(-1, n, d)
    kf = k.reshape(-1, n, d)
    vf = v.reshape(-1, n, d)
    o = np.empty((qf.shape[0], rows.size, d), dtype=np.float64)
    lse = np.empty((qf.shape[0], rows.size), dtype=np.float64)
    for h in range(qf.shape[0]):
        for c0 in range(0, rows.size, chunk):
            r = rows[c0:c0 + chunk]
            oh, lh, _ = _head_3pass(qf[h], kf[h], vf[h], causal, scale, r)
            o[h, c0:c0 + r.size] = oh
            lse[h, c0:c0 + r.size] = lh
    return o.reshape(*lead, rows.size, d), lse.reshape(*lead, rows.size)


def attention_online(q, k, v, causal: bool, scale: float, bc: int, trace=None,
                     rescale_threshold: float | None = None):
    """Tiled online-softmax model of the same forward pass, float64, one head.

    This is the update the GPU kernel implements, written in the order of the
    FA2 diagram's concept pseudo-code: for each key tile j of bc keys,
      S = scale * Q K_j^T, masked;
      m_new = max(m, rowmax S);
      alpha = exp(m - m_new)            (1 when both are -inf, reading R5);
      P = exp(S - m_new)                (0 at masked entries);
      l = alpha * l + rowsum P          (reading R1);
      acc = alpha * acc + P V_j;
      m = m_new                         (reading R1);
    then O = acc / l and LSE = m + ln l.

    q, k, v: float64 [N, d].  trace: optional callable(j0, m, l, acc) called
    after every tile with copies of the state, for worked-example tests.

    rescale_threshold (reading R6): when given as tau >= 0, the reference m of
    a row moves to the new maximum only when that maximum exceeds m by more
    than tau (or m is still -inf); otherwise m stays, alpha = 1 and the new
    p = exp(s - m) may exceed 1 (by at most e^tau).  O = acc / l and
    LSE = m + ln l use the same reference, so the result is the same exact
    value; only the point at which acc and l are rescaled changes (the
    conditional rescale of the FlashAttention v4 diagram, in its exact form).
    Returns (O [N, d], LSE [N]).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    _check_shapes(q, k, v)
    if q.ndim != 2:
        raise ValueError("attention_online takes one head: [N, d]")
    if bc < 1:
        raise ValueError("bc must be >= 1")
    n, d = q.shape
    rows = np.arange(n, dtype=np.int64)
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    acc = np.zeros((n, d))
    for j0 in range(0, n, bc):
        j1 = min(j0 + bc, n)
        s = scale * (q @ k[j0:j1].T)
        vis = visible_mask(rows, j1, causal)[:, j0:j1]
        s = np.where(vis, s, -np.inf)
        m_new = np.maximum(m, s.max(axis=1))
        if rescale_threshold is not None:
            keep = np.isfinite(m) & (m_new - m <= rescale_threshold)
            m_new = np.where(keep, m, m_new)
        dead = np.isneginf(m_new)                     # no visible key yet
        ref = np.where(dead, 0.0, m_new)              # guarded subtrahend
        alpha = np.where(dead, 1.0, np.exp(m - ref))
        p = np.exp(s - ref[:, None])                  # masked: exp(-inf) = 0
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ v[j0:j1]
        m = m_new
        if trace is not None:
            trace(j0, m.copy(), l.copy(), acc.copy())
    o = acc / l[:, None]
    lse = m + np.log(l)
    return o, lse

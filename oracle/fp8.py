"""CPU oracle for the FP8 (E4M3) attention forward pass.

TEST INFRASTRUCTURE ONLY.  Like ``oracle/attention.py`` this module is the
independent checker of the HIP path: only ``tests/``, the smoke check and the
``cpu_baseline`` leg of the benchmark may import it.  It shares no code with
the HIP library or its binding and imports neither.  Everything is float64
NumPy; the E4M3 format is decoded and rounded here from its definition.

Sources (web pages on the subject):
  * "FlashAttention v2 better parallelism + work partitioning" diagram, panel
    on what v2 changes: FP8 arithmetic is one of the hardware capabilities
    that v2 leaves unused.
  * search-result page for "flash attention v2 论文", snippet on the Triton
    fused-attention tutorial, which lists fp8 among its cases.
  * every other step as in ``oracle/attention.py``: standard attention and the
    3-pass safe softmax (search page, "0x01" / "0x02"), the per-tile online
    update (v2 diagram, concept pseudo-code panel; v4 diagram, pseudo-code
    panel) and the conditional rescale of the v4 diagram in its exact form
    (reading R6 there).

The pages give no FP8 scheme.  READINGS:
  F1  Inputs are 8-bit codes in the OCP E4M3 format: 1 sign bit, 4 exponent
      bits with bias 7, 3 mantissa bits; exponent field 0 holds the
      subnormals m * 2^-9; the codes S.1111.111 are NaN; there are no
      infinities; the largest finite magnitude is 448.  Each tensor comes with
      one float32 descale factor: the real input is decode(code) * descale.
  F2  The operation is exact attention of the dequantised inputs:
      ``attention_fp8`` is ``attention_3pass`` of them.
  F3  The P.V product takes P in E4M3.  Within each key tile of ``bc`` keys,
      P = exp(S - m) is multiplied by 2^shift and rounded to the nearest E4M3
      value (ties to even); acc accumulates round(2^shift P) V while l
      accumulates the unrounded 2^shift P.  Then O = acc / l (2^shift cancels)
      and LSE = m + ln l - shift ln 2.
  F4  The reference m of a row follows R6 with threshold tau: it moves to the
      tile max only when that exceeds m by more than tau (or m is still
      -inf).  So 2^shift P <= 2^shift e^tau; shift = 6 with tau = 2.75 ln 2
      keeps it at most 2^8.75 ~= 430.5 < 448, while values down to 2^-12 of
      the reference stay normal E4M3 numbers.  (With shift 8 and tau 0.75 ln 2
      the reference of a 32-row group moved in about half of the tiles of
      N(0,1) inputs, against 6 % here, at the same error.)
  F5  Rounding to E4M3 saturates: magnitudes above 448 give 448.  F4 keeps P
      below that; the rule only makes the rounding function total.

Pins: ``tests/test_oracle_fp8.py`` (every code against PyTorch's
float8_e4m3fn decoding, closed-form codes, rounding against PyTorch's
conversion and at midpoints, brute force on a tiny head, a hand-worked
rounding example, exactness when every P is a power of two, the derived
quantisation bound).
"""

from __future__ import annotations

import math

import numpy as np

from .attention import attention_3pass, visible_mask

__all__ = [
    "E4M3_MAX",
    "e4m3_decode",
    "e4m3_round",
    "dequantise",
    "attention_fp8",
    "attention_online_fp8",
    "P_SHIFT",
    "TAU_LOG2",
]

#: largest finite E4M3 magnitude (reading F1): 1.75 * 2^8
E4M3_MAX = 448.0
#: P is scaled by 2^P_SHIFT before rounding (reading F3)
P_SHIFT = 6
#: threshold of the lazy reference in base-2 units (reading F4); tau = TAU_LOG2 * ln 2
TAU_LOG2 = 2.75


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code (reading F1), float64; NaN codes give NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7 == 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    sub = m * 2.0 ** -9
    mag = np.where(e == 0, sub, normal)
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_round(x) -> np.ndarray:
    """Round float64 values to the nearest E4M3 value, ties to even, saturating
    at +-448 (reading F5).  Returns the rounded values as float64.

    The grid spacing at |x| in [2^e, 2^(e+1)) is 2^(e-3) for e >= -6 (normal
    numbers: 3 mantissa bits) and 2^-9 below 2^-6 (subnormals).  Dividing by
    a power of two is exact, so np.round (half to even) rounds exactly.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, ex = np.frexp(a)                       # a = f * 2^ex, f in [0.5, 1): floor(log2 a) = ex - 1
    spacing = np.exp2(np.maximum(ex - 1 - 3, -9).astype(np.float64))
    r = np.round(a / spacing) * spacing
    r = np.minimum(r, E4M3_MAX)
    return np.copysign(r, x)


def dequantise(codes, descale: float) -> np.ndarray:
    """decode(code) * descale, float64 (reading F1)."""
    return e4m3_decode(codes) * float(descale)


def attention_fp8(q8, k8, v8, descale_q: float, descale_k: float, descale_v: float,
                  causal: bool, scale: float, rows=None):
    """Exact attention of the dequantised inputs (reading F2).

    q8, k8, v8: uint8 E4M3 codes [..., N, d].  Returns (O, LSE) in float64 as
    ``attention_3pass`` does.
    """
    q = dequantise(q8, descale_q)
    k = dequantise(k8, descale_k)
    v = dequantise(v8, descale_v)
    return attention_3pass(q, k, v, causal, scale, rows=rows)


def attention_online_fp8(q8, k8, v8, descale_q: float, descale_k: float, descale_v: float,
                         causal: bool, scale: float, bc: int, tau: float = TAU_LOG2 * math.log(2.0),
                         shift: int = P_SHIFT, round_p: bool = True, trace=None):
    """Tiled online-softmax model of the FP8 forward pass, one head, float64.

    The steps of ``attention_online`` (per key tile of bc keys: S = scale Q K^T
    masked; m_new from the tile max under the lazy reference of reading F4;
    alpha = exp(m - m_new); P = exp(S - m_new); l = alpha l + rowsum;
    acc = alpha acc + ... ; m = m_new), with P entering the P.V product as
    round(2^shift P) in E4M3 and l summing 2^shift P (reading F3).

    q8, k8, v8: uint8 codes [N, d].  round_p=False skips the rounding (then
    the model is the exact online softmax).  trace: optional
    callable(j0, m, p_scaled, p_rounded) after every tile, with m the
    reference after the tile and the [N, tile] matrices of 2^shift P before
    and after rounding.
    Returns (O [N, d], LSE [N]).
    """
    q = dequantise(q8, descale_q)
    k = dequantise(k8, descale_k)
    v = dequantise(v8, descale_v)
    if q.ndim != 2 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("attention_online_fp8 takes one head: [N, d] codes")
    if bc < 1:
        raise ValueError("bc must be >= 1")
    n, d = q.shape
    rows = np.arange(n, dtype=np.int64)
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    acc = np.zeros((n, d))
    two_s = 2.0 ** shift
    for j0 in range(0, n, bc):
        j1 = min(j0 + bc, n)
        s = scale * (q @ k[j0:j1].T)
        vis = visible_mask(rows, j1, causal)[:, j0:j1]
        s = np.where(vis, s, -np.inf)
        m_tile = s.max(axis=1)
        move = np.isneginf(m) | (m_tile > m + tau)        # reading F4 (R6 with threshold tau)
        m_new = np.where(move, m_tile, m)
        dead = np.isneginf(m_new)                         # no visible key yet
        ref = np.where(dead, 0.0, m_new)
        alpha = np.where(dead, 1.0, np.exp(m - ref))
        p_scaled = two_s * np.exp(s - ref[:, None])       # 2^shift P, masked entries 0
        p_rounded = e4m3_round(p_scaled) if round_p else p_scaled
        l = alpha * l + p_scaled.sum(axis=1)
        acc = alpha[:, None] * acc + p_rounded @ v[j0:j1]
        m = m_new
        if trace is not None:
            trace(j0, m.copy(), p_scaled.copy(), p_rounded.copy())
    o = acc / l[:, None]
    lse = m + np.log(l) - shift * math.log(2.0)
    return o, lse

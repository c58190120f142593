"""Seeded synthetic inputs for the attention workloads (forward and backward).

This module is shared by the tests, the benchmark and the smoke check.  It
draws random numbers and rounds them to the input dtype; it holds none of the
attention arithmetic, and neither the oracle nor the HIP binding depends on it.

Recipe (the same for every workload):
  * generator: NumPy PCG64 ``default_rng(seed)``;
  * draw order: Q, then K, then V, each as float32 ``standard_normal`` of shape
    [B, H, N, d], multiplied by ``sigma``;
  * optional key offset: one scalar c[b, h, j] ~ U(lo, hi) per key row, drawn
    after V and added to all d entries of K[b, h, j, :];
  * rounding: float32 -> fp16 or bf16, round-to-nearest-even (PyTorch's CPU
    cast).  The GPU and the oracle consume these same rounded tensors; the
    oracle sees them upcast exactly to float64;
  * upstream gradient dO of the backward pass: its own generator,
    ``default_rng(GRAD_SEED_OFFSET + seed)``, one float32 ``standard_normal``
    draw of shape [B, H, N, d] (not scaled by sigma), rounded the same way.

FP8 inputs (8-bit E4M3 codes with one float32 descale factor per tensor):
  * ``make_inputs_fp8``: the same float32 draws as above; each tensor x gets
    descale = max|x| / 448 (rounded to float32) and codes = E4M3(x / descale),
    PyTorch's CPU cast to float8_e4m3fn (nearest even), read back as bytes;
  * ``make_exact_fp8``: inputs on which the FP8 pass has no rounding besides
    summation order and the output cast.  Each head has 16 random positions
    out of d; every K row holds +-1 at all 16, every Q row +-1 at 6 or 7 of
    them (code 0x38 is 1.0, 0xB8 is -1.0, the rest 0x00); descales 1/2 and
    1/4 and scale 8 ln 2 make scale * q.k * log2(e) an integer in [-7, 7],
    so every 2^6 P lies on the E4M3 grid (2^-8 .. 2^8), away from the
    midpoints.  V is drawn as in ``make_inputs_fp8``.  Draw order: V (as
    above, seed), then from default_rng(EXACT_SEED_OFFSET + seed) the head
    positions, the Q positions, the Q signs, the Q counts and the K signs.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "HEADLINE", "make_inputs", "make_grad_output", "workload_inputs",
           "workload_grad_output", "to_f64", "torch_dtype", "make_inputs_fp8", "make_exact_fp8",
           "FP8_WORKLOADS", "FP8_HEADLINE", "workload_inputs_fp8"]

_DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16}

#: dO is drawn from default_rng(GRAD_SEED_OFFSET + seed)
GRAD_SEED_OFFSET = 1000
#: the sparse +-1 Q and K of make_exact_fp8 come from default_rng(EXACT_SEED_OFFSET + seed)
EXACT_SEED_OFFSET = 2000
#: largest finite E4M3 magnitude
_E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention forward problem: shapes, dtype, masking and input recipe."""

    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "fp16" | "bf16" | "fp8" (E4M3 inputs, bf16 output)
    causal: bool
    seed: int
    sigma: float = 1.0
    key_offset: tuple | None = None   # (lo, hi) of the per-key-row uniform offset on K

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def flops(self) -> float:
        """Counted FLOPs: 4*B*H*N^2*d, halved when causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    @property
    def bwd_flops(self) -> float:
        """Counted backward FLOPs: the five products (S, dP, dV, dK, dQ) of
        2*N^2*d each, 10*B*H*N^2*d, halved when causal."""
        f = 10.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    @property
    def bwd_hbm_bytes(self) -> int:
        """Algorithmic HBM bytes of the backward pass: Q, K, V, O, dO read once,
        dQ, dK, dV written once, LSE read and D written and read (fp32)."""
        rows = self.B * self.H * self.N
        return 8 * rows * self.d * 2 + 3 * rows * 4

    @property
    def hbm_bytes(self) -> int:
        """Algorithmic HBM bytes: Q, K, V read once, O written once, fp32 LSE
        (FP8: 1-byte Q, K, V and a bf16 O)."""
        rows = self.B * self.H * self.N
        if self.dtype == "fp8":
            return rows * self.d * (3 + 2) + 4 * rows
        return 4 * rows * self.d * 2 + 4 * rows

    def describe(self) -> dict:
        return {
            "workload": self.name, "B": self.B, "H": self.H, "N": self.N, "d": self.d,
            "dtype": self.dtype, "causal": self.causal, "scale": "1/sqrt(d)",
            "inputs": f"N(0,{self.sigma}^2)" + (" as E4M3 with per-tensor descale" if self.dtype == "fp8" else "") + (
                f", K += U({self.key_offset[0]},{self.key_offset[1]}) per key row"
                if self.key_offset else ""),
            "seed": self.seed,
        }


WORKLOADS = {
    w.name: w for w in [
        Workload("b1h1n128d64_fp16", 1, 1, 128, 64, "fp16", False, seed=1),
        Workload("b4h16n1024d64_fp16", 4, 16, 1024, 64, "fp16", False, seed=2),
        Workload("b4h16n1024d64_fp16_causal", 4, 16, 1024, 64, "fp16", True, seed=2),
        Workload("b8h32n2048d128_bf16", 8, 32, 2048, 128, "bf16", False, seed=3),
        Workload("b2h16n4096d128_bf16_causal", 2, 16, 4096, 128, "bf16", True, seed=4),
        Workload("b1h32n16384d128_bf16_causal_koff", 1, 32, 16384, 128, "bf16", True, seed=5,
                 sigma=0.5, key_offset=(-4.0, 4.0)),
    ]
}

#: the throughput headline: B=8, H=32, N=2048, d=128, bf16, non-causal
HEADLINE = "b8h32n2048d128_bf16"


def torch_dtype(name: str) -> torch.dtype:
    return _DTYPES[name]


def make_inputs(B: int, H: int, N: int, d: int, dtype: str, seed: int,
                sigma: float = 1.0, key_offset=None):
    """Return (q, k, v) as contiguous CPU torch tensors [B, H, N, d] of ``dtype``."""
    if dtype not in _DTYPES:
        raise ValueError(f"dtype must be one of {sorted(_DTYPES)}")
    td = _DTYPES[dtype]
    return tuple(torch.from_numpy(x).to(td).contiguous() for x in _draw(B, H, N, d, seed, sigma, key_offset))


def _draw(B, H, N, d, seed, sigma, key_offset):
    """The float32 draws (q, k, v) of the recipe above."""
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        s = np.float32(sigma)
        q *= s
        k *= s
        v *= s
    if key_offset is not None:
        lo, hi = key_offset
        c = rng.uniform(lo, hi, size=(B, H, N, 1)).astype(np.float32)
        k += c
    return q, k, v


def _to_e4m3(x: np.ndarray):
    """(codes uint8 tensor, descale): descale = max|x| / 448 as float32,
    codes = E4M3(x / descale) by PyTorch's CPU cast."""
    amax = float(np.abs(x).max()) if x.size else 0.0
    descale = np.float32(amax / _E4M3_MAX) if amax > 0 else np.float32(1.0)
    y = np.clip(x / descale, -_E4M3_MAX, _E4M3_MAX).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    return codes, float(descale)


def make_inputs_fp8(B: int, H: int, N: int, d: int, seed: int, sigma: float = 1.0, key_offset=None):
    """FP8 inputs: ((q8, k8, v8), (descale_q, descale_k, descale_v)), the codes
    as contiguous uint8 CPU tensors [B, H, N, d]."""
    q, k, v = _draw(B, H, N, d, seed, sigma, key_offset)
    (q8, dq), (k8, dk), (v8, dv) = _to_e4m3(q), _to_e4m3(k), _to_e4m3(v)
    return (q8, k8, v8), (dq, dk, dv)


#: scale of make_exact_fp8: scale * (1/2) * (1/4) * log2(e) = 1
EXACT_FP8_SCALE = 8.0 * math.log(2.0)


def make_exact_fp8(B: int, H: int, N: int, d: int, seed: int):
    """Inputs with integer base-2 scores (see the module recipe): returns
    ((q8, k8, v8), (1/2, 1/4, descale_v), scale)."""
    _, _, v = _draw(B, H, N, d, seed, 1.0, None)
    v8, dv = _to_e4m3(v)
    rng = np.random.default_rng(EXACT_SEED_OFFSET + seed)
    head_pos = np.argsort(rng.random((B, H, 1, d)), axis=-1)[..., :16]          # [B, H, 1, 16]
    q_pick = np.argsort(rng.random((B, H, N, 16)), axis=-1)[..., :7]            # 7 of the 16
    q_pos = np.take_along_axis(np.broadcast_to(head_pos, (B, H, N, 16)), q_pick, axis=-1)
    q_sign = rng.integers(0, 2, size=(B, H, N, 7))
    q_count = 6 + rng.integers(0, 2, size=(B, H, N, 1))                          # keep 6 or 7
    k_sign = rng.integers(0, 2, size=(B, H, N, 16))

    def codes(pos, sign, keep=None):
        c = np.zeros((B, H, N, d), dtype=np.uint8)
        val = np.where(sign == 1, 0xB8, 0x38).astype(np.uint8)
        if keep is not None:
            val = np.where(keep, val, 0).astype(np.uint8)
        np.put_along_axis(c, pos, val, axis=-1)
        return torch.from_numpy(c).contiguous()

    q8 = codes(q_pos, q_sign, np.arange(7)[None, None, None, :] < q_count)
    k8 = codes(np.broadcast_to(head_pos, (B, H, N, 16)), k_sign)
    return (q8, k8, v8), (0.5, 0.25, dv), EXACT_FP8_SCALE


def make_grad_output(B: int, H: int, N: int, d: int, dtype: str, seed: int):
    """The upstream gradient dO [B, H, N, d] of ``dtype`` (CPU, contiguous)."""
    if dtype not in _DTYPES:
        raise ValueError(f"dtype must be one of {sorted(_DTYPES)}")
    rng = np.random.default_rng(GRAD_SEED_OFFSET + seed)
    g = rng.standard_normal((B, H, N, d), dtype=np.float32)
    return torch.from_numpy(g).to(_DTYPES[dtype]).contiguous()


def workload_grad_output(w: Workload):
    """The seeded dO of a named workload."""
    return make_grad_output(w.B, w.H, w.N, w.d, w.dtype, w.seed)


def workload_inputs(w: Workload):
    """The seeded inputs of a named workload."""
    return make_inputs(w.B, w.H, w.N, w.d, w.dtype, w.seed, w.sigma, w.key_offset)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a fp16/bf16/fp32 tensor (any device) to a float64 array."""
    return t.detach().to("cpu").to(torch.float64).numpy()


#: FP8 workloads: E4M3 inputs (make_inputs_fp8), bf16 output; the same shapes,
#: seeds and recipes as the 16-bit workloads they are named after
FP8_WORKLOADS = {
    w.name: w for w in [
        Workload("b8h32n2048d128_fp8", 8, 32, 2048, 128, "fp8", False, seed=3),
        Workload("b2h16n4096d128_fp8_causal", 2, 16, 4096, 128, "fp8", True, seed=4),
        Workload("b4h16n1024d64_fp8", 4, 16, 1024, 64, "fp8", False, seed=2),
    ]
}

#: the FP8 throughput workload: the headline shape with E4M3 inputs
FP8_HEADLINE = "b8h32n2048d128_fp8"


def workload_inputs_fp8(w: Workload):
    """The seeded E4M3 inputs and descales of a named FP8 workload."""
    return make_inputs_fp8(w.B, w.H, w.N, w.d, w.seed, w.sigma, w.key_offset)

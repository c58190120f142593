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
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "HEADLINE", "make_inputs", "make_grad_output", "workload_inputs",
           "workload_grad_output", "to_f64", "torch_dtype"]

_DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16}

#: dO is drawn from default_rng(GRAD_SEED_OFFSET + seed)
GRAD_SEED_OFFSET = 1000


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention forward problem: shapes, dtype, masking and input recipe."""

    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "fp16" | "bf16"
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
        """Algorithmic HBM bytes: Q, K, V read once, O written once, fp32 LSE."""
        el = 2
        return 4 * self.B * self.H * self.N * self.d * el + 4 * self.B * self.H * self.N

    def describe(self) -> dict:
        return {
            "workload": self.name, "B": self.B, "H": self.H, "N": self.N, "d": self.d,
            "dtype": self.dtype, "causal": self.causal, "scale": "1/sqrt(d)",
            "inputs": f"N(0,{self.sigma}^2)" + (
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
    td = _DTYPES[dtype]
    return tuple(torch.from_numpy(x).to(td).contiguous() for x in (q, k, v))


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

"""The seeded input recipe: shapes, determinism, rounding and the key offset."""

import math

import numpy as np
import torch

import workloads
import workloads as W
from workloads import WORKLOADS, make_inputs, to_f64


def test_workload_table():
    names = set(WORKLOADS)
    assert workloads.HEADLINE in names
    w = WORKLOADS[workloads.HEADLINE]
    assert (w.B, w.H, w.N, w.d, w.dtype, w.causal) == (8, 32, 2048, 128, "bf16", False)
    assert w.flops == 4 * 8 * 32 * 2048 ** 2 * 128
    c = WORKLOADS["b2h16n4096d128_bf16_causal"]
    assert c.flops == 4 * 2 * 16 * 4096 ** 2 * 128 / 2
    assert w.hbm_bytes == 8 * 8 * 32 * 2048 * 128 + 4 * 8 * 32 * 2048


def test_deterministic_and_rounded():
    a = make_inputs(2, 3, 17, 8, "bf16", seed=5)
    b = make_inputs(2, 3, 17, 8, "bf16", seed=5)
    c = make_inputs(2, 3, 17, 8, "bf16", seed=6)
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16 and x.shape == (2, 3, 17, 8) and x.is_contiguous()
        assert torch.equal(x, y)
    assert not torch.equal(a[0], c[0])
    q16, _, _ = make_inputs(1, 1, 4, 4, "fp16", seed=1)
    assert q16.dtype == torch.float16


def test_rounding_is_rne_of_the_fp32_draw():
    rng = np.random.default_rng(9)
    q32 = rng.standard_normal((1, 1, 5, 4), dtype=np.float32)
    q, _, _ = make_inputs(1, 1, 5, 4, "bf16", seed=9)
    # bf16 RNE by integer arithmetic on the fp32 bit pattern
    bits = q32.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    ref = rounded.astype(np.uint32).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(to_f64(q), ref)


def test_key_offset_is_per_key_row():
    q0, k0, v0 = make_inputs(1, 2, 64, 16, "bf16", seed=3, sigma=0.5)
    q1, k1, v1 = make_inputs(1, 2, 64, 16, "bf16", seed=3, sigma=0.5, key_offset=(-4.0, 4.0))
    assert torch.equal(q0, q1) and torch.equal(v0, v1)
    diff = to_f64(k1) - to_f64(k0)
    # the offset is constant along d for each key row, up to bf16 rounding of the sum
    row_mean = diff.mean(axis=-1, keepdims=True)
    assert np.all(np.abs(row_mean) <= 4.1)
    assert np.max(np.abs(diff - row_mean)) < 0.05
    assert row_mean.std() > 1.0


def test_fp8_inputs_recipe():
    (q8, k8, v8), (dq, dk, dv) = W.make_inputs_fp8(2, 3, 40, 64, seed=4)
    q, k, v = W.make_inputs(2, 3, 40, 64, "bf16", seed=4)
    for codes, desc, x16 in ((q8, dq, q), (k8, dk, k), (v8, dv, v)):
        assert codes.dtype == torch.uint8 and codes.shape == (2, 3, 40, 64) and codes.is_contiguous()
        assert ((codes & 0x7F) != 0x7F).all()                    # no NaN codes
        # the codes decode (PyTorch) to the float32 draws within E4M3 rounding
        back = codes.view(torch.float8_e4m3fn).double() * desc
        assert torch.allclose(back, x16.double(), rtol=2 ** -4 + 2 ** -8, atol=2 ** -9 * desc)
    again = W.make_inputs_fp8(2, 3, 40, 64, seed=4)
    assert all(torch.equal(a, b) for a, b in zip(again[0], (q8, k8, v8))) and again[1] == (dq, dk, dv)


def test_fp8_exact_inputs_recipe():
    (q8, k8, v8), (dq, dk, dv), scale = W.make_exact_fp8(1, 2, 100, 128, seed=6)
    assert (dq, dk) == (0.5, 0.25)
    assert set(q8.unique().tolist()) <= {0x00, 0x38, 0xB8} and set(k8.unique().tolist()) <= {0x00, 0x38, 0xB8}
    nq = (q8 != 0).sum(-1)
    assert ((nq == 6) | (nq == 7)).all() and (nq == 6).any() and (nq == 7).any()
    assert ((k8 != 0).sum(-1) == 16).all()
    q = q8.view(torch.float8_e4m3fn).double() * dq
    k = k8.view(torch.float8_e4m3fn).double() * dk
    t = scale * (q @ k.transpose(-1, -2)) / math.log(2.0)
    assert (t - t.round()).abs().max() < 1e-12 and t.abs().max() <= 7

"""The seeded input recipe: shapes, determinism, rounding and the key offset."""

import numpy as np
import torch

import workloads
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

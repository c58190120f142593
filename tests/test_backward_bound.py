"""CPU pins of the backward pass's elementwise error bound (tests/bwd_bounds.py).

The GPU parity test accepts a gradient element when its distance to the fp64
oracle is within a bound derived from the rounding the kernels perform.  Two
properties make that bound meaningful, and both are checked here without a
GPU:
  * it is not too tight: a NumPy model of the kernels' arithmetic (P from the
    saved fp32 LSE, P and dS rounded to the input dtype, dS formed from the
    fp32 or from the rounded P, D from the O stored in the dtype, outputs
    rounded to the dtype) stays inside it;
  * it is not vacuous: plausible kernel mistakes (D dropped, dS without the
    factor P, scale dropped, causal mask dropped, a product not transposed,
    the LSE taken in the wrong base) land outside it for some element.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from bwd_bounds import head_bounds, worst_ratio
from workloads import make_grad_output, make_inputs, to_f64

LOG2E = 1.4426950408889634


def rnd(x, dtype):
    """Round to the 16-bit dtype (RNE) and back to fp64."""
    td = torch.bfloat16 if dtype == "bf16" else torch.float16
    return torch.from_numpy(np.ascontiguousarray(x)).to(td).to(torch.float64).numpy()


def f32(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def kernel_model(q, k, v, o_r, lse32, do, causal, scale, dtype, mistake=None, p16_in_ds=False):
    """The kernels' arithmetic for one head, optionally with one planted mistake.
    p16_in_ds: dS formed from the 16-bit P (the pipelined dK/dV kernel) instead of the fp32 P."""
    n = q.shape[0]
    vis = oracle.visible_mask(np.arange(n), n, causal)
    if mistake == "unmasked_p":
        vis = np.ones_like(vis)
    s = f32(q @ k.T)
    lse2 = f32(lse32 * LOG2E) if mistake != "lse_base_e" else lse32
    p = f32(np.exp2(np.where(vis, f32(s * f32(scale * LOG2E)) - lse2[:, None], -np.inf)))
    dv = rnd(rnd(p, dtype).T @ do, dtype)
    dp = f32(do @ v.T)
    delta = f32((do * o_r).sum(axis=1))
    if mistake == "no_delta":
        delta = np.zeros_like(delta)
    p_ds = rnd(p, dtype) if p16_in_ds else p
    ds = f32(dp - delta[:, None]) if mistake == "ds_without_p" else f32(p_ds * (dp - delta[:, None]))
    ds_r = rnd(ds, dtype)
    sq = 1.0 if mistake == "dq_no_scale" else scale
    dq = rnd(sq * (ds_r @ k), dtype)
    dk = rnd(scale * (ds_r @ q), dtype) if mistake == "dk_no_transpose" else rnd(scale * (ds_r.T @ q), dtype)
    if mistake == "dv_uses_ds":
        dv = rnd(ds_r.T @ do, dtype)
    return dq, dk, dv, delta


def case(dtype, causal, seed, n=96, d=64):
    q, k, v = (to_f64(x)[0, 0] for x in make_inputs(1, 1, n, d, dtype, seed))
    do = to_f64(make_grad_output(1, 1, n, d, dtype, seed))[0, 0]
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attention_3pass(q, k, v, causal, scale)
    o_r = rnd(o, dtype)
    lse32 = f32(lse)
    ref = oracle.attention_backward(q, k, v, do, causal, scale)
    bounds = head_bounds(q, k, v, o_r, do, causal, scale, dtype, ref)
    return q, k, v, o_r, lse32, do, scale, ref, bounds


@pytest.mark.parametrize("p16_in_ds", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_kernel_rounding_stays_inside_the_bound(dtype, causal, p16_in_ds):
    q, k, v, o_r, lse32, do, scale, ref, bounds = case(dtype, causal, seed=101)
    got = kernel_model(q, k, v, o_r, lse32, do, causal, scale, dtype, p16_in_ds=p16_in_ds)
    ratios = [worst_ratio(g, r, b) for g, r, b in zip(got, ref, bounds)]
    print(dtype, causal, p16_in_ds, ["%.3f" % x for x in ratios])
    assert max(ratios) <= 1.0, ratios


@pytest.mark.parametrize("mistake", ["no_delta", "ds_without_p", "dq_no_scale", "dk_no_transpose",
                                     "dv_uses_ds", "lse_base_e", "unmasked_p"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_planted_mistakes_break_the_bound(mistake, dtype):
    causal = True   # the unmasked-P mistake only exists with a mask
    q, k, v, o_r, lse32, do, scale, ref, bounds = case(dtype, causal, seed=202)
    got = kernel_model(q, k, v, o_r, lse32, do, causal, scale, dtype, mistake=mistake)
    ratios = [worst_ratio(g, r, b) for g, r, b in zip(got, ref, bounds)]
    print(mistake, dtype, ["%.3g" % x for x in ratios])
    assert max(ratios) > 1.0, (mistake, ratios)

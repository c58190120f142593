"""Pins of the FP8 oracle (oracle/fp8.py) to things other than itself.

* the E4M3 decoding of every code against PyTorch's float8_e4m3fn (a library
  routine) and against closed-form values of the format;
* rounding: grid values are fixed points, midpoints go to the even code,
  random values agree with PyTorch's float8_e4m3fn cast, large values saturate;
* exact attention of the dequantised inputs by brute force on a tiny head and
  through the descale invariances;
* the tiled model: equal to exact attention when every P is a power of two
  (the exact-input recipe), equal to it when the rounding is switched off,
  a hand-worked two-key example whose result depends on the tiling, the
  derived quantisation bound, and the reference threshold in the trace.
"""

import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention_3pass
from oracle.fp8 import (E4M3_MAX, P_SHIFT, TAU_LOG2, attention_fp8, attention_online_fp8, dequantise,
                        e4m3_decode, e4m3_round)

TAU = TAU_LOG2 * math.log(2.0)


def torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy()).view(torch.float8_e4m3fn).double().numpy()


def test_decode_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    ref = torch_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2                                     # 0x7F and 0xFF
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


@pytest.mark.parametrize("code,value", [
    (0x38, 1.0), (0x40, 2.0), (0x3C, 1.5), (0x7E, 448.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9),
    (0x08, 2.0 ** -6), (0xB8, -1.0), (0xFE, -448.0), (0x00, 0.0),
])
def test_decode_closed_forms(code, value):
    assert e4m3_decode(np.array([code], dtype=np.uint8))[0] == value


def test_decode_negative_zero_and_nan():
    v = e4m3_decode(np.array([0x80, 0x7F, 0xFF], dtype=np.uint8))
    assert v[0] == 0.0 and np.signbit(v[0])
    assert np.isnan(v[1]) and np.isnan(v[2])


def finite_grid():
    codes = np.arange(256, dtype=np.uint8)
    v = e4m3_decode(codes)
    keep = np.isfinite(v)
    return codes[keep], v[keep]


def test_round_fixed_points():
    _, v = finite_grid()
    assert np.array_equal(e4m3_round(v), v)


def test_round_midpoints_ties_to_even():
    codes, v = finite_grid()
    pos = v > 0
    order = np.argsort(v[pos])
    c, x = codes[pos][order], v[pos][order]
    mid = (x[:-1] + x[1:]) / 2                                # exact in float64
    even = np.where(c[:-1] % 2 == 0, x[:-1], x[1:])
    assert np.array_equal(e4m3_round(mid), even)
    assert np.array_equal(e4m3_round(-mid), -even)
    eps = 1e-9 * (x[1:] - x[:-1])
    assert np.array_equal(e4m3_round(mid - eps), x[:-1])
    assert np.array_equal(e4m3_round(mid + eps), x[1:])
    # between 0 and the smallest subnormal 2^-9
    assert e4m3_round(np.array([2.0 ** -10]))[0] == 0.0
    assert e4m3_round(np.array([2.0 ** -10 * 1.001]))[0] == 2.0 ** -9


def test_round_matches_torch_cast():
    rng = np.random.default_rng(11)
    mag = np.exp2(rng.uniform(-13, math.log2(E4M3_MAX), size=200_000))
    x = mag * np.where(rng.random(mag.size) < 0.5, -1.0, 1.0)
    x = x.astype(np.float32).astype(np.float64)               # values the cast sees exactly
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(e4m3_round(x), ref)


def test_round_saturates():
    x = np.array([448.0, 449.0, 463.9, 464.0, 1e6, -500.0])
    assert np.array_equal(e4m3_round(x), [448.0, 448.0, 448.0, 448.0, 448.0, -448.0])


def test_attention_fp8_brute_force_tiny():
    # one head, N = 3, d = 2; codes chosen by hand
    q8 = np.array([[0x38, 0x00], [0x40, 0xB8], [0x30, 0x3C]], dtype=np.uint8)   # [1,0],[2,-1],[0.5,1.5]
    k8 = np.array([[0x38, 0x38], [0xC0, 0x30], [0x00, 0x40]], dtype=np.uint8)   # [1,1],[-2,0.5],[0,2]
    v8 = np.array([[0x38, 0x40], [0xB8, 0x00], [0x44, 0x3C]], dtype=np.uint8)   # [1,2],[-1,0],[3,1.5]
    dq, dk, dv, scale = 0.5, 2.0, 0.25, 0.7
    q = [[1, 0], [2, -1], [0.5, 1.5]]
    k = [[1, 1], [-2, 0.5], [0, 2]]
    v = [[1, 2], [-1, 0], [3, 1.5]]
    for causal in (False, True):
        o, lse = attention_fp8(q8, k8, v8, dq, dk, dv, causal, scale)
        for i in range(3):
            keys = range(i + 1) if causal else range(3)
            s = [scale * sum(dq * q[i][t] * dk * k[j][t] for t in range(2)) for j in keys]
            z = sum(math.exp(x) for x in s)
            for t in range(2):
                want = sum(math.exp(x) / z * dv * v[j][t] for x, j in zip(s, keys))
                assert abs(o[i, t] - want) < 1e-14
            assert abs(lse[i] - math.log(z)) < 1e-14


def test_attention_fp8_descale_invariances():
    (q8, k8, v8), (dq, dk, dv) = W.make_inputs_fp8(1, 2, 50, 64, seed=21)
    q8, k8, v8 = q8.numpy(), k8.numpy(), v8.numpy()
    o, lse = attention_fp8(q8, k8, v8, dq, dk, dv, True, 0.125)
    o2, lse2 = attention_fp8(q8, k8, v8, 2 * dq, dk, 2 * dv, True, 0.0625)
    assert np.allclose(o2, 2 * o, rtol=1e-13, atol=1e-15)
    assert np.allclose(lse2, lse, rtol=1e-13, atol=1e-13)
    # the dequantised inputs through the 16-bit-path definition
    o3, lse3 = attention_3pass(dequantise(q8, dq), dequantise(k8, dk), dequantise(v8, dv), True, 0.125)
    assert np.array_equal(o3, o) and np.array_equal(lse3, lse)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,bc", [(64, 128), (128, 64), (64, 32)])
def test_online_fp8_exact_inputs_equal_exact_attention(causal, d, bc):
    (q8, k8, v8), (dq, dk, dv), scale = W.make_exact_fp8(1, 1, 300, d, seed=5)
    q8, k8, v8 = q8[0, 0].numpy(), k8[0, 0].numpy(), v8[0, 0].numpy()
    seen = []
    o, lse = attention_online_fp8(q8, k8, v8, dq, dk, dv, causal, scale, bc,
                                  trace=lambda j0, m, ps, pr: seen.append(np.abs(pr - ps).max() <= 1e-12 * ps.max()))
    assert all(seen)                        # every 2^8 P is (to fp64 rounding) a power of two on the E4M3 grid
    o_ref, lse_ref = attention_fp8(q8, k8, v8, dq, dk, dv, causal, scale)
    assert np.abs(o - o_ref).max() < 1e-12
    assert np.abs(lse - lse_ref).max() < 1e-12


def test_online_fp8_exact_inputs_reject_a_missing_shift():
    # planted mistake: rounding P without the 2^8 shift sends 2^-16 .. 2^-10 to 0
    (q8, k8, v8), (dq, dk, dv), scale = W.make_exact_fp8(1, 1, 300, 128, seed=5)
    q8, k8, v8 = q8[0, 0].numpy(), k8[0, 0].numpy(), v8[0, 0].numpy()
    o, _ = attention_online_fp8(q8, k8, v8, dq, dk, dv, False, scale, 64, shift=0)
    o_ref, _ = attention_fp8(q8, k8, v8, dq, dk, dv, False, scale)
    assert np.abs(o - o_ref).max() > 1e-6


@pytest.mark.parametrize("causal", [False, True])
def test_online_fp8_without_rounding_is_exact(causal):
    (q8, k8, v8), (dq, dk, dv) = W.make_inputs_fp8(1, 1, 333, 128, seed=8)
    q8, k8, v8 = q8[0, 0].numpy(), k8[0, 0].numpy(), v8[0, 0].numpy()
    scale = 1 / math.sqrt(128)
    o, lse = attention_online_fp8(q8, k8, v8, dq, dk, dv, causal, scale, 64, round_p=False)
    o_ref, lse_ref = attention_fp8(q8, k8, v8, dq, dk, dv, causal, scale)
    assert np.abs(o - o_ref).max() < 1e-12
    assert np.abs(lse - lse_ref).max() < 1e-12


def two_key_example(bc):
    # keys: index 0 with score 0, index 1 with score ln(256/101); V = -2 and 1
    scale = math.log(256.0 / 101.0)
    q8 = np.array([[0x38]], dtype=np.uint8)
    k8 = np.array([[0x00], [0x38]], dtype=np.uint8)
    v8 = np.array([[0xC0], [0x38]], dtype=np.uint8)
    # two rows so that the shapes agree: row 1 is a copy of row 0's query
    q8 = np.vstack([q8, q8])
    # explicit shift 8 and threshold 0.75 (base 2), which the numbers below follow
    return attention_online_fp8(q8, k8, v8, 1.0, 1.0, 1.0, False, scale, bc, tau=0.75 * math.log(2.0), shift=8)


def test_online_fp8_hand_example():
    # one tile: reference = ln(256/101); 2^8 P = [101, 256] -> E4M3 [104, 256]
    # (grid spacing 8 in [64, 128)); O = (104 * -2 + 256 * 1) / (101 + 256)
    o, lse = two_key_example(bc=2)
    assert abs(o[0, 0] - 48.0 / 357.0) < 1e-15
    assert abs(lse[0] - math.log(1.0 + 256.0 / 101.0)) < 1e-15
    # one key per tile: reference 0 after key 0 (2^8 P = 256 exactly); key 1
    # exceeds it by ln(256/101) > tau, so the reference moves: acc = -512 is
    # rescaled by 101/256 to -202, then + 256 * 1; l = 101 + 256
    o, lse = two_key_example(bc=1)
    assert abs(o[0, 0] - 54.0 / 357.0) < 1e-15
    assert abs(lse[0] - math.log(1.0 + 256.0 / 101.0)) < 1e-15


def test_online_fp8_quantisation_bound():
    # |O_model - O_exact| <= sum_j |round(p_j) - p_j| |v_j| / l with
    # |round(p) - p| <= max(2^-4 p, 2^-10) (half the E4M3 spacing: relative
    # 2^-4 for normal numbers, absolute 2^-10 among the subnormals), all p in
    # the units of the final reference
    (q8, k8, v8), (dq, dk, dv) = W.make_inputs_fp8(1, 1, 512, 64, seed=9)
    q8, k8, v8 = q8[0, 0].numpy(), k8[0, 0].numpy(), v8[0, 0].numpy()
    scale = 1 / 8
    tiles = []
    o, _ = attention_online_fp8(q8, k8, v8, dq, dk, dv, False, scale, 64,
                                trace=lambda j0, m, ps, pr: tiles.append((j0, m, ps)))
    o_ref, _ = attention_fp8(q8, k8, v8, dq, dk, dv, False, scale)
    v = dequantise(v8, dv)
    m_final = tiles[-1][1]
    num = np.zeros_like(o)
    den = np.zeros(o.shape[0])
    for j0, m, ps in tiles:
        f = np.exp(m - m_final)[:, None]
        half = np.maximum(ps * 2.0 ** -4, 2.0 ** -10)
        num += (half * f) @ np.abs(v[j0:j0 + ps.shape[1]])
        den += (ps * f).sum(axis=1)
    bound = num / den[:, None]
    err = np.abs(o - o_ref)
    assert (err <= bound * (1 + 1e-9)).all()
    assert err.max() > 1e-3 * bound.max()        # the rounding is really there


def test_online_fp8_reference_threshold():
    (q8, k8, v8), (dq, dk, dv) = W.make_inputs_fp8(1, 1, 640, 128, seed=10, sigma=1.0)
    q8, k8, v8 = q8[0, 0].numpy(), k8[0, 0].numpy(), v8[0, 0].numpy()
    scale = 1 / math.sqrt(128)
    ms, pmax = [], []
    attention_online_fp8(q8, k8, v8, dq, dk, dv, False, scale, 64,
                         trace=lambda j0, m, ps, pr: (ms.append(m), pmax.append(ps.max())))
    s = scale * dequantise(q8, dq) @ dequantise(k8, dk).T
    for t in range(1, len(ms)):
        tile_max = s[:, 64 * t:64 * (t + 1)].max(axis=1)
        moved = ms[t] != ms[t - 1]
        assert np.array_equal(moved, tile_max > ms[t - 1] + TAU)
        assert np.allclose(ms[t][moved], tile_max[moved], rtol=1e-13, atol=0)
    assert (ms[-1] >= s.max(axis=1) - TAU).all()
    # reading F4: 2^8 P never exceeds 2^(8 + 0.75)
    assert max(pmax) <= 2.0 ** (P_SHIFT + TAU_LOG2) * (1 + 1e-12)

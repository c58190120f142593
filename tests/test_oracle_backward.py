"""Pins of the backward oracle against things other than itself (CPU only)."""

import math

import numpy as np
import pytest
import torch

import oracle

import importlib
abm = importlib.import_module("oracle.backward")


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def loss(q, k, v, do, causal, scale):
    o, _ = oracle.attention_3pass(q, k, v, causal, scale)
    return float((o * do).sum())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [0.7, -0.4])
def test_finite_differences(causal, scale):
    """Central differences of the forward oracle's sum(O * dO) in every input entry (tiny head)."""
    n, d = 5, 3
    q, k, v, do = (rand((n, d), s) for s in (1, 2, 3, 4))
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, causal, scale)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = loss(args["q"], args["k"], args["v"], do, causal, scale)
            args[name] = xm
            fm = loss(args["q"], args["k"], args["v"], do, causal, scale)
            num[idx] = (fp - fm) / (2 * eps)
        assert np.allclose(num, g, atol=1e-7, rtol=1e-6), name


@pytest.mark.parametrize("causal", [False, True])
def test_torch_autograd_fp64(causal):
    """PyTorch's CPU fp64 scaled_dot_product_attention differentiated by autograd."""
    b, h, n, d = 2, 3, 37, 16
    q, k, v, do = (rand((b, h, n, d), s) for s in (5, 6, 7, 8))
    scale = 1.0 / math.sqrt(d)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    out.backward(torch.tensor(do))
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, causal, scale)
    for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.allclose(got, ref.numpy(), atol=1e-12, rtol=1e-10)


@pytest.mark.parametrize("causal", [False, True])
def test_column_sum_identities(causal):
    """Rows of dS sum to 0, so sum_j dK_j = 0; rows of P sum to 1, so sum_j dV_j = sum_i dO_i."""
    n, d = 41, 8
    q, k, v, do = (rand((n, d), s) for s in (9, 10, 11, 12))
    _, dk, dv, _ = oracle.attention_backward(q, k, v, do, causal, 0.5)
    assert np.allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    assert np.allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)


def test_delta_equals_do_dot_o():
    n, d = 33, 8
    q, k, v, do = (rand((n, d), s) for s in (13, 14, 15, 16))
    o, _ = oracle.attention_3pass(q, k, v, True, 0.3)
    _, _, _, delta = oracle.attention_backward(q, k, v, do, True, 0.3)
    assert np.allclose(delta, (do * o).sum(axis=1), atol=1e-12)


def test_batch_dims_match_per_head():
    q, k, v, do = (rand((2, 2, 9, 4), s) for s in (17, 18, 19, 20))
    full = oracle.attention_backward(q, k, v, do, False, 0.9)
    for b in range(2):
        for h in range(2):
            one = oracle.attention_backward(q[b, h], k[b, h], v[b, h], do[b, h], False, 0.9)
            for x, y in zip(full, one):
                assert np.allclose(x[b, h], y, atol=1e-14)


def test_rejects_non_f64():
    x = np.zeros((3, 2), dtype=np.float32)
    with pytest.raises(TypeError):
        oracle.attention_backward(x, x, x, x, False, 1.0)


def _mutant(kind):
    """A copy of the per-head backward with one planted mistake."""
    def head(q, k, v, do, causal, scale):
        n = q.shape[0]
        s = scale * (q @ k.T)
        vis = oracle.visible_mask(np.arange(n), n, causal)
        s = np.where(vis, s, -np.inf)
        e = np.exp(s - s.max(axis=1)[:, None])
        p = e / e.sum(axis=1)[:, None]
        dv = (p @ do) if kind == "dv_no_transpose" else p.T @ do
        dp = do @ v.T
        delta = (p * dp).sum(axis=1)
        if kind == "no_delta":
            delta = np.zeros_like(delta)
        ds = (dp - delta[:, None]) if kind == "ds_without_p" else p * (dp - delta[:, None])
        dq = (ds @ k) if kind == "dq_no_scale" else scale * (ds @ k)
        dk = scale * (ds @ q) if kind == "dk_no_transpose" else scale * (ds.T @ q)
        return dq, dk, dv, delta
    return head


@pytest.mark.parametrize("kind", ["dv_no_transpose", "no_delta", "ds_without_p", "dq_no_scale", "dk_no_transpose"])
def test_pins_catch_planted_mistakes(kind, monkeypatch):
    """Each planted mistake fails the autograd pin or a column-sum identity."""
    monkeypatch.setattr(abm, "_head_backward", _mutant(kind))
    caught = False
    for check in (lambda: test_torch_autograd_fp64(True), lambda: test_column_sum_identities(False)):
        try:
            check()
        except AssertionError:
            caught = True
    assert caught, kind

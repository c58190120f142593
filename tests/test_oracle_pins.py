"""Pins of the CPU oracle to facts outside itself (no GPU needed).

Each pin ties the oracle to something it does not compute itself: pure-Python
brute force of the attention definition on tiny inputs, the hand-worked
examples in tests/golden/, closed forms, invariants of softmax attention and
PyTorch's float64 CPU attention as a library special case.  The last group
plants mistakes in the oracle and checks that the pins catch every one.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oracle_mod

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "online_softmax_worked_examples.txt")


# ---------------------------------------------------------------- helpers

def _parse_value(tok):
    if tok.startswith("ln"):
        return math.log(float(tok[2:]))
    return float(tok)


def load_golden():
    ex = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, field, vals = (p.strip() for p in line.split("|"))
            ex.setdefault(name, {})[field] = np.array([_parse_value(t) for t in vals.split()])
    return ex


def brute_force(q, k, v, causal, scale):
    """Attention from its definition with Python floats: exp(s) / sum exp(s).

    No max subtraction (inputs are small), math.fsum for exact-ish sums, plain
    loops.  Shares nothing with the oracle's NumPy code.
    """
    n, d = len(q), len(q[0])
    o = [[0.0] * d for _ in range(n)]
    lse = [0.0] * n
    for i in range(n):
        keys = range(i + 1) if causal else range(n)
        w = {}
        for j in keys:
            s = scale * math.fsum(q[i][t] * k[j][t] for t in range(d))
            w[j] = math.exp(s)
        z = math.fsum(w.values())
        lse[i] = math.log(z)
        for t in range(d):
            o[i][t] = math.fsum(w[j] * v[j][t] for j in keys) / z
    return np.array(o), np.array(lse)


def rand_head(rng, n, d, sigma=1.0):
    return tuple(rng.standard_normal((n, d)) * sigma for _ in range(3))


def attn3(q, k, v, causal, scale):
    return oracle.attention_3pass(q, k, v, causal, scale)


# ---------------------------------------------------------------- pins
# Each pin takes an attention callable (q, k, v, causal, scale) -> (O, LSE) on
# one head [N, d] so that the same pins can be run against planted mistakes.

def pin_bruteforce(attn):
    rng = np.random.default_rng(101)
    for n, d, causal, scale in [(1, 1, False, 1.0), (3, 2, False, 0.7), (5, 3, True, 0.5),
                                (7, 4, False, -0.3), (6, 3, True, 1.3), (4, 5, False, 0.0)]:
        q, k, v = rand_head(rng, n, d)
        o, lse = attn(q, k, v, causal, scale)
        ob, lb = brute_force(q.tolist(), k.tolist(), v.tolist(), causal, scale)
        np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-12)


def pin_golden(attn):
    ex = load_golden()
    for name, e in ex.items():
        q = e["q"].reshape(1, 1)
        n = e["k"].size
        # one query row: place it at the last position so that causal == non-causal
        qq = np.zeros((n, 1))
        qq[-1] = q[0]
        k = e["k"].reshape(n, 1)
        v = e["v"].reshape(n, 1)
        for causal in (False, True):
            o, lse = attn(qq, k, v, causal, 1.0)
            np.testing.assert_allclose(o[-1, 0], e["O"][0], rtol=1e-15, atol=1e-14)
            np.testing.assert_allclose(lse[-1], e["LSE"][0], rtol=1e-15, atol=1e-14)


def pin_constant_v(attn):
    rng = np.random.default_rng(7)
    for causal in (False, True):
        q, k, _ = rand_head(rng, 9, 4)
        c = rng.standard_normal(4)
        v = np.tile(c, (9, 1))
        o, _ = attn(q, k, v, causal, 0.8)
        np.testing.assert_allclose(o, np.tile(c, (9, 1)), rtol=0, atol=1e-14)


def pin_causal_row0(attn):
    rng = np.random.default_rng(8)
    q, k, v = rand_head(rng, 6, 3)
    scale = 0.9
    o, lse = attn(q, k, v, True, scale)
    np.testing.assert_array_equal(o[0], v[0])
    np.testing.assert_allclose(lse[0], scale * math.fsum(q[0] * k[0]), rtol=0, atol=1e-14)


def pin_scale_zero(attn):
    rng = np.random.default_rng(9)
    q, k, v = rand_head(rng, 8, 3)
    o, lse = attn(q, k, v, False, 0.0)
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (8, 1)), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, np.full(8, math.log(8)), rtol=0, atol=1e-14)
    o, lse = attn(q, k, v, True, 0.0)
    for i in range(8):
        np.testing.assert_allclose(o[i], v[: i + 1].mean(axis=0), rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[i], math.log(i + 1), rtol=0, atol=1e-14)


def pin_shift_invariance(attn):
    rng = np.random.default_rng(10)
    q, k, v = rand_head(rng, 7, 5)
    u = rng.standard_normal(5)
    scale = 0.6
    for causal in (False, True):
        o1, l1 = attn(q, k, v, causal, scale)
        o2, l2 = attn(q, k + u, v, causal, scale)
        np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l2, l1 + scale * (q @ u), rtol=0, atol=1e-12)


def pin_permutation(attn):
    rng = np.random.default_rng(11)
    q, k, v = rand_head(rng, 8, 3)
    perm = rng.permutation(8)
    o1, l1 = attn(q, k, v, False, 0.7)
    o2, l2 = attn(q, k[perm], v[perm], False, 0.7)       # joint key permutation
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-13)
    o3, l3 = attn(q[perm], k, v, False, 0.7)             # query permutation
    np.testing.assert_allclose(o3, o1[perm], rtol=0, atol=1e-13)
    np.testing.assert_allclose(l3, l1[perm], rtol=0, atol=1e-13)


def pin_torch_sdpa(attn):
    rng = np.random.default_rng(12)
    for n, d, causal, scale in [(16, 8, False, 0.35), (33, 16, True, 0.25), (20, 3, True, 1.7)]:
        q, k, v = rand_head(rng, n, d)
        o, lse = attn(q, k, v, causal, scale)
        tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
        ot = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
        s = scale * (tq @ tk.transpose(-1, -2))
        if causal:
            s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
        lt = torch.logsumexp(s, dim=-1)
        np.testing.assert_allclose(o, ot[0, 0].numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lt[0, 0].numpy(), rtol=0, atol=1e-12)


ALL_PINS = [pin_bruteforce, pin_golden, pin_constant_v, pin_causal_row0, pin_scale_zero,
            pin_shift_invariance, pin_permutation, pin_torch_sdpa]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin_3pass(pin):
    pin(attn3)


def online_as_attn(bc):
    def f(q, k, v, causal, scale):
        return oracle.attention_online(q, k, v, causal, scale, bc)
    return f


@pytest.mark.parametrize("bc", [1, 2, 3, 64])
@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin_online(pin, bc):
    pin(online_as_attn(bc))


# ---------------------------------------------------------------- more oracle facts

def test_rows_sum_to_one():
    rng = np.random.default_rng(13)
    for causal in (False, True):
        q, k, _ = rand_head(rng, 40, 16, sigma=2.0)
        p = oracle.softmax_probs(q, k, causal, 0.5)
        np.testing.assert_allclose(p.sum(axis=1), np.ones(40), rtol=0, atol=1e-13)
        assert (p >= 0).all()
        if causal:
            assert np.all(p[np.triu_indices(40, 1)] == 0.0)


@pytest.mark.parametrize("n", [1, 2, 3, 5, 17, 64, 130])
@pytest.mark.parametrize("d", [1, 3, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_online_equals_3pass(n, d, causal):
    rng = np.random.default_rng(1000 + 7 * n + d)
    q, k, v = rand_head(rng, n, d)
    scale = 1.0 / math.sqrt(d)
    o3, l3 = attn3(q, k, v, causal, scale)
    for bc in sorted({1, 2, 7, 16, n}):
        o, lse = oracle.attention_online(q, k, v, causal, scale, bc)
        np.testing.assert_allclose(o, o3, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, l3, rtol=0, atol=1e-12)


@pytest.mark.parametrize("tau", [0.0, 0.5, 3.0, 8.0 * math.log(2.0)])
@pytest.mark.parametrize("causal", [False, True])
def test_online_lazy_rescale_is_exact(tau, causal):
    """A reference max that lags the running max by <= tau gives the same O, LSE."""
    rng = np.random.default_rng(2024)
    q, k, v = rand_head(rng, 97, 16, sigma=1.5)
    k = k + rng.uniform(-4, 4, size=(97, 1))       # per-key offsets: frequent max jumps
    o3, l3 = attn3(q, k, v, causal, 0.5)
    for bc in (1, 7, 32):
        o, lse = oracle.attention_online(q, k, v, causal, 0.5, bc, rescale_threshold=tau)
        np.testing.assert_allclose(o, o3, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, l3, rtol=0, atol=1e-12)


def test_lazy_rescale_keeps_reference_within_threshold():
    """With the threshold, m never trails the true running max by more than tau."""
    rng = np.random.default_rng(7)
    q, k, v = rand_head(rng, 40, 8, sigma=2.0)
    tau = 2.0
    seen = []
    oracle.attention_online(q, k, v, False, 1.0, 4, rescale_threshold=tau,
                            trace=lambda j0, m, l, acc: seen.append((j0, m)))
    s = q @ k.T
    for j0, m in seen:
        true_max = s[:, : j0 + 4].max(axis=1)
        assert np.all(m <= true_max + 1e-12) and np.all(true_max - m <= tau + 1e-12)


def test_online_state_matches_golden_steps():
    ex = load_golden()
    for name, e in ex.items():
        n = e["k"].size
        states = {}
        oracle.attention_online(e["q"].reshape(1, 1) * np.ones((n, 1)), e["k"].reshape(n, 1),
                                e["v"].reshape(n, 1), False, 1.0, 1,
                                trace=lambda j0, m, l, acc: states.__setitem__(j0, (m, l, acc)))
        for j0 in range(n):
            key = f"state{j0}_m_l_acc"
            if key in e:
                m, l, acc = states[j0]
                np.testing.assert_allclose([m[0], l[0], acc[0, 0]], e[key], rtol=1e-15, atol=1e-15)


def test_online_state_invariant():
    """After each tile: m = max of seen scores, l = sum exp(s - m), acc = sum exp(s - m) v."""
    rng = np.random.default_rng(14)
    n, d, bc, scale = 11, 3, 4, 0.8
    q, k, v = rand_head(rng, n, d)
    for causal in (False, True):
        def check(j0, m, l, acc):
            seen = min(j0 + bc, n)
            for i in range(n):
                keys = [j for j in range(seen) if (not causal or j <= i)]
                if not keys:
                    assert m[i] == -math.inf and l[i] == 0 and np.all(acc[i] == 0)
                    continue
                s = [scale * math.fsum(q[i] * k[j]) for j in keys]
                mi = max(s)
                assert abs(m[i] - mi) < 1e-13
                assert abs(l[i] - math.fsum(math.exp(x - mi) for x in s)) < 1e-12
                for t in range(d):
                    ref = math.fsum(math.exp(x - mi) * v[j, t] for x, j in zip(s, keys))
                    assert abs(acc[i, t] - ref) < 1e-12
        oracle.attention_online(q, k, v, causal, scale, bc, trace=check)


def test_rows_subset_and_batch_dims():
    rng = np.random.default_rng(15)
    q, k, v = (rng.standard_normal((2, 3, 50, 8)) for _ in range(3))
    o, lse = oracle.attention_3pass(q, k, v, True, 0.4, chunk=7)
    rows = np.array([0, 13, 49])
    o2, l2 = oracle.attention_3pass(q, k, v, True, 0.4, rows=rows)
    # chunking changes BLAS blocking only: agreement to rounding
    np.testing.assert_allclose(o2, o[..., rows, :], rtol=0, atol=1e-14)
    np.testing.assert_allclose(l2, lse[..., rows], rtol=0, atol=1e-14)
    for b in range(2):
        for h in range(3):
            oh, lh = oracle.attention_3pass(q[b, h], k[b, h], v[b, h], True, 0.4)
            np.testing.assert_allclose(oh, o[b, h], rtol=0, atol=1e-14)
            np.testing.assert_allclose(lh, lse[b, h], rtol=0, atol=1e-14)


def test_large_logits_stay_finite():
    """Scores far beyond exp's range: the safe softmax keeps O and LSE finite."""
    q = np.array([[30.0], [-30.0], [1.0]])
    k = np.array([[30.0], [29.0], [-30.0]])
    v = np.array([[1.0], [2.0], [3.0]])
    o, lse = oracle.attention_3pass(q, k, v, False, 1.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    # row 0: scores 900, 870, -900 -> essentially all weight on key 0
    assert abs(o[0, 0] - 1.0) < 1e-12 and abs(lse[0] - 900.0) < 1e-12


def test_rejects_non_float64():
    x = np.zeros((4, 2), dtype=np.float32)
    with pytest.raises(TypeError):
        oracle.attention_3pass(x, x, x, False, 1.0)


# ---------------------------------------------------------------- planted mistakes

def _mut_transposed_scores(q, k, v, causal, scale, rows):
    # roles of Q and K swapped: s_ij = k_i . q_j
    return _finish(scale * (k[rows] @ q.T), v, rows, causal)


def _finish(s, v, rows, causal, lse_with_max=True, normalise=True, diag=True, flip=False):
    n = v.shape[0]
    j = np.arange(n)[None, :]
    i = np.asarray(rows)[:, None]
    if causal:
        vis = (j >= i) if flip else ((j <= i) if diag else (j < i))
        s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    p = e / l[:, None] if normalise else e
    lse = (m + np.log(l)) if lse_with_max else np.log(l)
    return p @ v, lse, p


MUTANTS = {
    "transposed_scores": _mut_transposed_scores,
    "causal_flipped": lambda q, k, v, c, sc, r: _finish(sc * (q[r] @ k.T), v, r, c, flip=True),
    "causal_no_diagonal": lambda q, k, v, c, sc, r: _finish(sc * (q[r] @ k.T), v, r, c, diag=False),
    "lse_drops_max": lambda q, k, v, c, sc, r: _finish(sc * (q[r] @ k.T), v, r, c, lse_with_max=False),
    "no_normalise": lambda q, k, v, c, sc, r: _finish(sc * (q[r] @ k.T), v, r, c, normalise=False),
    "scale_dropped": lambda q, k, v, c, sc, r: _finish(q[r] @ k.T, v, r, c),
    "scale_squared": lambda q, k, v, c, sc, r: _finish(sc * sc * (q[r] @ k.T), v, r, c),
    "v_rows_reversed": lambda q, k, v, c, sc, r: _finish(sc * (q[r] @ k.T), v[::-1], r, c),
    "k_for_v": lambda q, k, v, c, sc, r: _finish(sc * (q[r] @ k.T), k, r, c),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes_3pass(name, monkeypatch):
    monkeypatch.setattr(oracle_mod, "_head_3pass", MUTANTS[name])
    failures = 0
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(attn3)
        except AssertionError:
            failures += 1
    assert failures >= 1, f"no pin caught mutant {name}"


def _online_mutant(kind):
    """A copy of the online update with one planted mistake."""
    def f(q, k, v, causal, scale):
        n, d = q.shape
        rows = np.arange(n)
        m = np.full(n, -np.inf)
        l = np.zeros(n)
        acc = np.zeros((n, d))
        bc = 2
        for j0 in range(0, n, bc):
            j1 = min(j0 + bc, n)
            s = scale * (q @ k[j0:j1].T)
            vis = oracle.visible_mask(rows, j1, causal)[:, j0:j1]
            s = np.where(vis, s, -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            dead = np.isneginf(m_new)
            ref = np.where(dead, 0.0, m_new)
            alpha = np.where(dead, 1.0, np.exp(m - ref))
            p = np.exp(s - ref[:, None])
            if kind == "l_not_rescaled":
                l = l + p.sum(axis=1)
            elif kind == "l_not_accumulated":
                l = alpha * l
            else:
                l = alpha * l + p.sum(axis=1)
            if kind == "acc_not_rescaled":
                acc = acc + p @ v[j0:j1]
            else:
                acc = alpha[:, None] * acc + p @ v[j0:j1]
            if kind != "m_not_updated":
                m = m_new
        with np.errstate(all="ignore"):
            return acc / l[:, None], m + np.log(l)
    return f


@pytest.mark.parametrize("kind", ["l_not_rescaled", "l_not_accumulated", "acc_not_rescaled", "m_not_updated"])
def test_pins_catch_planted_mistakes_online(kind):
    failures = 0
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(_online_mutant(kind))
        except AssertionError:
            failures += 1
    assert failures >= 1, f"no pin caught online mutant {kind}"

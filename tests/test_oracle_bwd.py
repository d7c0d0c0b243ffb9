"""Pins of the fp64 backward oracle (``oracle.attention_bwd``).

The pages describe the backward pass only by what it keeps and recomputes, so
the oracle is the chain rule through the forward definition. It is pinned
here against things other than that derivation: central finite differences of
the forward oracle, torch.autograd through a plain float64 softmax attention,
the invariants the softmax fixes (each row of P sums to 1, a shift of a row of
scores changes nothing) and closed forms (one key; uniform attention).
"""
import numpy as np
import pytest
import torch

import oracle


def _data(seed, bh, n, d):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((bh, n, d)) for _ in range(4)]


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_matches_finite_differences(causal):
    q, k, v, g = _data(11 + causal, 2, 6, 5)
    scale = 0.7
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, scale, causal)

    def loss(q_, k_, v_):
        o, _ = oracle.attention(q_, k_, v_, scale, causal)
        return float(np.sum(o * g))

    h = 1e-5
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [xp if t is x else t for t in (q, k, v)]
            args_m = [xm if t is x else t for t in (q, k, v)]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.max(np.abs(num - grad)) < 1e-7, name


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_matches_autograd(causal):
    q, k, v, g = _data(21 + causal, 3, 37, 16)
    scale = 0.25
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, scale, causal)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = scale * torch.matmul(tq, tk.transpose(-1, -2).contiguous())
    if causal:
        n = q.shape[1]
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), tv)
    o.backward(torch.tensor(g))
    for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_invariants(causal):
    q, k, v, g = _data(31 + causal, 2, 50, 8)
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, 0.5, causal)
    # every row of dS sums to zero (shift invariance), so the keys' gradients cancel
    assert np.max(np.abs(dk.sum(axis=1))) < 1e-12 * max(1.0, np.abs(dk).max()) * 50
    # every row of P sums to one, so the values' gradients add up to the output gradient
    np.testing.assert_allclose(dv.sum(axis=1), g.sum(axis=1), rtol=1e-12, atol=1e-12)


def test_bwd_closed_forms():
    # one key: O = v, so dv = dO and nothing reaches q or k
    q, k, v, g = _data(41, 2, 1, 8)
    for causal in (False, True):
        dq, dk, dv = oracle.attention_bwd(q, k, v, g, 1.3, causal)
        np.testing.assert_array_equal(dv, g)
        assert np.all(dq == 0) and np.all(dk == 0)
    # q = 0: uniform weights 1/n; dv_j = mean_i dO_i, dk = 0,
    # dq_i = scale/n * sum_j (dO_i . (v_j - mean v)) k_j
    _, k, v, g = _data(42, 1, 9, 4)
    q = np.zeros_like(k)
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, 0.8, False)
    n = k.shape[1]
    np.testing.assert_allclose(dv[0], np.repeat(g[0].mean(axis=0, keepdims=True), n, axis=0), atol=1e-14)
    assert np.max(np.abs(dk)) < 1e-15
    vc = v[0] - v[0].mean(axis=0)
    np.testing.assert_allclose(dq[0], 0.8 / n * (g[0] @ vc.T) @ k[0], atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_row_and_column_samplers_match_full_backward(causal):
    # the samplers used at full size against the full chain-rule oracle
    rng = np.random.default_rng(31 + causal)
    n, d = 203, 16
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    dq, dk, dv = oracle.attention_bwd(q[None], k[None], v[None], g[None], 0.3, causal)
    idx = np.array([0, 1, 2, 63, 64, 127, 128, 150, 201, 202])
    np.testing.assert_allclose(oracle.attention_bwd_rows(q, k, v, g, idx, 0.3, causal), dq[0][idx],
                               rtol=0, atol=1e-12)
    sk, sv = oracle.attention_bwd_cols(q, k, v, g, idx, 0.3, causal)
    np.testing.assert_allclose(sk, dk[0][idx], rtol=0, atol=1e-12)
    np.testing.assert_allclose(sv, dv[0][idx], rtol=0, atol=1e-12)

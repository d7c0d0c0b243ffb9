"""The pages' tiled online-softmax attention, in fp64 numpy (test infrastructure).

Used only to pin the plain oracle against the algorithm the pages describe:
the online-softmax recurrence ("FlashAttention系列优化", FlashAttentionV1 /
算法设计 pseudocode: running max m and running sum d with the e^(m_old - m_new)
correction), the FlashAttention-2 update of the unscaled output
(same page, FlashAttentionV2 equations: O2 = diag(e^(m1-m2)) O1 + e^(S2-m2) V2,
then one final diag(l)^-1), and the logsumexp L = m + log l kept by the forward
pass (91haoming.cn article, FlashAttention v2 / forward pass improvements).

Row blocks of Br queries form the outer loop, column blocks of Bc keys the inner
loop (FlashAttention-2 loop order, "Flash Attention 再学习", FlashAttention v2
section). Nothing here is shared with the HIP library.
"""
from __future__ import annotations

import numpy as np


def online_softmax(x):
    """Two-pass online softmax of a 1-D vector, element by element (pseudocode of
    the FlashAttentionV1 section; the output index is read as i, see the
    readings list). Returns (y, m, d)."""
    m = -np.inf
    dsum = 0.0
    for xj in x:
        m_new = max(m, xj)
        # the e^(m_old - m_new) factor corrects the running sum to the new max
        corr = 0.0 if m == -np.inf else np.exp(m - m_new)
        dsum = dsum * corr + np.exp(xj - m_new)
        m = m_new
    y = np.array([np.exp(xi - m) / dsum for xi in x])
    return y, m, dsum


def tiled_attention(q, k, v, Br: int, Bc: int, scale: float = 1.0, causal: bool = False,
                    dtype=np.float64):
    """One head, q [N, d], k/v [N_k, d]. Returns (O [N, d], L [N]).

    Tiles may be larger than N or not divide it. Masked scores are -inf; a
    correction factor between two -inf maxima is taken as 0 (the reading for
    rows with nothing visible yet).
    """
    q = np.asarray(q, dtype=dtype)
    k = np.asarray(k, dtype=dtype)
    v = np.asarray(v, dtype=dtype)
    n, d = q.shape
    nk = k.shape[0]
    out = np.zeros((n, d), dtype=dtype)
    lse = np.zeros((n,), dtype=dtype)
    for r0 in range(0, n, Br):
        rows = np.arange(r0, min(r0 + Br, n))
        qi = q[rows]
        acc = np.zeros((len(rows), d), dtype=dtype)     # unscaled output
        ell = np.zeros((len(rows),), dtype=dtype)       # unscaled running sum
        m = np.full((len(rows),), -np.inf, dtype=dtype)  # running row max
        for c0 in range(0, nk, Bc):
            cols = np.arange(c0, min(c0 + Bc, nk))
            s = (qi @ k[cols].T) * dtype(scale)
            if causal:
                s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
            m_new = np.maximum(m, s.max(axis=1))
            finite = np.isfinite(m_new)
            safe_m = np.where(finite, m_new, 0.0)
            alpha = np.where(np.isfinite(m), np.exp(m - safe_m), 0.0)
            p = np.exp(s - safe_m[:, None])
            ell = alpha * ell + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ v[cols]
            m = m_new
        with np.errstate(divide="ignore", invalid="ignore"):
            out[rows] = np.where(ell[:, None] > 0, acc / ell[:, None], 0.0)
            lse[rows] = np.where(ell > 0, m + np.log(ell), -np.inf)
    return out, lse


def merge_partials(ms, ls, accs):
    """Combine per-chunk partial states (m_k, l_k, unscaled acc_k) of one row with
    the same rescale identity the FlashAttention-2 update uses. Returns (O, L)."""
    ms = np.asarray(ms, dtype=np.float64)
    ls = np.asarray(ls, dtype=np.float64)
    accs = np.asarray(accs, dtype=np.float64)
    mm = np.max(ms)
    w = np.where(np.isfinite(ms), np.exp(ms - mm), 0.0)
    ell = np.sum(w * ls)
    o = (w[:, None] * accs).sum(axis=0) / ell
    return o, mm + np.log(ell)

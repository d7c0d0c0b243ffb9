"""Block-sparse attention with dropout: plain fp64 CPU reference.

TEST INFRASTRUCTURE ONLY (see the package docstring): only the test suite,
the package smoke check and the benchmark's CPU leg use it; it shares no code
with the HIP library.

What it computes, per (batch, head), written out from the definitions:
  s_ij = scale * q_i . k_j, visible iff block_mask[i // 128][j // 128] != 0
         and (not causal or j <= i)     (block-sparse FlashAttention, 91haoming
         .cn FlashAttention v1-v3 article, v1 results: attention restricted to
         the kept blocks of a block mask; 128 x 128 blocks)
  p_ij = softmax over the visible keys of row i (row with none: all 0)
  o_i  = sum_j p_ij z_ij / (1 - p_drop) v_j, z_ij = keep decision (dropout on
         the attention weights, the "masking and dropout" of the same article)
  L_i  = logsumexp of the visible scores (before dropout)
The keep decision uses Philox4x32-10 as published by Salmon, Moraes, Dror and
Shaw ("Parallel random numbers: as easy as 1, 2, 3", SC 2011): key (seed low,
seed high 32 bits), counter (j // 4, i, b * H + h, 0); z_ij = 0 iff word j % 4
of the output is below floor(p_drop * 2^32), p_drop taken as the float32
value the C interface receives.
"""
from __future__ import annotations

import numpy as np

_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x32 with 10 rounds on uint32 arrays (broadcast); returns 4 arrays."""
    c = [np.asarray(x, dtype=np.uint64) & _MASK32 for x in (c0, c1, c2, c3)]
    key0, key1 = k0 & 0xFFFFFFFF, k1 & 0xFFFFFFFF
    for _ in range(10):
        p0 = _M0 * c[0]
        p1 = _M1 * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c = [hi1 ^ c[1] ^ np.uint64(key0), lo1, hi0 ^ c[3] ^ np.uint64(key1), lo0]
        key0 = (key0 + _W0) & 0xFFFFFFFF
        key1 = (key1 + _W1) & 0xFFFFFFFF
    return [x.astype(np.uint32) for x in c]


def _as_f32(p: float) -> float:
    return float(np.float32(p))


def drop_threshold(p_drop: float) -> int:
    """floor(p * 2^32) for the probability as the library receives it: the
    dropout_p argument of the C interface is a 32-bit float, so p is first
    rounded to float32 (0.1 gives 429496736, not 429496729)."""
    return int(_as_f32(p_drop) * 4294967296.0)


def keep_rows(rows, n: int, bh: int, p_drop: float, seed: int) -> np.ndarray:
    """z [len(rows), n] (bool): keep decisions of query rows `rows` against
    keys 0..n-1 of head bh; True where the weight is kept."""
    rows = np.asarray(rows, dtype=np.uint64).reshape(-1)
    thr = drop_threshold(p_drop)
    if thr == 0:
        return np.ones((rows.size, n), dtype=bool)
    i = rows[:, None]
    j4 = np.arange((n + 3) // 4, dtype=np.uint64)[None, :]
    words = philox4x32_10(j4, i, np.uint64(bh), np.uint64(0), seed & 0xFFFFFFFF, seed >> 32)
    u = np.stack(words, axis=-1).reshape(rows.size, -1)[:, :n]   # u[r, j] = word j % 4 of counter j // 4
    return u >= np.uint32(thr)


def keep_mask(n: int, bh: int, p_drop: float, seed: int) -> np.ndarray:
    """z [n, n] (bool) of one head: True where the weight is kept."""
    return keep_rows(np.arange(n), n, bh, p_drop, seed)


def block_sparse_attention(q, k, v, block_mask, scale: float, causal: bool, p_drop: float = 0.0,
                           seed: int = 0, block: int = 128):
    """q, k, v [B, H, N, d] (any float); block_mask [nb, nb]. Returns (o, lse) fp64."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    bm = np.asarray(block_mask) != 0
    B, H, N, d = q.shape
    idx = np.arange(N)
    vis = bm[idx[:, None] // block, idx[None, :] // block]
    if causal:
        vis &= idx[None, :] <= idx[:, None]
    o = np.zeros((B, H, N, d))
    lse = np.full((B, H, N), -np.inf)
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h] @ k[b, h].T)
            s = np.where(vis, s, -np.inf)
            m = s.max(axis=1)
            rows = np.isfinite(m)
            e = np.zeros_like(s)
            e[rows] = np.exp(s[rows] - m[rows, None])
            l = e.sum(axis=1)
            p = np.zeros_like(s)
            p[rows] = e[rows] / l[rows, None]
            z = keep_mask(N, b * H + h, p_drop, seed)
            o[b, h] = (p * z / (1.0 - _as_f32(p_drop))) @ v[b, h]
            lse[b, h, rows] = m[rows] + np.log(l[rows])
    return o, lse


def block_sparse_attention_rows(q_rows, rows, k, v, block_mask, scale: float, causal: bool, bh: int,
                                p_drop: float = 0.0, seed: int = 0, block: int = 128):
    """The same definition for selected query rows of one head.

    q_rows [R, d] are the queries at positions `rows`; k, v [N, d]; bh = b * H
    + h names the head in the dropout counter. Returns (o [R, d], lse [R]) fp64.
    """
    q_rows, k, v = (np.asarray(x, dtype=np.float64) for x in (q_rows, k, v))
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    bm = np.asarray(block_mask) != 0
    n = k.shape[0]
    j = np.arange(n)
    vis = bm[rows[:, None] // block, j[None, :] // block]
    if causal:
        vis &= j[None, :] <= rows[:, None]
    s = np.where(vis, scale * (q_rows @ k.T), -np.inf)
    m = s.max(axis=1)
    live = np.isfinite(m)
    e = np.zeros_like(s)
    e[live] = np.exp(s[live] - m[live, None])
    l = e.sum(axis=1)
    p = np.zeros_like(s)
    p[live] = e[live] / l[live, None]
    z = keep_rows(rows, n, bh, p_drop, seed)
    o = (p * z / (1.0 - _as_f32(p_drop))) @ v
    lse = np.full(rows.size, -np.inf)
    lse[live] = m[live] + np.log(l[live])
    return o, lse

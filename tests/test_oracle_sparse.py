"""Pins of the block-sparse / dropout oracle (oracle/sparse.py): the Philox
known-answer vectors of the generator's publication (tests/golden), reduction
to the plain attention oracle when every block is kept, independence of
diagonal blocks, empty rows, the keep rate, and unbiasedness of dropout (the
mean over seeds approaches the output without dropout)."""
import os

import numpy as np
import pytest

import oracle
from oracle import sparse

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def test_philox_known_answers():
    n = 0
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        c, k, o = [[int(x, 16) for x in part.split()] for part in line.split("|")]
        got = sparse.philox4x32_10(*[np.array([x], dtype=np.uint64) for x in c], k[0], k[1])
        assert [int(g[0]) for g in got] == o
        n += 1
    assert n == 3


def _qkv(seed, B, H, N, d):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, N, d)) for _ in range(3)]


@pytest.mark.parametrize("causal", [False, True])
def test_full_mask_is_plain_attention(causal):
    q, k, v = _qkv(1, 1, 2, 300, 16)
    nb = 3
    o, l = sparse.block_sparse_attention(q, k, v, np.ones((nb, nb)), 0.25, causal)
    ro, rl = oracle.attention(q, k, v, 0.25, causal)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, rl, rtol=0, atol=1e-12)


def test_diagonal_blocks_are_independent_and_empty_rows():
    q, k, v = _qkv(2, 1, 1, 300, 8)
    mask = np.eye(3)
    mask[2, 2] = 0                                   # block row 2 keeps nothing
    o, l = sparse.block_sparse_attention(q, k, v, mask, 0.5, False)
    for b in range(2):
        sl = slice(128 * b, 128 * (b + 1))
        ro, rl = oracle.attention(q[:, :, sl], k[:, :, sl], v[:, :, sl], 0.5, False)
        np.testing.assert_allclose(o[:, :, sl], ro, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l[:, :, sl], rl, rtol=0, atol=1e-12)
    assert np.all(o[:, :, 256:] == 0) and np.all(np.isneginf(l[:, :, 256:]))


def test_keep_rate_and_unbiased_dropout():
    z = sparse.keep_mask(512, 3, 0.3, seed=1234)
    frac = z.mean()
    assert abs(frac - 0.7) < 5 * np.sqrt(0.3 * 0.7 / z.size)
    q, k, v = _qkv(3, 1, 1, 40, 4)
    ref, _ = sparse.block_sparse_attention(q, k, v, np.ones((1, 1)), 0.5, True)
    acc = np.zeros_like(ref)
    for s in range(400):
        o, _ = sparse.block_sparse_attention(q, k, v, np.ones((1, 1)), 0.5, True, p_drop=0.25, seed=s)
        acc += o
    assert np.max(np.abs(acc / 400 - ref)) < 0.08

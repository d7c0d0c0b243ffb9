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


# ------------------------------------------------------------------------------------
# The (query, key) -> generator mapping of the dropout decision, pinned apart from the
# vectorised oracle: a scalar Philox4x32-10 written from the generator's published
# definition (ten rounds of two 32x32->64 multiplies with the round keys bumped by the
# Weyl constants), checked against the same known answers, then a per-element loop that
# applies the contract of fa_fwd_block_sparse in include/fa.h literally:
#   counter (j / 4, i, b * H + h, 0), key (seed low, seed high), word j % 4,
#   dropped iff that word < floor(dropout_p * 2^32), dropout_p the float32 argument.

def _philox_scalar(counter, key):
    mul = (0xD2511F53, 0xCD9E8D57)
    weyl = (0x9E3779B9, 0xBB67AE85)
    x = list(counter)
    k = list(key)
    for _ in range(10):
        prod_a = mul[0] * x[0]
        prod_b = mul[1] * x[2]
        x = [((prod_b >> 32) ^ x[1] ^ k[0]) & 0xFFFFFFFF, prod_b & 0xFFFFFFFF,
             ((prod_a >> 32) ^ x[3] ^ k[1]) & 0xFFFFFFFF, prod_a & 0xFFFFFFFF]
        k = [(k[0] + weyl[0]) & 0xFFFFFFFF, (k[1] + weyl[1]) & 0xFFFFFFFF]
    return x


def test_scalar_philox_known_answers():
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        c, k, o = [[int(x, 16) for x in part.split()] for part in line.split("|")]
        assert _philox_scalar(c, k) == o


def _kept_by_contract(i, j, bh, p_drop, seed):
    thr = int(float(np.float32(p_drop)) * 2 ** 32)
    words = _philox_scalar((j // 4, i, bh, 0), (seed & 0xFFFFFFFF, seed >> 32))
    return not (words[j % 4] < thr)


def test_keep_mask_known_answer_word_order():
    # counter (0, 0, 0, 0), key (0, 0) is the first known-answer vector: words
    # 6627e8d5 e169c58d bc57ac4c 9b00dbd8. With p = 0.7 the threshold is
    # 0xb3333300 (float32(0.7) * 2^32), so words 0 and 3 drop, 1 and 2 keep:
    # query 0, keys 0..3 of head 0 with seed 0 read exactly those words in order.
    assert sparse.drop_threshold(0.7) == 0xB3333300
    z = sparse.keep_mask(4, 0, 0.7, seed=0)
    assert z[0].tolist() == [False, True, True, False]


@pytest.mark.parametrize("seed", [0, 0x1234_5678_9ABC_DEF0, 11])
def test_keep_mask_matches_contract_per_element(seed):
    # i != j, j % 4 != 0, rows and heads with distinct values, so a swapped
    # counter word or a wrong word index would show
    n = 37
    for bh, p in ((0, 0.1), (5, 0.25), (1023, 0.5)):
        z = sparse.keep_mask(n, bh, p, seed)
        for i, j in ((0, 1), (3, 30), (17, 6), (36, 35), (9, 9), (2, 27), (30, 3)):
            assert bool(z[i, j]) == _kept_by_contract(i, j, bh, p, seed), (bh, p, i, j)
        r = sparse.keep_rows([3, 30, 17], n, bh, p, seed)
        for a, i in enumerate((3, 30, 17)):
            for j in (1, 2, 3, 5, 6, 7, 29, 30, 31, 33):
                assert bool(r[a, j]) == _kept_by_contract(i, j, bh, p, seed)


def test_threshold_uses_float32_probability():
    assert sparse.drop_threshold(0.1) == 429496736          # float32(0.1) * 2^32, floored
    assert sparse.drop_threshold(0.5) == 2 ** 31
    assert sparse.drop_threshold(0.0) == 0


@pytest.mark.parametrize("causal,p_drop", [(False, 0.0), (True, 0.0), (True, 0.3)])
def test_rows_match_full_definition(causal, p_drop):
    q, k, v = _qkv(4, 1, 2, 300, 16)
    rng = np.random.default_rng(5)
    mask = (rng.random((3, 3)) < 0.6).astype(np.uint8)
    mask[1, :] = 0
    o, l = sparse.block_sparse_attention(q, k, v, mask, 0.3, causal, p_drop=p_drop, seed=99)
    rows = np.array([0, 1, 127, 128, 129, 200, 255, 256, 299])
    for h in range(2):
        ro, rl = sparse.block_sparse_attention_rows(q[0, h][rows], rows, k[0, h], v[0, h], mask, 0.3, causal,
                                                    bh=h, p_drop=p_drop, seed=99)
        np.testing.assert_allclose(ro, o[0, h][rows], rtol=0, atol=1e-12)
        np.testing.assert_array_equal(np.isfinite(rl), np.isfinite(l[0, h][rows]))
        fin = np.isfinite(rl)
        np.testing.assert_allclose(rl[fin], l[0, h][rows][fin], rtol=0, atol=1e-12)

"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: the worked
example of the "FlashAttention系列优化" code listing (agreement of its naive and
tiled forms, since the page prints no values), closed forms, invariants,
library routines (scipy logsumexp / softmax, torch casts), the OCP E4M3 spec
points, and pure-Python brute force on tiny inputs.
"""
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import online
from exact_attention_106_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _masked_scores(q, k, scale, causal):
    s = scale * (q @ k.T)
    if causal:
        n, m = s.shape
        s = np.where(np.arange(m)[None, :] > np.arange(n)[:, None], -np.inf, s)
    return s


# --- P1: the page's worked example (seed 456, 16 x 8, Br = 4, Bc = d = 8) ----------------

def test_config1_worked_example_agreement():
    c = inputs.config1()
    q = c.q[0, 0].double()
    k = c.k[0, 0].double()
    v = c.v[0, 0].double()
    # the listing's "expected_attention": softmax(Q K^T) V with torch, here in fp64
    expected = torch.softmax(q @ k.T, dim=1) @ v
    o, lse = oracle.attention(c.q.double().numpy(), c.k.double().numpy(), c.v.double().numpy(),
                              scale=1.0, causal=False)
    np.testing.assert_allclose(o[0, 0], expected.numpy(), rtol=0, atol=1e-14)
    # the listing's tiled loop with its tile sizes, in fp64 and in the listing's fp32
    to, tl = online.tiled_attention(q.numpy(), k.numpy(), v.numpy(), Br=4, Bc=8)
    np.testing.assert_allclose(o[0, 0], to, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], tl, rtol=0, atol=1e-14)
    to32, _ = online.tiled_attention(c.q[0, 0].numpy(), c.k[0, 0].numpy(), c.v[0, 0].numpy(),
                                     Br=4, Bc=8, dtype=np.float32)
    np.testing.assert_allclose(o[0, 0], to32, rtol=0, atol=1e-6)
    # the seed/generator reproduce the listing's first draw (uniform [0, 1))
    assert c.q.shape == (1, 1, 16, 8) and float(c.q.min()) >= 0.0 and float(c.q.max()) < 1.0


# --- P2: tiled online softmax == 3-pass, any tile sizes ------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d,br,bc", [(37, 5, 4, 8), (50, 16, 7, 13), (9, 3, 16, 32), (64, 8, 64, 1)])
def test_tiled_equals_three_pass(n, d, br, bc, causal):
    rng = np.random.default_rng(n * 100 + d)
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    o, lse = oracle.attention(q, k, v, scale=0.37, causal=causal)
    to, tl = online.tiled_attention(q, k, v, Br=br, Bc=bc, scale=0.37, causal=causal)
    np.testing.assert_allclose(o, to, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, tl, rtol=0, atol=1e-12)


def test_online_softmax_pseudocode_equals_softmax():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(41) * 5
    y, m, dsum = online.online_softmax(x)
    np.testing.assert_allclose(y, scipy.special.softmax(x), rtol=1e-13, atol=0)
    assert m == x.max()
    np.testing.assert_allclose(m + math.log(dsum), scipy.special.logsumexp(x), rtol=1e-14)


# --- P3 / P4 / P10: normalisation, logsumexp, P itself -------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one(causal):
    rng = np.random.default_rng(3)
    q, k = _rand(rng, 2, 33, 12), _rand(rng, 2, 33, 12)
    v = np.ones((2, 33, 12))
    o, _ = oracle.attention(q, k, v, scale=0.5, causal=causal)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_lse_is_logsumexp(causal):
    rng = np.random.default_rng(4)
    q, k, v = _rand(rng, 45, 16), _rand(rng, 45, 16), _rand(rng, 45, 16)
    _, lse = oracle.attention(q, k, v, scale=0.25, causal=causal)
    ref = scipy.special.logsumexp(_masked_scores(q, k, 0.25, causal), axis=1)
    np.testing.assert_allclose(lse, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_identity_values_give_softmax(causal):
    rng = np.random.default_rng(5)
    n = 24
    q, k = _rand(rng, n, n), _rand(rng, n, n)
    o, lse = oracle.attention(q, k, np.eye(n), scale=0.3, causal=causal)
    s = _masked_scores(q, k, 0.3, causal)
    np.testing.assert_allclose(o, scipy.special.softmax(s, axis=1), rtol=0, atol=1e-14)
    with np.errstate(over="ignore"):
        np.testing.assert_allclose(o, np.exp(s - lse[:, None]), rtol=0, atol=1e-14)


def test_scale_is_applied_to_scores():
    rng = np.random.default_rng(6)
    q, k, v = _rand(rng, 10, 4), _rand(rng, 10, 4), _rand(rng, 10, 4)
    o1, l1 = oracle.attention(q, k, v, scale=2.0, causal=False)
    o2, l2 = oracle.attention(2.0 * q, k, v, scale=1.0, causal=False)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)


# --- P5 / P6 / P12: invariants -------------------------------------------------------------

def test_kv_permutation_invariance():
    rng = np.random.default_rng(7)
    q, k, v = _rand(rng, 30, 8), _rand(rng, 30, 8), _rand(rng, 30, 8)
    perm = rng.permutation(30)
    o, l = oracle.attention(q, k, v, 0.5, False)
    o2, l2 = oracle.attention(q, k[perm], v[perm], 0.5, False)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, l2, rtol=0, atol=1e-13)
    qp = rng.permutation(30)
    o3, l3 = oracle.attention(q[qp], k, v, 0.5, False)
    np.testing.assert_allclose(o3, o[qp], rtol=0, atol=0)
    np.testing.assert_allclose(l3, l[qp], rtol=0, atol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_orthogonal_rotation_invariance(causal):
    rng = np.random.default_rng(8)
    d = 32
    q, k, v = _rand(rng, 40, d), _rand(rng, 40, d), _rand(rng, 40, d)
    r = inputs.haar_orthogonal(np.random.Generator(np.random.PCG64(9)), d)
    o, l = oracle.attention(q, k, v, 0.2, causal)
    o2, l2 = oracle.attention(q @ r, k @ r, v, 0.2, causal)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, l2, rtol=0, atol=1e-12)


def test_causality_future_keys_do_not_matter():
    rng = np.random.default_rng(10)
    q, k, v = _rand(rng, 20, 6), _rand(rng, 20, 6), _rand(rng, 20, 6)
    o, l = oracle.attention(q, k, v, 1.0, True)
    k2, v2 = k.copy(), v.copy()
    k2[12:] = 1e3 * _rand(rng, 8, 6)
    v2[12:] = np.nan
    o2, l2 = oracle.attention(q, k2, v2, 1.0, True)
    np.testing.assert_array_equal(o[:12], o2[:12])
    np.testing.assert_array_equal(l[:12], l2[:12])


# --- P7: brute force on tiny inputs (pure Python, math.exp) --------------------------------

def _brute(q, k, v, scale, causal):
    n, d = len(q), len(q[0])
    out, lse = [], []
    for i in range(n):
        js = [j for j in range(len(k)) if (not causal or j <= i)]
        s = {j: scale * sum(q[i][c] * k[j][c] for c in range(d)) for j in js}
        m = max(s.values())
        w = {j: math.exp(s[j] - m) for j in js}
        tot = sum(w.values())
        out.append([sum(w[j] * v[j][c] for j in js) / tot for c in range(d)])
        lse.append(m + math.log(tot))
    return np.array(out), np.array(lse)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 1), (3, 2), (8, 8), (7, 5)])
def test_brute_force_tiny(n, d, causal):
    rng = np.random.default_rng(n * 7 + d)
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    o, l = oracle.attention(q, k, v, 0.7, causal)
    bo, bl = _brute(q.tolist(), k.tolist(), v.tolist(), 0.7, causal)
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, bl, rtol=0, atol=1e-13)


def test_brute_force_rectangular_and_batched():
    rng = np.random.default_rng(11)
    q, k, v = _rand(rng, 2, 3, 5, 4), _rand(rng, 2, 3, 7, 4), _rand(rng, 2, 3, 7, 4)
    o, l = oracle.attention(q, k, v, 0.9, False)
    for b in range(2):
        for h in range(3):
            bo, bl = _brute(q[b, h].tolist(), k[b, h].tolist(), v[b, h].tolist(), 0.9, False)
            np.testing.assert_allclose(o[b, h], bo, rtol=0, atol=1e-13)
            np.testing.assert_allclose(l[b, h], bl, rtol=0, atol=1e-13)


# --- P8 / P9 / P11: closed forms and limits ------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_mean_of_visible_values(causal):
    rng = np.random.default_rng(12)
    n = 17
    v = _rand(rng, n, 5)
    o, l = oracle.attention(np.zeros((n, 5)), _rand(rng, n, 5), v, 1.0, causal)
    for i in range(n):
        cnt = i + 1 if causal else n
        np.testing.assert_allclose(o[i], v[:cnt].mean(axis=0), rtol=0, atol=1e-14)
        np.testing.assert_allclose(l[i], math.log(cnt), rtol=0, atol=1e-14)


def test_single_key():
    rng = np.random.default_rng(13)
    q, k, v = _rand(rng, 1, 6), _rand(rng, 1, 6), _rand(rng, 1, 6)
    o, l = oracle.attention(q, k, v, 0.5, False)
    np.testing.assert_array_equal(o[0], v[0])
    np.testing.assert_allclose(l[0], 0.5 * float(q[0] @ k[0]), rtol=0, atol=1e-15)
    q, k, v = _rand(rng, 9, 6), _rand(rng, 9, 6), _rand(rng, 9, 6)
    o, l = oracle.attention(q, k, v, 0.5, True)
    np.testing.assert_array_equal(o[0], v[0])
    np.testing.assert_allclose(l[0], 0.5 * float(q[0] @ k[0]), rtol=0, atol=1e-15)


def test_large_logits_no_overflow_hard_attention_limit():
    rng = np.random.default_rng(14)
    q, k, v = _rand(rng, 12, 8), _rand(rng, 12, 8), _rand(rng, 12, 8)
    o, l = oracle.attention(q, k, v, 1e3, False)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    s = q @ k.T
    top = np.argmax(s, axis=1)
    srt = np.sort(s, axis=1)
    gap_ok = (srt[:, -1] - srt[:, -2]) * 1e3 > 50
    np.testing.assert_allclose(o[gap_ok], v[top[gap_ok]], rtol=0, atol=1e-12)


def test_empty_inputs():
    o, l = oracle.attention(np.zeros((0, 4)), np.zeros((0, 4)), np.zeros((0, 4)), 1.0, False)
    assert o.shape == (0, 4) and l.shape == (0,)


# --- rows API == full API -------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_rows_api_matches_full(causal):
    rng = np.random.default_rng(15)
    q, k, v = _rand(rng, 50, 8), _rand(rng, 50, 8), _rand(rng, 50, 8)
    o, l = oracle.attention(q, k, v, 0.4, causal)
    rows = np.array([0, 3, 49, 17])
    ro, rl = oracle.attention_rows(q[rows], rows, k, v, 0.4, causal)
    np.testing.assert_array_equal(ro, o[rows])
    np.testing.assert_array_equal(rl, l[rows])


# --- P13 / P14 / P15: paged decode ----------------------------------------------------------

def _small_pool(seed=21, nan_tails=True):
    return inputs.paged_pool(num_seqs=6, H=3, d=8, ctx_lo=1, ctx_hi=70, seed=seed,
                             share=0.5, nan_tails=nan_tails)


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def test_paged_decode_equals_gathered_attention():
    p = _small_pool()
    q = p.q.float().double().numpy()
    o, l = oracle.paged_decode(q, _bits(p.kcache), _bits(p.vcache), p.block_table.numpy(),
                               p.ctx_lens.numpy(), p.scale)
    kc = p.kcache.double().numpy()
    vc = p.vcache.double().numpy()
    bt = p.block_table.numpy()
    for s in range(q.shape[0]):
        ctx = int(p.ctx_lens[s])
        pages = bt[s, (np.arange(ctx) // 16)]
        slots = np.arange(ctx) % 16
        for h in range(q.shape[1]):
            kk = kc[pages, h, slots]
            vv = vc[pages, h, slots]
            ro, rl = oracle.attention(q[s, h][None], kk, vv, p.scale, False)
            np.testing.assert_allclose(o[s, h], ro[0], rtol=0, atol=1e-14)
            np.testing.assert_allclose(l[s, h], rl[0], rtol=0, atol=1e-14)
            # == the last row of a causal prefill whose last query is the decode query
            qq = np.concatenate([_rand(np.random.default_rng(s), ctx - 1, q.shape[2]), q[s, h][None]])
            po, pl = oracle.attention(qq, kk, vv, p.scale, True)
            np.testing.assert_allclose(o[s, h], po[-1], rtol=0, atol=1e-13)
            np.testing.assert_allclose(l[s, h], pl[-1], rtol=0, atol=1e-13)
        assert np.all(np.isfinite(o[s]))


def test_paged_decode_placement_invariance():
    p = _small_pool()
    kb, vb = _bits(p.kcache), _bits(p.vcache)
    bt = p.block_table.numpy()
    o, l = oracle.paged_decode(p.q.float().numpy(), kb, vb, bt, p.ctx_lens.numpy(), p.scale)
    # move every physical page to a new slot of a larger pool; unshare the pairs
    rng = np.random.default_rng(22)
    n = kb.shape[0]
    new_pos = rng.permutation(2 * n)[:n]
    kb2 = np.zeros((2 * n,) + kb.shape[1:], np.uint16)
    vb2 = np.zeros_like(kb2)
    kb2[new_pos], vb2[new_pos] = kb, vb
    bt2 = np.where(bt >= 0, new_pos[np.maximum(bt, 0)], -1).astype(np.int32)
    o2, l2 = oracle.paged_decode(p.q.float().numpy(), kb2, vb2, bt2, p.ctx_lens.numpy(), p.scale)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(l, l2)


def test_split_merge_identity():
    rng = np.random.default_rng(23)
    q, k, v = _rand(rng, 1, 16), _rand(rng, 100, 16), _rand(rng, 100, 16)
    o, l = oracle.attention(q, k, v, 0.25, False)
    bounds = [0, 7, 40, 41, 100]
    ms, ls, accs = [], [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        s = 0.25 * (k[a:b] @ q[0])
        m = s.max()
        w = np.exp(s - m)
        ms.append(m), ls.append(w.sum()), accs.append(w @ v[a:b])
    mo, ml = online.merge_partials(ms, ls, accs)
    np.testing.assert_allclose(mo, o[0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(ml, l[0], rtol=0, atol=1e-13)


# --- P16 / P17: input decoders --------------------------------------------------------------

def test_e4m3_decoder_spec_points():
    path = os.path.join(GOLDEN, "e4m3_ocp_points.txt")
    codes, vals = [], []
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        c, v = line.split()
        codes.append(int(c, 16))
        vals.append(float(v))
    got = oracle.e4m3_to_f64(np.array(codes, dtype=np.uint8))
    for c, want, g in zip(codes, vals, got):
        if math.isnan(want):
            assert math.isnan(g), hex(c)
        else:
            assert g == want and math.copysign(1, g) == math.copysign(1, want), hex(c)


def test_e4m3_decoder_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])


def test_bf16_decoder_matches_torch():
    rng = np.random.default_rng(24)
    x = torch.from_numpy(rng.standard_normal(5000).astype(np.float32) * 100).to(torch.bfloat16)
    got = oracle.bf16_bits_to_f64(_bits(x))
    np.testing.assert_array_equal(got, x.double().numpy())


def test_block_dequant_uses_each_tokens_block_scale():
    # 2 heads, 130 tokens: tokens 0..127 use block 0's scale, 128..129 block 1's
    x8 = np.full((2, 130, 3), 0x38, dtype=np.uint8)       # every code decodes to 1.0
    scales = np.array([[2.0, 3.0], [5.0, 7.0]], dtype=np.float32)
    out = oracle.dequant_e4m3(x8, scales, block=128)
    np.testing.assert_array_equal(out[0, :128], 2.0)
    np.testing.assert_array_equal(out[0, 128:], 3.0)
    np.testing.assert_array_equal(out[1, :128], 5.0)
    np.testing.assert_array_equal(out[1, 128:], 7.0)

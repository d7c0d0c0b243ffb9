"""The largest sizes the C ABI accepts, against the fp64 oracle: B*H*N*d <=
2^31 - 1 elements per tensor through fa_fwd, fa_fwd_fp8, fa_fwd_block_sparse
and fa_bwd (sampled rows, and for the backward sampled keys), 65535 sequences
through fa_paged_decode and 65535 sequence-heads through fa_paged_prefill.

Two shapes push the addressing to its limits: 8192 heads of 2047 tokens (the
last head starts 4.29e9 bytes into each bf16 tensor; ragged last row block),
and a single causal head of 8,388,808 tokens (2.15e9 bytes, past 2^31, with
the last K/V tiles beyond byte offset 2^31 of the head and a ragged tail).
Tolerances as for the other tests of each path: bf16 O max-abs 2e-2, FP8
8e-2 + half a bf16 ulp, L 1e-3; backward as in test_gpu_bwd."""
import sys

import numpy as np
import pytest
import torch

import oracle
import exact_attention_106_amd as fa
from exact_attention_106_amd import inputs

pytestmark = pytest.mark.gpu

MAX_ELEMS = (1 << 31) - 1


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def f64(t):
    return oracle.bf16_bits_to_f64(t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))


def check(name, o, l, ro, rl):
    got_o, got_l = f64(o), l.cpu().double().numpy()
    assert np.all(np.isfinite(got_o)), name + ": non-finite O"
    eo = float(np.max(np.abs(got_o - ro)))
    el = float(np.max(np.abs(got_l - rl)))
    log("%s: max|dO|=%.3e max|dL|=%.3e" % (name, eo, el))
    assert eo <= 2e-2 and el <= 1e-3, name


def test_fwd_most_heads(gpu):
    B, H, N, d = 2, 4096, 2047, 128
    assert B * H * N * d <= MAX_ELEMS < B * H * (N + 1) * d
    log("fa_fwd bf16 B%d H%d N%d d%d non-causal (ABI maximum elements)" % (B, H, N, d))
    x = inputs.dense_on_device(B, H, N, d, seed=4242, device=gpu)
    o, l = fa.fa_fwd(x.q, x.k, x.v, scale=x.scale, causal=False)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 1791, 1792, 2046])
    for b, h in ((0, 0), (0, 4095), (1, 1234), (1, 4095)):
        ro, rl = oracle.attention_rows(f64(x.q[b, h, rows]), rows, f64(x.k[b, h]), f64(x.v[b, h]), x.scale, False)
        check("b%d h%d" % (b, h), o[b, h, rows], l[b, h, rows], ro, rl)


def test_fwd_longest_head(gpu):
    N, d = 8_388_808, 128
    assert N * d <= MAX_ELEMS and N * d * 2 > 1 << 31 and N % 256 == 200
    log("fa_fwd bf16 B1 H1 N%d d%d causal (one head past 2^31 bytes)" % (N, d))
    x = inputs.dense_on_device(1, 1, N, d, seed=4243, device=gpu, causal=True)
    o, l = fa.fa_fwd(x.q, x.k, x.v, scale=x.scale, causal=True)
    torch.cuda.synchronize()
    log("  kernel done; oracle on sampled rows")
    rows = np.array([0, 1, 1 << 22, (1 << 23) - 1, 1 << 23, N - 100, N - 1])
    ro, rl = oracle.attention_rows(f64(x.q[0, 0, rows]), rows, f64(x.k[0, 0]), f64(x.v[0, 0]), x.scale, True)
    check("N%d causal" % N, o[0, 0, rows], l[0, 0, rows], ro, rl)
    # A row that sees millions of keys averages them down to |O| ~ 1e-3, where
    # the absolute bound says nothing (O = 0 would meet it); such rows are held
    # to the same 2e-2 relative to the row's largest |O|.
    got = f64(o[0, 0, rows])
    for r, i in enumerate(rows):
        if i >= 1 << 22:
            peak = float(np.abs(ro[r]).max())
            rel = float(np.abs(got[r] - ro[r]).max()) / peak
            log("  row %d: max|O_ref| %.3e, max|dO| / max|O_ref| = %.3e" % (i, peak, rel))
            assert rel <= 2e-2, i


def test_fp8_most_heads(gpu):
    B, H, N, d = 2, 4096, 2047, 128
    log("fa_fwd_fp8 B%d H%d N%d d%d causal (ABI maximum elements)" % (B, H, N, d))
    x = inputs.fp8_on_device(B, H, N, d, seed=4244, device=gpu, causal=True)
    o, l = fa.fa_fwd_fp8(x.q8, x.k8, x.v8, x.q_scale, x.k_scale, x.v_scale, scale=x.scale, causal=True)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 1791, 1792, 2046])
    for b, h in ((0, 0), (1, 4095)):
        q, k, v = (oracle.dequant_e4m3(c[b, h].cpu().numpy(), s[b, h].cpu().numpy())
                   for c, s in ((x.q8, x.q_scale), (x.k8, x.k_scale), (x.v8, x.v_scale)))
        ro, rl = oracle.attention_rows(q[rows], rows, k, v, x.scale, True)
        got_o, got_l = f64(o[b, h, rows]), l[b, h, rows].cpu().double().numpy()
        e = np.abs(got_o - ro)
        tol = 8e-2 + 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ro), 2.0 ** -126))) - 8)
        log("fp8 b%d h%d: max|dO|=%.3e max|dL|=%.3e" % (b, h, float(e.max()), float(np.abs(got_l - rl).max())))
        assert np.all(np.isfinite(got_o)) and np.all(e <= tol)
        assert float(np.abs(got_l - rl).max()) <= 1e-3


def test_bwd_most_heads(gpu):
    """fa_bwd with 8192 heads of 2047 tokens: dq on sampled rows, dk and dv on
    sampled keys of the first and last heads, against the oracle's chain rule
    (tolerance per tensor as in the other backward tests: 1e-2 * max|ref| +
    half a bf16 ulp + 1e-5, with max|ref| taken over the sampled entries)."""
    B, H, N, d = 2, 4096, 2047, 128
    log("fa_bwd bf16 B%d H%d N%d d%d causal (ABI maximum elements)" % (B, H, N, d))
    x = inputs.dense_on_device(B, H, N, d, seed=4245, device=gpu, causal=True)
    do = inputs.dense_on_device(B, H, N, d, seed=4246, device=gpu).q
    o, lse = fa.fa_fwd(x.q, x.k, x.v, scale=x.scale, causal=True)
    dq, dk, dv = fa.fa_bwd(x.q, x.k, x.v, o, lse, do, scale=x.scale, causal=True)
    torch.cuda.synchronize()
    idx = np.array([0, 1, 127, 128, 1000, 1920, 2046])
    for b, h in ((0, 0), (1, 4095)):
        q, k, v, g = (f64(t[b, h]) for t in (x.q, x.k, x.v, do))
        rq = oracle.attention_bwd_rows(q, k, v, g, idx, x.scale, True)
        rk, rv = oracle.attention_bwd_cols(q, k, v, g, idx, x.scale, True)
        for nm, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            got = f64(got[b, h, idx])
            err = np.abs(got - ref)
            tol = 1e-2 * float(np.abs(ref).max()) + 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 8) + 1e-5
            log("bwd b%d h%d %s: max err %.3e (max|ref| %.3e)" % (b, h, nm, float(err.max()), float(np.abs(ref).max())))
            assert np.all(np.isfinite(got)) and np.all(err <= tol), nm


def bits16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def test_decode_most_sequences(gpu):
    """fa_paged_decode with 65535 sequences (the most it accepts) of 1..100
    tokens, pairs sharing prompt pages, NaN page tails: every sequence against
    the oracle; the table also passes fa_check_paged_tables."""
    p = inputs.paged_pool(num_seqs=65535, H=2, d=128, ctx_lo=1, ctx_hi=100, seed=4247, share=0.5, device=gpu)
    log("fa_paged_decode S65535 H2 d128 ctx 1..100 (most sequences), %d pages" % p.n_unique_pages)
    chk = fa.fa_check_paged_tables(p.block_table, p.ctx_lens, 16, p.kcache.shape[0])
    o, l = fa.fa_paged_decode(p.q, p.kcache, p.vcache, p.block_table, p.ctx_lens, scale=p.scale)
    torch.cuda.synchronize()
    assert chk.cpu().tolist() == [0, -1]
    ro, rl = oracle.paged_decode(f64(p.q), bits16(p.kcache), bits16(p.vcache), p.block_table.cpu().numpy(),
                                 p.ctx_lens.cpu().numpy(), p.scale)
    check("decode S65535", o, l, ro, rl)


def test_paged_prefill_most_sequence_heads(gpu):
    """fa_paged_prefill with num_seqs * H = 65535 (the most it accepts): 65535
    sequences of 1..100 tokens, the 3 newest of each as queries (those at
    negative positions see nothing: O = 0, L = -inf); 400 sequences, the last
    ones among them, against the oracle."""
    S, n_new = 65535, 3
    p = inputs.paged_pool(num_seqs=S, H=1, d=128, ctx_lo=1, ctx_hi=100, seed=4248, share=0.5, device=gpu)
    q = inputs.dense_on_device(S, 1, n_new, 128, seed=4249, device=gpu).q
    log("fa_paged_prefill S65535 H1 n_new3 d128 (most sequence-heads)")
    o, l = fa.fa_paged_prefill(q, p.kcache, p.vcache, p.block_table, p.ctx_lens, scale=p.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    sel = np.unique(np.concatenate([rng.choice(S - 8, 392, replace=False), np.arange(S - 8, S)]))
    ro, rl = oracle.paged_prefill(f64(q[sel]), bits16(p.kcache), bits16(p.vcache),
                                  p.block_table.cpu().numpy()[sel], p.ctx_lens.cpu().numpy()[sel], p.scale)
    got_o, got_l = f64(o[sel]), l[sel].cpu().double().numpy()
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(got_l), fin) and (~fin).any()
    assert np.all(got_o[~fin] == 0)
    eo = float(np.max(np.abs(got_o - ro)))
    el = float(np.max(np.abs(got_l[fin] - rl[fin])))
    log("paged prefill S65535: max|dO|=%.3e max|dL|=%.3e" % (eo, el))
    assert eo <= 2e-2 and el <= 1e-3


def test_block_sparse_most_heads(gpu):
    """fa_fwd_block_sparse with 8192 heads of 2047 tokens, half the causal
    blocks kept, dropout 0.1 (the last head's counter carries b*H + h = 8191):
    sampled rows of the first and last heads. O bound 2e-2 / (1 - p)."""
    from oracle import sparse
    B, H, N, d, p_drop, seed = 2, 4096, 2047, 128, 0.1, 0x0123_4567_89AB_CDEF
    log("fa_fwd_block_sparse B%d H%d N%d d%d causal p=%.1f (ABI maximum elements)" % (B, H, N, d, p_drop))
    x = inputs.dense_on_device(B, H, N, d, seed=4250, device=gpu, causal=True)
    mask = inputs.block_mask(N, density=0.5, seed=4251, causal=True)
    o, l = fa.fa_fwd_block_sparse(x.q, x.k, x.v, mask.to(gpu), scale=x.scale, causal=True, dropout_p=p_drop,
                                  seed=seed)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 1791, 1792, 2046])
    for b, h in ((0, 0), (1, 4095)):
        ro, rl = sparse.block_sparse_attention_rows(f64(x.q[b, h, rows]), rows, f64(x.k[b, h]), f64(x.v[b, h]),
                                                    mask.numpy(), x.scale, True, bh=b * H + h, p_drop=p_drop,
                                                    seed=seed)
        got_o, got_l = f64(o[b, h, rows]), l[b, h, rows].cpu().double().numpy()
        eo, el = float(np.abs(got_o - ro).max()), float(np.abs(got_l - rl).max())
        log("sparse b%d h%d: max|dO|=%.3e max|dL|=%.3e" % (b, h, eo, el))
        assert np.all(np.isfinite(got_o)) and eo <= 2e-2 / (1 - p_drop) and el <= 1e-3

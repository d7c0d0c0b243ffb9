"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Tolerances are max-abs over all compared elements:
  fp32 path  O, L <= 1e-5
  bf16 path  O <= 2e-2, L <= 1e-3
  fp8 path   O <= 8e-2 + half a bf16 ulp of |O_ref| (bf16 output rounding alone
             exceeds 8e-2 once |O| >= 32, which V outliers x20 can reach), L <= 1e-3
Full-size workloads are compared on sampled rows the oracle computes one by
one; small shapes (several tiles plus ragged tails) are compared in full.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_attention_106_amd import inputs

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def fa(gpu):
    import exact_attention_106_amd as fa_mod
    fa_mod.fa_version()   # loads libfa.so; raises if it is not built
    return fa_mod


def bits16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f64_bf16(t):
    return oracle.bf16_bits_to_f64(bits16(t))


def half_ulp_bf16(x):
    x = np.abs(x)
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 8)


def assert_close(name, got_o, got_l, ref_o, ref_l, tol_o, tol_l):
    got_o = np.asarray(got_o, dtype=np.float64)
    got_l = np.asarray(got_l, dtype=np.float64)
    assert np.all(np.isfinite(got_o)), name + ": non-finite O"
    assert np.all(np.isfinite(got_l)), name + ": non-finite L"
    err_o = np.abs(got_o - ref_o)
    tol = tol_o if np.isscalar(tol_o) else tol_o
    worst = float(np.max(err_o - tol)) if err_o.size else -1.0
    err_l = float(np.max(np.abs(got_l - ref_l))) if got_l.size else 0.0
    log("%s: max|dO|=%.3e max|dL|=%.3e" % (name, float(err_o.max()) if err_o.size else 0.0, err_l))
    assert worst <= 0, "%s: O error exceeds tolerance by %.3e" % (name, worst)
    assert err_l <= tol_l, "%s: L error %.3e" % (name, err_l)


# ---------------------------------------------------------------------------------- fp32

def test_f32_worked_example(fa, gpu):
    c = inputs.config1()
    log("fa_fwd_f32 worked example 16x8")
    o, l = fa.fa_fwd_f32(c.q.to(gpu), c.k.to(gpu), c.v.to(gpu), scale=1.0, causal=False)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(c.q.double().numpy(), c.k.double().numpy(), c.v.double().numpy(), 1.0, False)
    assert_close("f32 16x8", o.cpu().double().numpy(), l.cpu().double().numpy(), ro, rl, 1e-5, 1e-5)


@pytest.mark.parametrize("B,H,N,d,causal", [
    (1, 1, 1, 1, False), (2, 3, 100, 40, True), (1, 2, 130, 128, False), (1, 1, 257, 8, True),
    (2, 1, 64, 16, False), (1, 1, 200, 128, True)])
def test_f32_shapes(fa, gpu, B, H, N, d, causal):
    x = inputs.dense(B, H, N, d, seed=100 + N + d, dtype="f32")
    log("fa_fwd_f32 B%d H%d N%d d%d causal=%d" % (B, H, N, d, causal))
    o, l = fa.fa_fwd_f32(x.q.to(gpu), x.k.to(gpu), x.v.to(gpu), scale=x.scale, causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(x.q.double().numpy(), x.k.double().numpy(), x.v.double().numpy(), x.scale, causal)
    assert_close("f32", o.cpu().double().numpy(), l.cpu().double().numpy(), ro, rl, 1e-5, 1e-5)


# ---------------------------------------------------------------------------------- bf16

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 128, 200, 333])
def test_bf16_shapes(fa, gpu, N, d, causal):
    x = inputs.dense(2, 2, N, d, seed=1000 + N + d, dtype="bf16")
    log("fa_fwd bf16 B2 H2 N%d d%d causal=%d" % (N, d, causal))
    o, l = fa.fa_fwd(x.q.to(gpu), x.k.to(gpu), x.v.to(gpu), scale=x.scale, causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(f64_bf16(x.q), f64_bf16(x.k), f64_bf16(x.v), x.scale, causal)
    assert_close("bf16", f64_bf16(o), l.cpu().double().numpy(), ro, rl, 2e-2, 1e-3)


def test_bf16_single_head_large_logits(fa, gpu):
    # scale 1 on N(0,1) inputs gives logits of tens: the max subtraction must hold
    x = inputs.dense(1, 1, 300, 128, seed=77, dtype="bf16", scale=1.0)
    for causal in (False, True):
        log("fa_fwd bf16 large logits causal=%d" % causal)
        o, l = fa.fa_fwd(x.q.to(gpu), x.k.to(gpu), x.v.to(gpu), scale=1.0, causal=causal)
        torch.cuda.synchronize()
        ro, rl = oracle.attention(f64_bf16(x.q), f64_bf16(x.k), f64_bf16(x.v), 1.0, causal)
        assert_close("bf16 big logits", f64_bf16(o), l.cpu().double().numpy(), ro, rl, 2e-2, 1e-3)


def _sampled_rows(fa_out, x, rows, causal):
    """Compare (bh, i) rows of a [B, H, N, d] output with the oracle, head by head."""
    o, l = fa_out
    B, H, N, d = x.q.shape
    got_o, got_l, ref_o, ref_l = [], [], [], []
    heads = sorted({bh for bh, _ in rows})
    for bh in heads:
        b, h = divmod(bh, H)
        idx = np.array(sorted(i for hh, i in rows if hh == bh))
        kk = f64_bf16(x.k[b, h])
        vv = f64_bf16(x.v[b, h])
        qq = f64_bf16(x.q[b, h][torch.from_numpy(idx)])
        ro, rl = oracle.attention_rows(qq, idx, kk, vv, x.scale, causal)
        ref_o.append(ro), ref_l.append(rl)
        got_o.append(f64_bf16(o[b, h][torch.from_numpy(idx).to(o.device)]))
        got_l.append(l[b, h][torch.from_numpy(idx).to(l.device)].cpu().double().numpy())
    return np.concatenate(got_o), np.concatenate(got_l), np.concatenate(ref_o), np.concatenate(ref_l)


def _pick_rows(B, H, N, n, seed, br=128):
    rng = np.random.default_rng(seed)
    rows = set()
    for bh in rng.choice(B * H, size=min(B * H, 6), replace=False):
        for i in (0, 1, br - 1, br, N // 2, N - 2, N - 1):
            if 0 <= i < N:
                rows.add((int(bh), int(i)))
    while len(rows) < n:
        rows.add((int(rng.integers(B * H)), int(rng.integers(N))))
    return sorted(rows)


def test_bf16_mha_B4H16N2048d64_sampled(fa, gpu):
    x = inputs.config2()
    log("fa_fwd bf16 B4 H16 N2048 d64 (full size, sampled rows)")
    qd, kd, vd = x.q.to(gpu), x.k.to(gpu), x.v.to(gpu)
    out = fa.fa_fwd(qd, kd, vd, scale=x.scale, causal=False)
    o2, l2 = fa.fa_fwd(qd, kd, vd, scale=x.scale, causal=False)
    torch.cuda.synchronize()
    assert torch.equal(out[0], o2) and torch.equal(out[1], l2), "not bitwise deterministic"
    rows = _pick_rows(4, 16, 2048, 300, seed=2)
    g_o, g_l, r_o, r_l = _sampled_rows(out, x, rows, False)
    assert_close("bf16 B4H16N2048d64", g_o, g_l, r_o, r_l, 2e-2, 1e-3)


def test_bf16_causal_B1H32N16384d128_sampled(fa, gpu):
    x = inputs.config3()
    log("fa_fwd bf16 causal B1 H32 N16384 d128 (full size, sampled rows)")
    out = fa.fa_fwd(x.q.to(gpu), x.k.to(gpu), x.v.to(gpu), scale=x.scale, causal=True)
    torch.cuda.synchronize()
    rows = _pick_rows(1, 32, 16384, 120, seed=3)
    g_o, g_l, r_o, r_l = _sampled_rows(out, x, rows, True)
    assert_close("bf16 causal B1H32N16384d128", g_o, g_l, r_o, r_l, 2e-2, 1e-3)


def test_bf16_causal_future_keys_do_not_matter(fa, gpu):
    x = inputs.dense(1, 2, 300, 128, seed=55, dtype="bf16")
    log("fa_fwd bf16 causal future-perturbation")
    o1, l1 = fa.fa_fwd(x.q.to(gpu), x.k.to(gpu), x.v.to(gpu), causal=True)
    k2, v2 = x.k.clone(), x.v.clone()
    k2[:, :, 150:] = 30.0
    v2[:, :, 150:] = -7.0
    o2, l2 = fa.fa_fwd(x.q.to(gpu), k2.to(gpu), v2.to(gpu), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :, :150], o2[:, :, :150])
    assert torch.equal(l1[:, :, :150], l2[:, :, :150])


# ---------------------------------------------------------------------------------- fp8

def _fp8_ref(x, rows=None):
    q = oracle.dequant_e4m3(x.q8.cpu().numpy(), x.q_scale.cpu().numpy())
    k = oracle.dequant_e4m3(x.k8.cpu().numpy(), x.k_scale.cpu().numpy())
    v = oracle.dequant_e4m3(x.v8.cpu().numpy(), x.v_scale.cpu().numpy())
    return q, k, v


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 100, 300])
def test_fp8_shapes(fa, gpu, N, causal):
    x = inputs.fp8_inputs(1, 2, N, 128, seed=300 + N, causal=causal)
    log("fa_fwd_fp8 B1 H2 N%d causal=%d" % (N, causal))
    o, l = fa.fa_fwd_fp8(x.q8.to(gpu), x.k8.to(gpu), x.v8.to(gpu), x.q_scale.to(gpu),
                         x.k_scale.to(gpu), x.v_scale.to(gpu), scale=x.scale, causal=causal)
    torch.cuda.synchronize()
    q, k, v = _fp8_ref(x)
    ro, rl = oracle.attention(q, k, v, x.scale, causal)
    assert_close("fp8", f64_bf16(o), l.cpu().double().numpy(), ro, rl, 8e-2 + half_ulp_bf16(ro), 1e-3)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 100, 300, 1000])
def test_fp8_d64_shapes(fa, gpu, N, causal):
    # d = 64: one 64-channel QK MFMA per key tile, 64-byte E4M3 K rows in LDS
    # (their own swizzle) and one V register load per lane per tile
    x = inputs.fp8_inputs(2, 2, N, 64, seed=700 + N, causal=causal)
    log("fa_fwd_fp8 B2 H2 N%d d64 causal=%d" % (N, causal))
    o, l = fa.fa_fwd_fp8(x.q8.to(gpu), x.k8.to(gpu), x.v8.to(gpu), x.q_scale.to(gpu),
                         x.k_scale.to(gpu), x.v_scale.to(gpu), scale=x.scale, causal=causal)
    torch.cuda.synchronize()
    q, k, v = _fp8_ref(x)
    ro, rl = oracle.attention(q, k, v, x.scale, causal)
    assert_close("fp8 d64", f64_bf16(o), l.cpu().double().numpy(), ro, rl, 8e-2 + half_ulp_bf16(ro), 1e-3)


def test_fp8_causal_B2H16N8192d128_sampled(fa, gpu):
    x = inputs.config4()
    log("fa_fwd_fp8 causal B2 H16 N8192 d128 (full size, sampled rows)")
    o, l = fa.fa_fwd_fp8(x.q8.to(gpu), x.k8.to(gpu), x.v8.to(gpu), x.q_scale.to(gpu),
                         x.k_scale.to(gpu), x.v_scale.to(gpu), scale=x.scale, causal=True)
    torch.cuda.synchronize()
    rows = _pick_rows(2, 16, 8192, 100, seed=4)
    q, k, v = _fp8_ref(x)
    got_o, got_l, ref_o, ref_l = [], [], [], []
    for bh in sorted({bh for bh, _ in rows}):
        b, h = divmod(bh, 16)
        idx = np.array(sorted(i for hh, i in rows if hh == bh))
        ro, rl = oracle.attention_rows(q[b, h][idx], idx, k[b, h], v[b, h], x.scale, True)
        ref_o.append(ro), ref_l.append(rl)
        sel = torch.from_numpy(idx).to(o.device)
        got_o.append(f64_bf16(o[b, h][sel]))
        got_l.append(l[b, h][sel].cpu().double().numpy())
    ref_o = np.concatenate(ref_o)
    assert_close("fp8 causal B2H16N8192d128", np.concatenate(got_o), np.concatenate(got_l), ref_o,
                 np.concatenate(ref_l), 8e-2 + half_ulp_bf16(ref_o), 1e-3)


# ---------------------------------------------------------------------------------- decode

def _decode(fa, p, gpu, kc=None, vc=None, bt=None):
    kc = p.kcache if kc is None else kc
    vc = p.vcache if vc is None else vc
    bt = p.block_table if bt is None else bt
    return fa.fa_paged_decode(p.q.to(gpu), kc.to(gpu), vc.to(gpu), bt.to(gpu), p.ctx_lens.to(gpu),
                              scale=p.scale)


def test_decode_small_pools(fa, gpu):
    for seed, (lo, hi) in ((31, (1, 700)), (32, (1, 40)), (33, (500, 1100))):
        p = inputs.paged_pool(num_seqs=7, H=4, d=128, ctx_lo=lo, ctx_hi=hi, seed=seed, share=0.3)
        log("fa_paged_decode S7 H4 ctx %d..%d" % (lo, hi))
        o, l = _decode(fa, p, gpu)
        torch.cuda.synchronize()
        ro, rl = oracle.paged_decode(f64_bf16(p.q), bits16(p.kcache), bits16(p.vcache),
                                     p.block_table.numpy(), p.ctx_lens.numpy(), p.scale)
        assert_close("decode small", f64_bf16(o), l.cpu().double().numpy(), ro, rl, 2e-2, 1e-3)


def test_decode_edge_contexts(fa, gpu):
    # ctx of exactly 1, 16, 17, 512, 513 tokens (page and chunk boundaries)
    p = inputs.paged_pool(num_seqs=5, H=2, d=128, ctx_lo=400, ctx_hi=600, seed=41, share=0.0,
                          nan_tails=False)
    ctx = torch.tensor([1, 16, 17, 512, 513], dtype=torch.int32)
    p.ctx_lens = ctx
    nb = (ctx + 15) // 16
    bt = torch.full_like(p.block_table, -1)
    nxt = 0
    for s in range(5):
        bt[s, :nb[s]] = torch.arange(nxt, nxt + int(nb[s]), dtype=torch.int32)
        nxt += int(nb[s])
        rem = int(ctx[s]) % 16
        if rem:   # slots past the context must never be read
            p.kcache[nxt - 1, :, rem:] = float("nan")
            p.vcache[nxt - 1, :, rem:] = float("nan")
    assert nxt <= p.kcache.shape[0]
    p.block_table = bt
    log("fa_paged_decode edge contexts")
    o, l = _decode(fa, p, gpu)
    torch.cuda.synchronize()
    ro, rl = oracle.paged_decode(f64_bf16(p.q), bits16(p.kcache), bits16(p.vcache), bt.numpy(),
                                 ctx.numpy(), p.scale)
    assert np.isfinite(ro).all()
    assert_close("decode edges", f64_bf16(o), l.cpu().double().numpy(), ro, rl, 2e-2, 1e-3)


def test_decode_shared_prefix_classes(fa, gpu):
    # Sequences 0..5 name the same first 80 pages (two full 32-page chunks and
    # part of a third), sequence 6 shares 40 pages with 0 and the rest have
    # their own: a class of six chunk-sharers, read in pairs, plus chunks that
    # are shared only partly. Contexts differ inside the shared pages' range.
    p = inputs.paged_pool(num_seqs=9, H=2, d=128, ctx_lo=1300, ctx_hi=2600, seed=61, share=0.0,
                          nan_tails=False)
    ctx = torch.tensor([2600, 1300, 1350, 2100, 1290, 2048, 1700, 900, 1024], dtype=torch.int32)
    p.ctx_lens = ctx
    nb = (ctx + 15) // 16
    P = p.kcache.shape[0]
    bt = torch.full_like(p.block_table, -1)
    g = torch.Generator().manual_seed(7)
    own = torch.randperm(P, generator=g).int()
    nxt = 0
    def fresh(n):
        nonlocal nxt
        r = own[nxt:nxt + n]
        nxt += n
        return r
    bt[0, :nb[0]] = fresh(int(nb[0]))
    for s in range(1, 9):
        k = 80 if s < 6 else (40 if s == 6 else 0)
        k = min(k, int(nb[s]))
        bt[s, :k] = bt[0, :k]
        bt[s, k:nb[s]] = fresh(int(nb[s]) - k)
    assert nxt <= P
    p.block_table = bt
    log("fa_paged_decode shared-prefix classes S9 H2")
    o, l = _decode(fa, p, gpu)
    torch.cuda.synchronize()
    ro, rl = oracle.paged_decode(f64_bf16(p.q), bits16(p.kcache), bits16(p.vcache), bt.numpy(),
                                 ctx.numpy(), p.scale)
    assert_close("decode shared", f64_bf16(o), l.cpu().double().numpy(), ro, rl, 2e-2, 1e-3)


def test_decode_placement_invariance(fa, gpu):
    p = inputs.paged_pool(num_seqs=6, H=4, d=128, ctx_lo=100, ctx_hi=900, seed=51, share=0.5)
    log("fa_paged_decode placement invariance")
    o1, l1 = _decode(fa, p, gpu)
    P = p.kcache.shape[0]
    g = torch.Generator().manual_seed(5)
    new_pos = torch.randperm(2 * P, generator=g)[:P]
    kc = torch.zeros((2 * P,) + tuple(p.kcache.shape[1:]), dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    kc[new_pos], vc[new_pos] = p.kcache, p.vcache
    bt = torch.where(p.block_table >= 0, new_pos[p.block_table.clamp(min=0).long()].int(), p.block_table)
    o2, l2 = _decode(fa, p, gpu, kc=kc, vc=vc, bt=bt)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_S64H32d128_full_size_sampled(fa, gpu):
    log("fa_paged_decode S64 H32 d128 ctx 512..32768 (full size, sampled sequences)")
    p = inputs.config5(device=gpu)
    o, l = fa.fa_paged_decode(p.q, p.kcache, p.vcache, p.block_table, p.ctx_lens, scale=p.scale)
    torch.cuda.synchronize()
    ctx = p.ctx_lens.cpu().numpy()
    bt = p.block_table.cpu().numpy()
    seqs = [int(np.argmax(ctx)), int(np.argmin(ctx)), 0, 1]   # 0 and 1 share a prefix
    for s in seqs:
        nb = (int(ctx[s]) + 15) // 16
        pages = torch.from_numpy(bt[s, :nb].astype(np.int64)).to(gpu)
        kc = bits16(p.kcache.index_select(0, pages))
        vc = bits16(p.vcache.index_select(0, pages))
        table = np.arange(nb, dtype=np.int32)[None, :]
        ro, rl = oracle.paged_decode(f64_bf16(p.q[s:s + 1]), kc, vc, table, ctx[s:s + 1], p.scale)
        assert_close("decode seq %d ctx %d" % (s, ctx[s]), f64_bf16(o[s:s + 1]),
                     l[s:s + 1].cpu().double().numpy(), ro, rl, 2e-2, 1e-3)



def test_decode_S4096_many_sharing_classes(fa, gpu):
    # 4096 sequences whose first two 32-page chunks come from small sets of page
    # lists (150 for chunk 0: classes of about 27 members, odd sizes included;
    # 3000 for chunk 1: mostly single members and pairs), then 1..5 pages of
    # their own. Grouping the chunk classes at this size must stay cheap and
    # every query must still see exactly its own pages.
    S, H, d = 4096, 1, 128
    rng = np.random.Generator(np.random.PCG64(71))
    ctx = rng.integers(1025, 1100, size=S, endpoint=True).astype(np.int64)
    nb = (ctx + 15) // 16
    n0, n1 = 150, 3000
    pick0 = rng.integers(0, n0, size=S)
    pick1 = rng.integers(0, n1, size=S)
    tails = nb - 64
    P = 32 * (n0 + n1) + int(tails.sum())
    perm = rng.permutation(P).astype(np.int32)
    table = np.full((S, int(nb.max())), -1, dtype=np.int32)
    nxt = 32 * (n0 + n1)
    for s in range(S):
        table[s, :32] = perm[32 * pick0[s]:32 * pick0[s] + 32]
        table[s, 32:64] = perm[32 * (n0 + pick1[s]):32 * (n0 + pick1[s]) + 32]
        table[s, 64:nb[s]] = perm[nxt:nxt + tails[s]]
        nxt += int(tails[s])
    assert nxt == P
    g = torch.Generator(device=gpu)
    g.manual_seed(71)
    kc = torch.randn((P, H, 16, d), generator=g, device=gpu).to(torch.bfloat16)
    vc = torch.randn((P, H, 16, d), generator=g, device=gpu).to(torch.bfloat16)
    q = torch.from_numpy(rng.standard_normal((S, H, d), dtype=np.float32)).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(d)
    log("fa_paged_decode S4096 H1 d128, shared chunk classes")
    o, l = fa.fa_paged_decode(q.to(gpu), kc, vc, torch.from_numpy(table).to(gpu),
                              torch.from_numpy(ctx.astype(np.int32)).to(gpu), scale=scale)
    torch.cuda.synchronize()
    big = np.flatnonzero(pick0 == np.bincount(pick0).argmax())[:9]   # members of one large class
    seqs = sorted(set(big.tolist()) | set(rng.choice(S, 40, replace=False).tolist()))
    for s in seqs:
        pages = torch.from_numpy(table[s, :nb[s]].astype(np.int64)).to(gpu)
        ro, rl = oracle.paged_decode(f64_bf16(q[s:s + 1]), bits16(kc.index_select(0, pages)),
                                     bits16(vc.index_select(0, pages)),
                                     np.arange(nb[s], dtype=np.int32)[None, :], ctx[s:s + 1], scale)
        assert_close("decode S4096 seq %d" % s, f64_bf16(o[s:s + 1]), l[s:s + 1].cpu().double().numpy(),
                     ro, rl, 2e-2, 1e-3)

# ---------------------------------------------------------------------------------- reference jumps

@pytest.mark.parametrize("d,causal", [(128, True), (128, False), (64, True), (64, False)])
def test_bf16_score_jumps_redo_the_tile_exactly(fa, gpu, d, causal):
    # After the first tile the kernel forms 2^(t - m) against the running
    # reference and redoes a tile exactly when a lane's weights pass 2^20.
    # Key 700 aligned with query 800 (x10) gives a score far past the first
    # tiles' (2^(t - m) overflows to inf on the fast path), and keys 300..363
    # scaled x8 raise many rows' maxima by more than 2^20.
    x = inputs.dense(1, 2, 1000, d, seed=4000 + d + causal, dtype="bf16")
    k = x.k.clone()
    k[:, :, 700] = (x.q[:, :, 800].float() * 10).to(torch.bfloat16)
    k[:, :, 300:364] = (k[:, :, 300:364].float() * 8).to(torch.bfloat16)
    log("fa_fwd bf16 score jumps d%d causal=%d" % (d, causal))
    o, l = fa.fa_fwd(x.q.to(gpu), k.to(gpu), x.v.to(gpu), scale=x.scale, causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(f64_bf16(x.q), f64_bf16(k), f64_bf16(x.v), x.scale, causal)
    assert_close("bf16 score jumps", f64_bf16(o), l.cpu().double().numpy(), ro, rl, 2e-2, 1e-3)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_score_jumps(fa, gpu, causal):
    # a K scale block x64 (keys 256..383): scores of those keys jump far past
    # the first tiles' for every query that sees them (the reference moves by
    # more than 2^20 within a row). The FP8 Q.K^T products carry a relative
    # error of a few 1e-4 (the E4M3 dot products of the MFMA; the same inputs
    # at x1 already give an L error of 1.6e-3 on one row of 2000), which grows
    # with the scores: L is held to 1e-3 relative to |L| here, O to the FP8 bound.
    x = inputs.fp8_inputs(1, 2, 1000, 128, seed=4100 + causal, causal=causal)
    ks = x.k_scale.clone()
    ks[:, :, 2] *= 64.0
    log("fa_fwd_fp8 score jumps causal=%d" % causal)
    o, l = fa.fa_fwd_fp8(x.q8.to(gpu), x.k8.to(gpu), x.v8.to(gpu), x.q_scale.to(gpu), ks.to(gpu),
                         x.v_scale.to(gpu), scale=x.scale, causal=causal)
    torch.cuda.synchronize()
    q = oracle.dequant_e4m3(x.q8.numpy(), x.q_scale.numpy())
    k = oracle.dequant_e4m3(x.k8.numpy(), ks.numpy())
    v = oracle.dequant_e4m3(x.v8.numpy(), x.v_scale.numpy())
    ro, rl = oracle.attention(q, k, v, x.scale, causal)
    got_l = l.cpu().double().numpy()
    assert_close("fp8 score jumps", f64_bf16(o), got_l, ro, rl, 8e-2 + half_ulp_bf16(ro), float("inf"))
    rel = float(np.max(np.abs(got_l - rl) / np.maximum(1.0, np.abs(rl))))
    log("fp8 score jumps: max |dL| / max(1, |L|) = %.3e" % rel)
    assert rel <= 1e-3

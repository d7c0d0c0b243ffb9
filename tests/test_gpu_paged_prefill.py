"""GPU parity of the paged (chunked) prefill and of the block manager's
copy-on-write path, through the C ABI, against the fp64 oracle.

Tolerances as for the bf16 forward: O max-abs 2e-2, L 1e-3. Page tails past
each context are NaN-filled and must not leak."""
import sys

import numpy as np
import pytest
import torch

import oracle
import exact_attention_106_amd as fa
from exact_attention_106_amd import inputs

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f64(t):
    return oracle.bf16_bits_to_f64(bits(t))


def check(name, o, l, ro, rl):
    got_o, got_l = f64(o), l.cpu().double().numpy()
    assert np.all(np.isfinite(got_o)), name + ": non-finite O"
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(got_l), fin), name + ": L finiteness"
    eo = float(np.max(np.abs(got_o - ro)))
    el = float(np.max(np.abs(got_l[fin] - rl[fin]))) if fin.any() else 0.0
    log("%s: max|dO|=%.3e max|dL|=%.3e" % (name, eo, el))
    assert eo <= 2e-2 and el <= 1e-3


@pytest.mark.parametrize("n_new,ctx_lo,ctx_hi", [(1, 130, 700), (17, 130, 700), (128, 130, 700),
                                                (130, 130, 700), (200, 300, 1100), (64, 10, 90)])
def test_paged_prefill_pools(gpu, n_new, ctx_lo, ctx_hi):
    p = inputs.paged_pool(num_seqs=4, H=2, d=128, ctx_lo=ctx_lo, ctx_hi=ctx_hi, seed=40 + n_new)
    q = inputs.dense(4, 2, n_new, 128, seed=41 + n_new).q
    log("fa_paged_prefill S4 H2 n_new=%d ctx=%s" % (n_new, p.ctx_lens.tolist()))
    o, l = fa.fa_paged_prefill(q.to(gpu), p.kcache.to(gpu), p.vcache.to(gpu), p.block_table.to(gpu),
                               p.ctx_lens.to(gpu), scale=p.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.paged_prefill(f64(q), bits(p.kcache), bits(p.vcache), p.block_table.numpy(),
                                  p.ctx_lens.numpy(), p.scale)
    check("paged prefill n_new=%d" % n_new, o, l, ro, rl)


@pytest.mark.parametrize("S,H,n_new,ctx_lo,ctx_hi", [
    (3, 3, 300, 100, 900),    # S*H not a multiple of 8 (plain workgroup order), ragged row block
    (5, 1, 600, 500, 1300),   # three row blocks, contexts not multiples of 64
    (2, 4, 520, 512, 1024),   # XCD-grouped order, a row block of 8 queries
    (2, 2, 700, 100, 400)])   # row blocks entirely before the context (O = 0, L = -inf)
def test_paged_prefill_grids(gpu, S, H, n_new, ctx_lo, ctx_hi):
    p = inputs.paged_pool(num_seqs=S, H=H, d=128, ctx_lo=ctx_lo, ctx_hi=ctx_hi, seed=60 + n_new)
    q = inputs.dense(S, H, n_new, 128, seed=61 + n_new).q
    log("fa_paged_prefill S%d H%d n_new=%d ctx=%s" % (S, H, n_new, p.ctx_lens.tolist()))
    o, l = fa.fa_paged_prefill(q.to(gpu), p.kcache.to(gpu), p.vcache.to(gpu), p.block_table.to(gpu),
                               p.ctx_lens.to(gpu), scale=p.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.paged_prefill(f64(q), bits(p.kcache), bits(p.vcache), p.block_table.numpy(),
                                  p.ctx_lens.numpy(), p.scale)
    check("paged prefill S%d H%d n_new=%d" % (S, H, n_new), o, l, ro, rl)
    assert np.array_equal(np.isneginf(l.cpu().numpy()), np.isneginf(rl)), "queries that see no key"


def test_paged_prefill_long_contexts(gpu):
    """Contexts of 33000-41000 tokens (up to ~640 key tiles): the kernel holds
    the page ids in LDS windows of 128 tiles, refilled as it goes, so every
    wave here reads windows 0-5, most of them refilled ones."""
    p = inputs.paged_pool(num_seqs=2, H=1, d=128, ctx_lo=33000, ctx_hi=41000, seed=90)
    q = inputs.dense(2, 1, 300, 128, seed=91).q
    log("fa_paged_prefill S2 H1 n_new=300 ctx=%s" % p.ctx_lens.tolist())
    assert int(p.ctx_lens.min()) > 5 * 128 * 64 // 2
    o, l = fa.fa_paged_prefill(q.to(gpu), p.kcache.to(gpu), p.vcache.to(gpu), p.block_table.to(gpu),
                               p.ctx_lens.to(gpu), scale=p.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.paged_prefill(f64(q), bits(p.kcache), bits(p.vcache), p.block_table.numpy(),
                                  p.ctx_lens.numpy(), p.scale)
    check("paged prefill long contexts", o, l, ro, rl)


def test_block_manager_fork_cow_prefill(gpu):
    """Prompt of 100 tokens, forked into three samples that each add 20 tokens:
    shared prompt pages, one copy-on-write per sample on the half-full last
    prompt page, K/V of the new tokens written into the pages the manager
    returns, then paged prefill of the 20 new tokens of every sample."""
    H, d, ps, P, MB = 2, 128, 16, 64, 16
    bm = fa.BlockManager(P, 4, MB, ps)
    g = torch.Generator().manual_seed(77)
    kc = torch.zeros((P, H, ps, d), dtype=torch.bfloat16)
    vc = torch.zeros((P, H, ps, d), dtype=torch.bfloat16)
    prompt_k = torch.randn((100, H, d), generator=g).to(torch.bfloat16)
    prompt_v = torch.randn((100, H, d), generator=g).to(torch.bfloat16)
    bm.add_seq(0, 100)
    table, _ = bm.block_table()
    for t in range(100):
        kc[table[0, t // ps], :, t % ps] = prompt_k[t]
        vc[table[0, t // ps], :, t % ps] = prompt_v[t]
    kc, vc = kc.to(gpu), vc.to(gpu)
    logical_k = {s: [prompt_k[t] for t in range(100)] for s in (0, 1, 2)}
    logical_v = {s: [prompt_v[t] for t in range(100)] for s in (0, 1, 2)}
    bm.fork(0, 1)
    bm.fork(0, 2)
    cows = []
    for step in range(20):
        for s in (0, 1, 2):
            src, dst = bm.append_token(s)
            if src >= 0:
                cows.append((src, dst))
                fa.fa_copy_pages(kc, vc, torch.tensor([src], dtype=torch.int32, device=gpu),
                                 torch.tensor([dst], dtype=torch.int32, device=gpu))
            t = bm.seq_len(s) - 1
            table, _ = bm.block_table()
            nk = torch.randn((H, d), generator=g).to(torch.bfloat16)
            nv = torch.randn((H, d), generator=g).to(torch.bfloat16)
            kc[int(table[s, t // ps]), :, t % ps] = nk.to(gpu)
            vc[int(table[s, t // ps]), :, t % ps] = nv.to(gpu)
            logical_k[s].append(nk)
            logical_v[s].append(nv)
    assert len(cows) == 2          # samples 1 and 2 copy page 6; sample 0 then owns it alone
    table, ctx = bm.block_table()
    q = inputs.dense(3, H, 20, d, seed=78).q
    o, l = fa.fa_paged_prefill(q.to(gpu), kc, vc, table[:3].contiguous().to(gpu), ctx[:3].contiguous().to(gpu))
    torch.cuda.synchronize()
    for s in range(3):
        k = torch.stack(logical_k[s]).permute(1, 0, 2)       # [H, 120, d]
        v = torch.stack(logical_v[s]).permute(1, 0, 2)
        pos = np.arange(100, 120)
        for hh in range(H):
            ro, rl = oracle.attention_rows(f64(q[s, hh]), pos, f64(k[hh]), f64(v[hh]), 1 / np.sqrt(d), True)
            check("fork/cow sample %d head %d" % (s, hh), o[s, hh], l[s, hh], ro, rl)


def test_copy_pages_exact(gpu):
    P, H, ps, d = 12, 3, 16, 128
    kc = torch.randn((P, H, ps, d), device=gpu).to(torch.bfloat16)
    vc = torch.randn((P, H, ps, d), device=gpu).to(torch.bfloat16)
    k0, v0 = kc.clone(), vc.clone()
    src = torch.tensor([3, 7, 0], dtype=torch.int32, device=gpu)
    dst = torch.tensor([9, 1, 11], dtype=torch.int32, device=gpu)
    fa.fa_copy_pages(kc, vc, src, dst)
    torch.cuda.synchronize()
    ek, ev = k0.clone(), v0.clone()
    for a, b in zip(src.tolist(), dst.tolist()):
        ek[b], ev[b] = k0[a], v0[a]
    assert torch.equal(kc, ek) and torch.equal(vc, ev)


def test_paged_prefill_workload_sampled(gpu):
    """The benchmark's workload (16 sequences, H = 32, last 2048 tokens of
    contexts 2048..16384) on sampled (sequence, head, token) rows."""
    p = inputs.paged_prefill_workload(device=gpu)
    log("fa_paged_prefill workload S16 H32 n_new=2048 (sampled rows)")
    o, l = fa.fa_paged_prefill(p.q, p.kcache, p.vcache, p.block_table, p.ctx_lens, scale=p.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    bt, cl = p.block_table.cpu().numpy(), p.ctx_lens.cpu().numpy()
    n_new = p.q.shape[2]
    for s, h in zip(rng.integers(0, 16, 6), rng.integers(0, 32, 6)):
        ctx = int(cl[s])
        t = np.arange(ctx)
        pages = torch.from_numpy(bt[s, t // 16].astype(np.int64)).to(gpu)
        slots = torch.from_numpy(t % 16).to(gpu)
        k = p.kcache[pages, int(h), slots]
        v = p.vcache[pages, int(h), slots]
        rows = np.sort(rng.choice(n_new, 8, replace=False))
        rows[0], rows[-1] = 0, n_new - 1
        pos = ctx - n_new + rows
        ro, rl = oracle.attention_rows(f64(p.q[s, h][rows]), pos, f64(k), f64(v), p.scale, True)
        check("workload s%d h%d" % (s, h), o[s, h][rows], l[s, h][rows], ro, rl)

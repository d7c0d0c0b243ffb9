"""GPU test of fa_check_paged_tables, through the C ABI, against a per-sequence
Python model of the paged calls' contract (PagedAttention block table,
"FlashAttention系列优化"): ctx_lens[s] in [0, max_blocks * page_size], and the
first ceil(ctx_lens[s] / page_size) entries of row s in [0, num_pages). The
check's result is exact: the number of sequences that break it, and the
smallest such index (-1 if none)."""
import sys

import numpy as np
import pytest
import torch

import exact_attention_106_amd as fa

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def model(table, ctx, page_size, num_pages):
    bad = []
    S, mb = table.shape
    for s in range(S):
        n = int(ctx[s])
        if n < 0 or n > mb * page_size:
            bad.append(s)
            continue
        used = -(-n // page_size)
        row = table[s, :used]
        if np.any((row < 0) | (row >= num_pages)):
            bad.append(s)
    return [len(bad), bad[0] if bad else -1]


def run(gpu, table, ctx, page_size, num_pages, out=None):
    t = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).to(gpu)
    c = torch.from_numpy(np.ascontiguousarray(ctx, dtype=np.int32)).to(gpu)
    r = fa.fa_check_paged_tables(t, c, page_size, num_pages, out=out)
    torch.cuda.synchronize()
    return r.cpu().tolist()


def valid_tables(rng, S, mb, page_size, num_pages):
    """Random contract-abiding tables: used entries in the pool, the rest
    garbage (-1, huge, negative), which the check must not read as errors."""
    ctx = rng.integers(0, mb * page_size + 1, size=S)
    ctx[: min(S, 3)] = [0, mb * page_size, 1][: min(S, 3)]
    table = rng.choice(np.array([-1, -7, num_pages, 1 << 30], dtype=np.int64), size=(S, mb))
    for s in range(S):
        used = -(-int(ctx[s]) // page_size)
        table[s, :used] = rng.integers(0, num_pages, size=used)
    return table, ctx


@pytest.mark.parametrize("S,mb,page_size,num_pages", [(1, 1, 16, 1), (7, 5, 16, 40), (64, 2048, 16, 131072),
                                                      (10000, 9, 3, 500)])
def test_valid_tables_pass(gpu, S, mb, page_size, num_pages):
    rng = np.random.default_rng(S + mb)
    table, ctx = valid_tables(rng, S, mb, page_size, num_pages)
    log("check_paged_tables valid S=%d mb=%d ps=%d P=%d" % (S, mb, page_size, num_pages))
    assert model(table, ctx, page_size, num_pages) == [0, -1]
    assert run(gpu, table, ctx, page_size, num_pages) == [0, -1]


def test_planted_errors(gpu):
    S, mb, ps, P = 10000, 9, 16, 300
    rng = np.random.default_rng(5)
    table, ctx = valid_tables(rng, S, mb, ps, P)
    ctx[5000], table[5000, :] = 3 * ps, -1
    table[5000, 2] = P                      # last used block, one past the pool
    ctx[9999] = 2 * ps + 1
    table[9999, 2] = -1                     # the partly used third block
    ctx[4096] = -1                          # negative length
    ctx[7777] = mb * ps + 1                 # longer than the row
    ctx[8000], table[8000, 1] = ps, -1      # unused entry: not an error
    ctx[8001], table[8001, 0] = 1, P - 1    # last page of the pool: fine
    want = model(table, ctx, ps, P)
    assert want == [4, 4096]
    log("check_paged_tables planted errors S=%d" % S)
    out = torch.full((2,), 12345, dtype=torch.int32, device=gpu)     # stale contents are overwritten
    assert run(gpu, table, ctx, ps, P, out=out) == want
    ctx[4096] = 0                           # second call on the same buffer: the next smallest
    assert run(gpu, table, ctx, ps, P, out=out) == [3, 5000]


def test_block_manager_tables_pass(gpu):
    bm = fa.BlockManager(64, 6, 12, 16)
    bm.add_seq(0, 100)
    bm.fork(0, 1)
    bm.add_seq(3, 17)
    for _ in range(20):
        bm.append_token(1)
    bm.add_seq(4, 1)
    bm.free_seq(4)
    table, ctx = bm.block_table()
    log("check_paged_tables block manager tables")
    assert model(table.numpy(), ctx.numpy(), 16, 64) == [0, -1]
    assert run(gpu, table.numpy(), ctx.numpy(), 16, 64) == [0, -1]
    assert run(gpu, table.numpy(), ctx.numpy(), 16, 7) == model(table.numpy(), ctx.numpy(), 16, 7)


def test_graph_replays(gpu):
    """The check recorded into a HIP graph: every replay, with the table
    changed eagerly in between, gives the eager result."""
    S, mb, ps, P = 300, 6, 16, 50
    rng = np.random.default_rng(9)
    table, ctx = valid_tables(rng, S, mb, ps, P)
    t = torch.from_numpy(table.astype(np.int32)).to(gpu)
    c = torch.from_numpy(ctx.astype(np.int32)).to(gpu)
    out = torch.empty((2,), dtype=torch.int32, device=gpu)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fa.fa_check_paged_tables(t, c, ps, P, out=out)      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.fa_check_paged_tables(t, c, ps, P, out=out)
    log("check_paged_tables graph replays")
    for rep in range(4):
        if rep:
            s = int(rng.integers(0, S))
            ctx[s] = max(int(ctx[s]), 1)
            table[s, 0] = P + rep
            t.copy_(torch.from_numpy(table.astype(np.int32)))
            c.copy_(torch.from_numpy(ctx.astype(np.int32)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().tolist()
        assert got == model(table, ctx, ps, P), rep
        eager = fa.fa_check_paged_tables(t, c, ps, P)
        torch.cuda.synchronize()
        assert eager.cpu().tolist() == got

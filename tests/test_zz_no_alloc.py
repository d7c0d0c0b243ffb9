"""The paged decode entry point that allocates nothing
(fa_paged_decode_noalloc, through the C ABI) against fa_paged_decode: same
kernels, so the outputs must agree bit for bit (a stricter bar than the bf16
tolerance). Two calls in a row on the shared static workspace, the second with
fewer sequences and shorter contexts than the first (its stale contents must
not leak into the second), then the first size again; and the host-side
rejection of sizes beyond the static buffer."""
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
    fa_mod.fa_version()
    return fa_mod


def _run_both(fa, p, gpu):
    q, kc, vc, bt, cl = (t.to(gpu) for t in (p.q, p.kcache, p.vcache, p.block_table, p.ctx_lens))
    o_ref, l_ref = fa.fa_paged_decode(q, kc, vc, bt, cl, scale=p.scale)
    o = torch.full_like(o_ref, float("nan"))
    l = torch.full_like(l_ref, float("nan"))
    fa.fa_paged_decode_noalloc(q, kc, vc, bt, cl, out=o, lse=l, scale=p.scale)
    torch.cuda.synchronize()
    return o, l, o_ref, l_ref


def test_noalloc_decode_matches_allocating_entry_point(fa, gpu):
    big = inputs.paged_pool(num_seqs=9, H=4, d=128, ctx_lo=900, ctx_hi=2600, seed=81, share=0.4)
    small = inputs.paged_pool(num_seqs=3, H=4, d=128, ctx_lo=1, ctx_hi=300, seed=82, share=0.0)
    for name, p in (("first, 9 sequences", big), ("second, 3 shorter sequences", small),
                    ("third, 9 sequences again", big)):
        log("fa_paged_decode_noalloc vs fa_paged_decode: %s" % name)
        o, l, o_ref, l_ref = _run_both(fa, p, gpu)
        assert torch.equal(o, o_ref), name + ": O differs"
        assert torch.equal(l, l_ref), name + ": L differs"
    # and the second size against the oracle, as every decode output
    o, l, _, _ = _run_both(fa, small, gpu)
    bits = lambda t: t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    ro, rl = oracle.paged_decode(oracle.bf16_bits_to_f64(bits(small.q)), bits(small.kcache), bits(small.vcache),
                                 small.block_table.numpy(), small.ctx_lens.numpy(), small.scale)
    assert np.max(np.abs(oracle.bf16_bits_to_f64(bits(o)) - ro)) <= 2e-2
    assert np.max(np.abs(l.cpu().double().numpy() - rl)) <= 1e-3


def test_noalloc_decode_rejects_sizes_beyond_the_buffer(fa, gpu):
    # 64 sequences x 32 heads x 2528 blocks needs 84.2 MB of workspace: rejected
    # on the host (no launch; the outputs keep their contents)
    limit = fa.fa_noalloc_scratch_bytes()
    assert limit == 80 << 20
    assert fa.fa_paged_decode_workspace_bytes(64, 32, 128, 16, 2528) > limit
    q = torch.zeros((64, 32, 128), dtype=torch.bfloat16, device=gpu)
    kc = torch.zeros((4, 32, 16, 128), dtype=torch.bfloat16, device=gpu)
    bt = torch.zeros((64, 2528), dtype=torch.int32, device=gpu)
    cl = torch.ones((64,), dtype=torch.int32, device=gpu)
    out = torch.full((64, 32, 128), 7.0, dtype=torch.bfloat16, device=gpu)
    with pytest.raises(fa.FaError) as e:
        fa.fa_paged_decode_noalloc(q, kc, kc, bt, cl, out=out)
    assert e.value.status == 8
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())

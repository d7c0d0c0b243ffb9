"""Seeded input generators: determinism and structural invariants (CPU)."""
import math

import numpy as np
import torch

import oracle
from exact_attention_106_amd import inputs


def test_dense_is_deterministic_and_bf16_rne():
    a = inputs.dense(1, 2, 33, 16, seed=7)
    b = inputs.dense(1, 2, 33, 16, seed=7)
    assert inputs.sha256_of(a.q, a.k, a.v) == inputs.sha256_of(b.q, b.k, b.v)
    c = inputs.dense(1, 2, 33, 16, seed=8)
    assert inputs.sha256_of(a.q) != inputs.sha256_of(c.q)
    # bf16 values are the RNE rounding of the fp32 draws
    rng = np.random.Generator(np.random.PCG64(7))
    q32 = rng.standard_normal((1, 2, 33, 16), dtype=np.float32)
    assert torch.equal(a.q, torch.from_numpy(q32).to(torch.bfloat16))
    assert a.scale == 0.25 and not a.causal


def test_haar_orthogonal():
    r = inputs.haar_orthogonal(np.random.Generator(np.random.PCG64(3)), 128)
    np.testing.assert_allclose(r.T @ r, np.eye(128), rtol=0, atol=1e-13)
    r2 = inputs.haar_orthogonal(np.random.Generator(np.random.PCG64(3)), 128)
    np.testing.assert_array_equal(r, r2)


def test_quantizer_blocks_and_saturation():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((2, 3, 300, 16)).astype(np.float32)
    x[0, 1, 5, 3] = 1e4
    codes, scales = inputs.quantize_e4m3_blocks(x)
    assert codes.dtype == torch.uint8 and codes.shape == x.shape
    assert scales.shape == (2, 3, 3)
    deq = oracle.dequant_e4m3(codes.numpy(), scales.numpy())
    assert np.all(np.isfinite(deq))
    # amax of each block maps to +-448 exactly (up to the fp32 division)
    xb = np.pad(x, [(0, 0), (0, 0), (0, 84), (0, 0)]).reshape(2, 3, 3, 128, 16)
    amax = np.abs(xb).max(axis=(-2, -1))
    np.testing.assert_allclose(scales.numpy(), amax / 448, rtol=1e-7)
    # relative error of e4m3 RNE is at most 2^-4 for normals; absolute 2^-10*scale for tiny values
    err = np.abs(deq - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * np.repeat(scales.numpy(), 128, axis=2)[:, :, :300, None])
    assert np.all(err <= bound * 1.0001)


def test_fp8_inputs_outliers_and_rotation():
    f = inputs.fp8_inputs(1, 2, 256, 32, seed=4, causal=True)
    g = inputs.fp8_inputs(1, 2, 256, 32, seed=4, causal=True)
    assert inputs.sha256_of(f.q8, f.k8, f.v8, f.q_scale) == inputs.sha256_of(g.q8, g.k8, g.v8, g.q_scale)
    assert f.q_scale.shape == (1, 2, 2)
    # no NaN code (0x7f / 0xff) is ever produced
    for t in (f.q8, f.k8, f.v8):
        assert not torch.any((t & 0x7F) == 0x7F)
    # without rotation the V outliers survive: exactly round(0.001 * numel) of them scaled by 20
    h = inputs.fp8_inputs(1, 1, 4000, 8, seed=5, rotate=False)
    v = oracle.dequant_e4m3(h.v8.numpy(), h.v_scale.numpy())
    assert np.sum(np.abs(v) > 8.0) >= 1


def test_paged_pool_invariants():
    p = inputs.paged_pool(num_seqs=10, H=2, d=8, ctx_lo=1, ctx_hi=200, seed=9, share=0.3)
    bt = p.block_table.numpy()
    ctx = p.ctx_lens.numpy()
    nb = (ctx + 15) // 16
    assert p.kcache.shape == (p.n_unique_pages, 2, 16, 8)
    used = []
    for s in range(10):
        assert np.all(bt[s, :nb[s]] >= 0) and np.all(bt[s, :nb[s]] < p.n_unique_pages)
        assert np.all(bt[s, nb[s]:] == -1)
        used.extend(bt[s, :nb[s]].tolist())
    counts = np.bincount(used, minlength=p.n_unique_pages)
    assert counts.min() >= 1 and counts.max() <= 2
    # sharing only within a pair, only as a prefix of full pages
    for s in range(1, 10, 2):
        sh = int(math.floor(0.3 * min(nb[s - 1], nb[s])))
        np.testing.assert_array_equal(bt[s, :sh], bt[s - 1, :sh])
        assert not set(bt[s, sh:nb[s]]) & set(bt[s - 1, :nb[s - 1]])
    assert p.n_unique_pages == nb.sum() - sum(int(math.floor(0.3 * min(nb[s - 1], nb[s])))
                                              for s in range(1, 10, 2))
    # tails past the context are NaN, valid slots are finite
    for s in range(10):
        last = bt[s, nb[s] - 1]
        rem = ctx[s] % 16
        if rem:
            assert torch.isnan(p.kcache[last, :, rem:]).all()
            assert torch.isfinite(p.kcache[last, :, :rem]).all()
    q = inputs.paged_pool(num_seqs=10, H=2, d=8, ctx_lo=1, ctx_hi=200, seed=9, share=0.3)
    assert inputs.sha256_of(p.kcache, p.vcache, p.block_table) == inputs.sha256_of(q.kcache, q.vcache, q.block_table)


def test_device_generators_seeded_and_in_range():
    """dense_on_device / fp8_on_device (run here on the CPU device): the same
    seed gives the same tensors, another seed others; E4M3 codes never NaN
    (0x7f / 0xff); block scales in [1/16, 1/8]."""
    a = inputs.dense_on_device(2, 3, 50, 64, seed=1, device="cpu")
    b = inputs.dense_on_device(2, 3, 50, 64, seed=1, device="cpu")
    c = inputs.dense_on_device(2, 3, 50, 64, seed=2, device="cpu")
    assert a.q.dtype == torch.bfloat16 and tuple(a.q.shape) == (2, 3, 50, 64)
    assert torch.equal(a.q, b.q) and torch.equal(a.v, b.v) and not torch.equal(a.q, c.q)
    assert abs(float(a.q.float().std()) - 1.0) < 0.1
    f = inputs.fp8_on_device(2, 3, 300, 128, seed=3, device="cpu")
    g = inputs.fp8_on_device(2, 3, 300, 128, seed=3, device="cpu")
    assert torch.equal(f.q8, g.q8) and torch.equal(f.v_scale, g.v_scale)
    for codes in (f.q8, f.k8, f.v8):
        assert codes.dtype == torch.uint8 and tuple(codes.shape) == (2, 3, 300, 128)
        assert not ((codes & 0x7F) == 0x7F).any()
    for s in (f.q_scale, f.k_scale, f.v_scale):
        assert tuple(s.shape) == (2, 3, 3)
        assert float(s.min()) >= 1 / 16 and float(s.max()) <= 1 / 8

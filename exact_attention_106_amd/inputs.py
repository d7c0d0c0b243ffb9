"""Seeded synthetic inputs for the attention workloads.

This module only draws and encodes inputs; it holds none of the attention
arithmetic. The CPU oracle and the HIP library both consume what it makes.

Workloads (shapes and value recipes):

* ``config1``: the worked example of the "FlashAttention系列优化" code listing:
  torch.manual_seed(456), then Q, K, V = torch.rand((16, 8)) in that order,
  fp32, scale 1, non-causal.
* ``dense``: Q, K, V ~ N(0, 1) drawn as fp32 from numpy PCG64(seed) in the
  order Q, K, V, rounded to bf16 (round-to-nearest-even) or kept fp32.
* ``fp8_inputs``: Q, K, V ~ N(0, 1) fp32 (PCG64(seed), order Q, K, V); per
  tensor exactly round(frac * numel) distinct flat positions multiplied by 20;
  Q and K multiplied by one Haar-random orthogonal d x d matrix (QR of a
  Gaussian with the column-sign correction); each (batch, head, 128-token) block
  quantised to OCP E4M3FN with scale = amax / 448 (fp32; amax 0 gives scale 1).
  This is the block quantisation and "incoherent processing" that the
  FlashAttention-3 part of "FlashAttention系列优化" (FP低精度) describes.
* ``paged_pool``: a PagedAttention-style KV cache (16-token pages, block table
  per sequence, PagedAttention section of the same page): context lengths
  uniform in [lo, hi]; sequences (2k, 2k+1) share their first
  floor(share * min(nb)) logical blocks through the same physical pages; unique
  pages get physical ids from a seeded permutation; page contents ~ N(0, 1)
  bf16; slots past a sequence's context in its last page hold NaN.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

PAGE_SIZE = 16
FP8_BLOCK = 128
E4M3_MAX = 448.0


@dataclass
class Dense:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    scale: float
    causal: bool
    name: str = ""

    @property
    def shape(self):
        return tuple(self.q.shape)


@dataclass
class Fp8:
    q8: torch.Tensor            # uint8 [B, H, N, d] (E4M3FN bit patterns)
    k8: torch.Tensor
    v8: torch.Tensor
    q_scale: torch.Tensor       # fp32 [B, H, ceil(N/128)]
    k_scale: torch.Tensor
    v_scale: torch.Tensor
    scale: float
    causal: bool
    name: str = ""

    @property
    def shape(self):
        return tuple(self.q8.shape)


@dataclass
class Paged:
    q: torch.Tensor             # bf16 [S, H, d]
    kcache: torch.Tensor        # bf16 [P, H, page_size, d]
    vcache: torch.Tensor
    block_table: torch.Tensor   # int32 [S, max_blocks], -1 padded
    ctx_lens: torch.Tensor      # int32 [S]
    scale: float
    page_size: int = PAGE_SIZE
    n_unique_pages: int = 0
    n_logical_pages: int = 0
    name: str = ""
    meta: dict = field(default_factory=dict)


def config1() -> Dense:
    """Worked example of the code listing (fp32, [1, 1, 16, 8])."""
    gen_state = torch.random.get_rng_state()
    try:
        torch.manual_seed(456)
        q = torch.rand((16, 8))
        k = torch.rand((16, 8))
        v = torch.rand((16, 8))
    finally:
        torch.random.set_rng_state(gen_state)
    return Dense(q.reshape(1, 1, 16, 8), k.reshape(1, 1, 16, 8), v.reshape(1, 1, 16, 8),
                 scale=1.0, causal=False, name="config1_f32_16x8")


def dense(B: int, H: int, N: int, d: int, seed: int, dtype: str = "bf16",
          scale: Optional[float] = None, causal: bool = False, device="cpu",
          name: str = "") -> Dense:
    rng = np.random.Generator(np.random.PCG64(seed))
    tensors = []
    for _ in range(3):
        x = torch.from_numpy(rng.standard_normal((B, H, N, d), dtype=np.float32))
        if dtype == "bf16":
            x = x.to(torch.bfloat16)
        elif dtype != "f32":
            raise ValueError(dtype)
        tensors.append(x.to(device))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return Dense(*tensors, scale=scale, causal=causal, name=name or f"dense_{dtype}_B{B}H{H}N{N}d{d}")


def dense_on_device(B: int, H: int, N: int, d: int, seed: int, device, scale: Optional[float] = None,
                    causal: bool = False, name: str = "") -> Dense:
    """Standard-normal bf16 Q, K, V drawn directly on the device by torch's
    seeded generator, for sizes whose host generation would take minutes (up
    to the 2^31 - 1 elements per tensor that the dense entry points accept).
    Not the same values as dense() for the same seed; the same seed on the
    same device gives the same tensors."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    tensors = [torch.randn((B, H, N, d), generator=g, device=device, dtype=torch.bfloat16) for _ in range(3)]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return Dense(*tensors, scale=scale, causal=causal, name=name or f"dense_dev_bf16_B{B}H{H}N{N}d{d}")


def fp8_on_device(B: int, H: int, N: int, d: int, seed: int, device, causal: bool = False,
                  name: str = "") -> Fp8:
    """E4M3 codes and per-block scales drawn on the device, for the largest
    sizes: codes are torch's float8_e4m3fn cast of 8 * N(0, 1) draws (|x| far
    below 448, so no NaN code), every block scale uniform in [1/16, 1/8], so
    the values are about N(0, 1). Not the block quantisation of bf16 inputs
    that fp8_inputs() performs."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    nsb = (N + FP8_BLOCK - 1) // FP8_BLOCK
    codes = [(8 * torch.randn((B, H, N, d), generator=g, device=device)).to(torch.float8_e4m3fn)
             .view(torch.uint8) for _ in range(3)]
    scales = [(1 + torch.rand((B, H, nsb), generator=g, device=device)) / 16 for _ in range(3)]
    return Fp8(*codes, *scales, scale=1.0 / math.sqrt(d), causal=causal,
               name=name or f"fp8_dev_B{B}H{H}N{N}d{d}")


def grad_out(B: int, H: int, N: int, d: int, seed: int, device="cpu") -> torch.Tensor:
    """Seeded upstream gradient dO for the backward pass: standard normal, bf16."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = torch.from_numpy(rng.standard_normal((B, H, N, d), dtype=np.float32))
    return x.to(torch.bfloat16).to(device)


def config2(device="cpu") -> Dense:
    return dense(4, 16, 2048, 64, seed=2, dtype="bf16", scale=1.0 / 8.0, causal=False,
                 device=device, name="mha_bf16_B4H16N2048d64")


def config3(device="cpu") -> Dense:
    return dense(1, 32, 16384, 128, seed=3, dtype="bf16", scale=1.0 / math.sqrt(128), causal=True,
                 device=device, name="causal_bf16_B1H32N16384d128")


def haar_orthogonal(rng: np.random.Generator, n: int) -> np.ndarray:
    """Haar-distributed orthogonal matrix: QR of a Gaussian, columns sign-fixed."""
    g = rng.standard_normal((n, n))
    qm, rm = np.linalg.qr(g)
    return qm * np.sign(np.diag(rm))[None, :]


def quantize_e4m3_blocks(x: np.ndarray, block: int = FP8_BLOCK):
    """x fp32 [..., N, d] -> (uint8 E4M3FN codes [..., N, d], fp32 scales [..., ceil(N/block)]).

    One scale per (leading index, block of ``block`` tokens x all d channels):
    scale = amax / 448, codes = round-to-nearest-even(clamp(x / scale)).
    """
    *lead, n, d = x.shape
    nblk = (n + block - 1) // block
    pad = nblk * block - n
    xp = np.pad(x, [(0, 0)] * len(lead) + [(0, pad), (0, 0)]) if pad else x
    xb = xp.reshape(*lead, nblk, block, d)
    amax = np.abs(xb).max(axis=(-2, -1)).astype(np.float32)
    scales = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = (xb / scales[..., None, None]).astype(np.float32)
    y = np.clip(y, -E4M3_MAX, E4M3_MAX).reshape(*lead, nblk * block, d)[..., :n, :]
    codes = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, torch.from_numpy(scales)


def fp8_inputs(B: int, H: int, N: int, d: int, seed: int, outlier_frac: float = 0.001,
               outlier_mult: float = 20.0, rotate: bool = True, scale: Optional[float] = None,
               causal: bool = True, device="cpu", name: str = "") -> Fp8:
    rng = np.random.Generator(np.random.PCG64(seed))
    xs = [rng.standard_normal((B, H, N, d), dtype=np.float32) for _ in range(3)]
    for x in xs:
        n_out = int(round(outlier_frac * x.size))
        if n_out:
            idx = rng.choice(x.size, size=n_out, replace=False)
            flat = x.reshape(-1)
            flat[idx] *= np.float32(outlier_mult)
    if rotate:
        r = haar_orthogonal(rng, d).astype(np.float32)
        xs[0] = xs[0] @ r
        xs[1] = xs[1] @ r
    outs = []
    scales = []
    for x in xs:
        c, s = quantize_e4m3_blocks(x)
        outs.append(c.to(device))
        scales.append(s.to(device))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return Fp8(*outs, *scales, scale=scale, causal=causal,
               name=name or f"fp8_B{B}H{H}N{N}d{d}")


def quant_inputs(B: int, H: int, N: int, d: int, seed: int, outlier_frac: float = 0.001,
                 outlier_mult: float = 20.0, device="cpu"):
    """bf16 x [B, H, N, d] (N(0,1) with a fraction of entries scaled up as
    outliers, as in fp8_inputs before rotation) and a bf16 Haar rotation [d, d]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((B, H, N, d), dtype=np.float32)
    n_out = int(round(outlier_frac * x.size))
    if n_out:
        idx = rng.choice(x.size, size=n_out, replace=False)
        x.reshape(-1)[idx] *= np.float32(outlier_mult)
    r = haar_orthogonal(rng, d).astype(np.float32)
    return (torch.from_numpy(x).to(torch.bfloat16).to(device),
            torch.from_numpy(r).to(torch.bfloat16).to(device))


def config4(device="cpu") -> Fp8:
    return fp8_inputs(2, 16, 8192, 128, seed=4, causal=True, device=device,
                      name="causal_fp8_B2H16N8192d128")


def paged_pool(num_seqs: int, H: int, d: int, ctx_lo: int, ctx_hi: int, seed: int,
               share: float = 0.1, page_size: int = PAGE_SIZE, max_blocks: Optional[int] = None,
               nan_tails: bool = True, scale: Optional[float] = None, device="cpu",
               chunk_pages: int = 2048, name: str = "") -> Paged:
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = rng.integers(ctx_lo, ctx_hi, size=num_seqs, endpoint=True).astype(np.int64)
    nb = (ctx + page_size - 1) // page_size
    if max_blocks is None:
        max_blocks = (ctx_hi + page_size - 1) // page_size
    # logical -> unique page index; pairs (2k, 2k+1) share a prompt prefix
    table_u = np.full((num_seqs, max_blocks), -1, dtype=np.int64)
    n_unique = 0
    for s in range(num_seqs):
        shared = 0
        if s % 2 == 1:
            shared = int(math.floor(share * min(nb[s - 1], nb[s])))
            table_u[s, :shared] = table_u[s - 1, :shared]
        cnt = int(nb[s]) - shared
        table_u[s, shared:nb[s]] = np.arange(n_unique, n_unique + cnt)
        n_unique += cnt
    perm = rng.permutation(n_unique).astype(np.int64)
    table = np.where(table_u >= 0, perm[np.maximum(table_u, 0)], -1).astype(np.int32)
    qf = rng.standard_normal((num_seqs, H, d), dtype=np.float32)
    q = torch.from_numpy(qf).to(torch.bfloat16).to(device)

    # page contents: torch generator on the target device, drawn chunk by chunk
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    caches = []
    for _ in range(2):
        c = torch.empty((n_unique, H, page_size, d), dtype=torch.bfloat16, device=device)
        for p0 in range(0, n_unique, chunk_pages):
            p1 = min(n_unique, p0 + chunk_pages)
            c[p0:p1] = torch.randn((p1 - p0, H, page_size, d), generator=g, device=device,
                                   dtype=torch.float32).to(torch.bfloat16)
        caches.append(c)
    if nan_tails:
        for s in range(num_seqs):
            rem = int(ctx[s] % page_size)
            if rem:
                last = int(table[s, nb[s] - 1])
                for c in caches:
                    c[last, :, rem:, :] = float("nan")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return Paged(q=q, kcache=caches[0], vcache=caches[1],
                 block_table=torch.from_numpy(table).to(device),
                 ctx_lens=torch.from_numpy(ctx.astype(np.int32)).to(device),
                 scale=scale, page_size=page_size, n_unique_pages=n_unique,
                 n_logical_pages=int(nb.sum()), name=name or f"paged_S{num_seqs}H{H}d{d}",
                 meta={"ctx_lo": ctx_lo, "ctx_hi": ctx_hi, "seed": seed, "share": share})


def paged_prefill_workload(device="cpu") -> Paged:
    """Chunked prefill through a block table: 16 sequences, H = 32, d = 128,
    contexts U{2048..16384} (PCG64(7)), shared prefixes and a shuffled pool as
    for the decode workload; q holds the last 2048 tokens of every sequence
    [16, 32, 2048, 128] (PCG64(8), N(0,1) -> bf16)."""
    p = paged_pool(16, 32, 128, 2048, 16384, seed=7, device=device, name="paged_prefill_S16H32d128")
    rng = np.random.Generator(np.random.PCG64(8))
    q = torch.from_numpy(rng.standard_normal((16, 32, 2048, 128), dtype=np.float32)).to(torch.bfloat16)
    p.q = q.to(device)
    return p


def block_mask(N: int, density: float, seed: int, causal: bool = True) -> torch.Tensor:
    """Seeded 128 x 128 block mask (uint8 [ceil(N/128)]^2) keeping a fraction
    `density` of the blocks (of the causal ones when causal), the diagonal
    always, so that every query keeps at least its own block."""
    nb = (N + 127) // 128
    rng = np.random.Generator(np.random.PCG64(seed))
    m = rng.random((nb, nb)) < density
    if causal:
        m &= np.tril(np.ones((nb, nb), dtype=bool))
    np.fill_diagonal(m, True)
    return torch.from_numpy(m.astype(np.uint8))


def config5(device="cpu") -> Paged:
    return paged_pool(64, 32, 128, 512, 32768, seed=5, device=device,
                      name="paged_decode_S64H32d128_ctx512-32768")


def sha256_of(*tensors) -> str:
    h = hashlib.sha256()
    for t in tensors:
        t = t.detach().cpu().contiguous()
        if t.dtype in (torch.bfloat16, torch.float8_e4m3fn):
            t = t.view(torch.uint8)
        h.update(t.numpy().tobytes())
    return h.hexdigest()

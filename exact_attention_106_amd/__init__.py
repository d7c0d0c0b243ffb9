"""MI355X (gfx950) fused exact attention: Python binding of libfa.so.

The functions carry the names of the C ABI in ``include/fa.h`` and only
marshal arguments: they check devices, dtypes and shapes, allocate outputs
with torch when the caller passes none, and call the library on the current
HIP stream. Every step of the computation runs in the library's HIP kernels;
there is no fallback. Importing this package does not load the library; the
first call does, and raises if it has not been built.
"""
from __future__ import annotations

import ctypes
import functools
import math
from typing import Optional, Sequence, Tuple

import torch

from . import _lib
from ._lib import FaError

__all__ = ["attention", "fa_fwd", "fa_fwd_f32", "fa_fwd_fp8", "fa_quantize_fp8", "fa_quantize_fp8_qkv", "fa_fwd_block_sparse", "fa_bwd", "fa_bwd_workspace_bytes",
           "fa_paged_decode", "fa_paged_decode_workspace_bytes", "fa_paged_decode_noalloc",
           "fa_noalloc_scratch_bytes", "fa_paged_prefill", "BlockManager",
           "fa_copy_pages", "fa_check_paged_tables",
           "fa_read_probe", "fa_status_str", "fa_version", "FaError"]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _on_device(fn):
    """Run an entry point under the device of its tensors: the library launches
    on the current HIP device with the caller's stream of that device, so all
    tensor arguments must share one device, which is made current for the call."""
    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        devs = {a.device for a in list(args) + list(kwargs.values())
                if isinstance(a, torch.Tensor) and a.device.type == "cuda"}
        if len(devs) > 1:
            raise ValueError("%s: all tensors must be on one device, got %s"
                             % (fn.__name__, sorted(str(d) for d in devs)))
        if not devs:
            return fn(*args, **kwargs)
        with torch.cuda.device(devs.pop()):
            return fn(*args, **kwargs)
    return wrapper


def _check_dev(name, t, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device (cuda/HIP) tensor" % name)
    if t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError("%s must have dtype %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _dense_common(q, k, v, dtype, out, lse, out_dtype):
    _check_dev("q", q, dtype)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    _check_dev("k", k, dtype, q.shape)
    _check_dev("v", v, dtype, q.shape)
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one device")
    B, H, N, d = q.shape
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=q.device)
    _check_dev("out", out, out_dtype, (B, H, N, d))
    if lse is not None:
        _check_dev("lse", lse, torch.float32, (B, H, N))
    return B, H, N, d, out


@_on_device
def fa_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: Optional[float] = None,
           causal: bool = False, out: Optional[torch.Tensor] = None,
           lse: Optional[torch.Tensor] = None, return_lse: bool = True
           ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """bf16 fused attention forward. q/k/v bf16 [B, H, N, d], d in {64, 128}.
    Returns (O bf16 [B, H, N, d], L fp32 [B, H, N] or None)."""
    B, H, N, d, out = _dense_common(q, k, v, torch.bfloat16, out, lse, torch.bfloat16)
    if lse is None and return_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = _lib.load().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, scale,
                            int(bool(causal)), _stream(q))
    _lib.check(st, "fa_fwd")
    return out, lse


@_on_device
def fa_fwd_f32(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: Optional[float] = None,
               causal: bool = False, out: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None, return_lse: bool = True
               ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """fp32 fused attention forward, 1 <= d <= 128."""
    B, H, N, d, out = _dense_common(q, k, v, torch.float32, out, lse, torch.float32)
    if lse is None and return_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = _lib.load().fa_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, scale,
                                int(bool(causal)), _stream(q))
    _lib.check(st, "fa_fwd_f32")
    return out, lse


def _as_u8(name, t):
    if isinstance(t, torch.Tensor) and t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    _check_dev(name, t, torch.uint8)
    return t


@_on_device
def fa_fwd_fp8(q8: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, q_scale: torch.Tensor,
               k_scale: torch.Tensor, v_scale: torch.Tensor, scale: Optional[float] = None,
               causal: bool = False, out: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None, return_lse: bool = True
               ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """FP8 (E4M3FN) fused attention forward with fp32 scales per (b, h, 128-token block).
    q8/k8/v8 uint8 or float8_e4m3fn [B, H, N, d], d in {64, 128}; scales fp32 [B, H, ceil(N/128)]."""
    q8, k8, v8 = _as_u8("q8", q8), _as_u8("k8", k8), _as_u8("v8", v8)
    if q8.dim() != 4:
        raise ValueError("q8 must be [B, H, N, d]")
    B, H, N, d = q8.shape
    _check_dev("k8", k8, torch.uint8, q8.shape)
    _check_dev("v8", v8, torch.uint8, q8.shape)
    nsb = (N + 127) // 128
    for nm, s in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)):
        _check_dev(nm, s, torch.float32, (B, H, nsb))
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    _check_dev("out", out, torch.bfloat16, (B, H, N, d))
    if lse is None and return_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    if lse is not None:
        _check_dev("lse", lse, torch.float32, (B, H, N))
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = _lib.load().fa_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_scale), _ptr(k_scale),
                                _ptr(v_scale), _ptr(out), _ptr(lse), B, H, N, d, scale,
                                int(bool(causal)), _stream(q8))
    _lib.check(st, "fa_fwd_fp8")
    return out, lse


@_on_device
def fa_quantize_fp8(x: torch.Tensor, rot: Optional[torch.Tensor] = None,
                    codes: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None
                    ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Fused incoherent rotation + FP8 block quantisation of bf16 x [B, H, N, 128]:
    y = x @ rot (rot bf16 [128, 128], or None for y = x), then per (b, h, 128-token
    block) scale = max|y| / 448 and E4M3FN codes of y / scale (nearest even).
    Returns (codes uint8 [B, H, N, 128], scales fp32 [B, H, ceil(N/128)]), the
    layout fa_fwd_fp8 reads."""
    _check_dev("x", x, torch.bfloat16)
    if x.dim() != 4:
        raise ValueError("x must be [B, H, N, d]")
    B, H, N, d = x.shape
    if rot is not None:
        _check_dev("rot", rot, torch.bfloat16, (d, d))
    if codes is None:
        codes = torch.empty((B, H, N, d), dtype=torch.uint8, device=x.device)
    codes = _as_u8("codes", codes)
    _check_dev("codes", codes, torch.uint8, (B, H, N, d))
    nsb = (N + 127) // 128
    if scales is None:
        scales = torch.empty((B, H, nsb), dtype=torch.float32, device=x.device)
    _check_dev("scales", scales, torch.float32, (B, H, nsb))
    st = _lib.load().fa_quantize_fp8(_ptr(x), _ptr(rot), _ptr(codes), _ptr(scales), B, H, N, d, _stream(x))
    _lib.check(st, "fa_quantize_fp8")
    return codes, scales


@_on_device
def fa_quantize_fp8_qkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, rot: Optional[torch.Tensor] = None,
                        out: Optional[Sequence[Tuple[torch.Tensor, torch.Tensor]]] = None
                        ) -> Tuple[Tuple[torch.Tensor, torch.Tensor], ...]:
    """fa_fwd_fp8's three inputs in one launch: Q and K rotated by rot (or not, if
    None), V never, each quantised as fa_quantize_fp8 does. Returns ((q_codes,
    q_scales), (k_codes, k_scales), (v_codes, v_scales)); out, if given, is that
    tuple of preallocated tensors."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(name, t, torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    _check_dev("k", k, torch.bfloat16, (B, H, N, d))
    _check_dev("v", v, torch.bfloat16, (B, H, N, d))
    if rot is not None:
        _check_dev("rot", rot, torch.bfloat16, (d, d))
    nsb = (N + 127) // 128
    if out is None:
        out = [(torch.empty((B, H, N, d), dtype=torch.uint8, device=q.device),
                torch.empty((B, H, nsb), dtype=torch.float32, device=q.device)) for _ in range(3)]
    if len(out) != 3:
        raise ValueError("out must hold three (codes, scales) pairs")
    res = []
    for name, (c, sc) in zip("qkv", out):
        c = _as_u8(name + "_codes", c)
        _check_dev(name + "_codes", c, torch.uint8, (B, H, N, d))
        _check_dev(name + "_scales", sc, torch.float32, (B, H, nsb))
        res.append((c, sc))
    (qc, qs), (kc, ks), (vc, vs) = res
    st = _lib.load().fa_quantize_fp8_qkv(_ptr(q), _ptr(k), _ptr(v), _ptr(rot), _ptr(qc), _ptr(kc), _ptr(vc),
                                         _ptr(qs), _ptr(ks), _ptr(vs), B, H, N, d, _stream(q))
    _lib.check(st, "fa_quantize_fp8_qkv")
    return tuple(res)


@_on_device
def fa_fwd_block_sparse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_mask: torch.Tensor,
                        scale: Optional[float] = None, causal: bool = False, dropout_p: float = 0.0,
                        seed: int = 0, out: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None, return_lse: bool = True
                        ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Block-sparse bf16 attention forward (128 x 128 blocks, d = 128) with optional
    dropout. block_mask: device uint8 (or bool) [ceil(N/128), ceil(N/128)]."""
    B, H, N, d, out = _dense_common(q, k, v, torch.bfloat16, out, lse, torch.bfloat16)
    if block_mask.dtype == torch.bool:
        block_mask = block_mask.to(torch.uint8)
    nb = (N + 127) // 128
    _check_dev("block_mask", block_mask, torch.uint8, (nb, nb))
    if lse is None and return_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = _lib.load().fa_fwd_block_sparse(_ptr(q), _ptr(k), _ptr(v), _ptr(block_mask), _ptr(out), _ptr(lse),
                                         B, H, N, d, scale, int(bool(causal)), float(dropout_p),
                                         int(seed) & 0xFFFFFFFFFFFFFFFF, _stream(q))
    _lib.check(st, "fa_fwd_block_sparse")
    return out, lse


def fa_bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(_lib.load().fa_bwd_workspace_bytes(B, H, N, d))


@_on_device
def fa_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
           dout: torch.Tensor, scale: Optional[float] = None, causal: bool = False,
           workspace: Optional[torch.Tensor] = None, dq: Optional[torch.Tensor] = None,
           dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None
           ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """bf16 attention backward for fa_fwd: (dq, dk, dv) bf16 [B, H, N, d] from
    q/k/v, the forward's O and L (lse), and dO. d in {64, 128}."""
    B, H, N, d, _ = _dense_common(q, k, v, torch.bfloat16, o, lse, torch.bfloat16)
    _check_dev("lse", lse, torch.float32, (B, H, N))
    _check_dev("dout", dout, torch.bfloat16, (B, H, N, d))
    grads = []
    for nm, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        if g is None:
            g = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q.device)
        _check_dev(nm, g, torch.bfloat16, (B, H, N, d))
        grads.append(g)
    need = fa_bwd_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_dev("workspace", workspace, (torch.uint8, torch.float32))
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    nbytes = workspace.numel() * workspace.element_size()
    st = _lib.load().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                            _ptr(grads[0]), _ptr(grads[1]), _ptr(grads[2]), B, H, N, d, scale,
                            int(bool(causal)), _ptr(workspace), nbytes, _stream(q))
    _lib.check(st, "fa_bwd")
    return grads[0], grads[1], grads[2]


class _Attention(torch.autograd.Function):
    """fa_fwd forward, fa_bwd backward (O and L kept from the forward)."""

    @staticmethod
    def forward(ctx, q, k, v, scale, causal):
        o, lse = fa_fwd(q, k, v, scale=scale, causal=causal)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.scale, ctx.causal = scale, causal
        return o

    @staticmethod
    def backward(ctx, dout):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = fa_bwd(q, k, v, o, lse, dout.to(torch.bfloat16).contiguous(), scale=ctx.scale,
                            causal=ctx.causal)
        return dq, dk, dv, None, None


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: Optional[float] = None,
              causal: bool = False) -> torch.Tensor:
    """Exact attention O = softmax(scale * Q K^T) V (bf16 [B, H, N, d], d in {64,
    128}) as a differentiable torch op: the forward is fa_fwd, the gradient
    fa_bwd with the forward's O and L, so a model can train through it."""
    return _Attention.apply(q, k, v, scale, bool(causal))


def fa_paged_decode_workspace_bytes(num_seqs: int, H: int, d: int, page_size: int,
                                    max_blocks_per_seq: int) -> int:
    return int(_lib.load().fa_paged_decode_workspace_bytes(num_seqs, H, d, page_size,
                                                           max_blocks_per_seq))


@_on_device
def fa_paged_decode(q: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor,
                    block_table: torch.Tensor, ctx_lens: torch.Tensor,
                    scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    return_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Paged-KV decode. q bf16 [S, H, d]; caches bf16 [P, H, page_size, d];
    block_table int32 [S, max_blocks]; ctx_lens int32 [S]."""
    _check_dev("q", q, torch.bfloat16)
    if q.dim() != 3:
        raise ValueError("q must be [S, H, d]")
    S, H, d = q.shape
    _check_dev("kcache", kcache, torch.bfloat16)
    if kcache.dim() != 4 or kcache.shape[1] != H or kcache.shape[3] != d:
        raise ValueError("kcache must be [P, H, page_size, d]")
    _check_dev("vcache", vcache, torch.bfloat16, kcache.shape)
    P, _, page_size, _ = kcache.shape
    _check_dev("block_table", block_table, torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != S:
        raise ValueError("block_table must be [S, max_blocks]")
    _check_dev("ctx_lens", ctx_lens, torch.int32, (S,))
    max_blocks = block_table.shape[1]
    need = fa_paged_decode_workspace_bytes(S, H, d, page_size, max_blocks)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=q.device)
    _check_dev("workspace", workspace, torch.uint8)
    if out is None:
        out = torch.empty((S, H, d), dtype=torch.bfloat16, device=q.device)
    _check_dev("out", out, torch.bfloat16, (S, H, d))
    if lse is None and return_lse:
        lse = torch.empty((S, H), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_dev("lse", lse, torch.float32, (S, H))
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = _lib.load().fa_paged_decode(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(block_table),
                                     _ptr(ctx_lens), _ptr(out), _ptr(lse), S, H, d, page_size,
                                     max_blocks, P, scale, _ptr(workspace),
                                     workspace.numel(), _stream(q))
    _lib.check(st, "fa_paged_decode")
    return out, lse


def fa_noalloc_scratch_bytes() -> int:
    return int(_lib.load().fa_noalloc_scratch_bytes())


@_on_device
def fa_paged_decode_noalloc(q: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor,
                            block_table: torch.Tensor, ctx_lens: torch.Tensor, out: torch.Tensor,
                            lse: Optional[torch.Tensor] = None, scale: Optional[float] = None) -> None:
    """fa_paged_decode with the library's static workspace: allocates nothing
    (no workspace, no outputs), so the caller passes `out` (and `lse`, or None).
    Same shapes as fa_paged_decode; raises FaError(FA_ERR_SCRATCH_LIMIT) when the
    sizes need more than fa_noalloc_scratch_bytes() of workspace."""
    _check_dev("q", q, torch.bfloat16)
    if q.dim() != 3:
        raise ValueError("q must be [S, H, d]")
    S, H, d = q.shape
    _check_dev("kcache", kcache, torch.bfloat16)
    if kcache.dim() != 4 or kcache.shape[1] != H or kcache.shape[3] != d:
        raise ValueError("kcache must be [P, H, page_size, d]")
    _check_dev("vcache", vcache, torch.bfloat16, kcache.shape)
    P, _, page_size, _ = kcache.shape
    _check_dev("block_table", block_table, torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != S:
        raise ValueError("block_table must be [S, max_blocks]")
    _check_dev("ctx_lens", ctx_lens, torch.int32, (S,))
    _check_dev("out", out, torch.bfloat16, (S, H, d))
    if lse is not None:
        _check_dev("lse", lse, torch.float32, (S, H))
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = _lib.load().fa_paged_decode_noalloc(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(block_table),
                                             _ptr(ctx_lens), _ptr(out), _ptr(lse), S, H, d, page_size,
                                             block_table.shape[1], P, scale, _stream(q))
    _lib.check(st, "fa_paged_decode_noalloc")


@_on_device
def fa_paged_prefill(q: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor,
                     block_table: torch.Tensor, ctx_lens: torch.Tensor, scale: Optional[float] = None,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     return_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Paged (chunked) prefill. q bf16 [S, H, n_new, d]: the n_new newest tokens of each
    sequence (positions ctx_lens[s] - n_new ..), attending causally to the paged cache."""
    _check_dev("q", q, torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [S, H, n_new, d]")
    S, H, n_new, d = q.shape
    _check_dev("kcache", kcache, torch.bfloat16)
    if kcache.dim() != 4 or kcache.shape[1] != H or kcache.shape[3] != d:
        raise ValueError("kcache must be [P, H, page_size, d]")
    _check_dev("vcache", vcache, torch.bfloat16, kcache.shape)
    P, _, page_size, _ = kcache.shape
    _check_dev("block_table", block_table, torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != S:
        raise ValueError("block_table must be [S, max_blocks]")
    _check_dev("ctx_lens", ctx_lens, torch.int32, (S,))
    if out is None:
        out = torch.empty((S, H, n_new, d), dtype=torch.bfloat16, device=q.device)
    _check_dev("out", out, torch.bfloat16, (S, H, n_new, d))
    if lse is None and return_lse:
        lse = torch.empty((S, H, n_new), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_dev("lse", lse, torch.float32, (S, H, n_new))
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = _lib.load().fa_paged_prefill(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(block_table),
                                      _ptr(ctx_lens), _ptr(out), _ptr(lse), S, H, n_new, d, page_size,
                                      block_table.shape[1], P, scale, _stream(q))
    _lib.check(st, "fa_paged_prefill")
    return out, lse


class BlockManager:
    """Paged KV block manager of libfa.so (fa_bm_*): on-demand pages, shared
    pages with reference counts, copy-on-write. The state is a host buffer
    owned by this object; every method is one library call."""

    def __init__(self, num_pages: int, max_seqs: int, max_blocks_per_seq: int, page_size: int = 16):
        lib = _lib.load()
        nbytes = int(lib.fa_bm_state_bytes(num_pages, max_seqs, max_blocks_per_seq))
        if nbytes == 0:
            raise ValueError("num_pages, max_seqs and max_blocks_per_seq must be positive")
        self._buf = ctypes.create_string_buffer(nbytes)
        self.num_pages, self.max_seqs, self.max_blocks, self.page_size = (
            num_pages, max_seqs, max_blocks_per_seq, page_size)
        _lib.check(lib.fa_bm_init(self._buf, nbytes, num_pages, max_seqs, max_blocks_per_seq, page_size),
                   "fa_bm_init")

    def add_seq(self, seq: int, num_tokens: int) -> None:
        _lib.check(_lib.load().fa_bm_add_seq(self._buf, seq, num_tokens), "fa_bm_add_seq")

    def fork(self, parent: int, child: int) -> None:
        _lib.check(_lib.load().fa_bm_fork(self._buf, parent, child), "fa_bm_fork")

    def append_token(self, seq: int) -> Tuple[int, int]:
        """Reserve one more token of seq; returns (src, dst) pages to copy first, or (-1, -1)."""
        src, dst = ctypes.c_int32(-1), ctypes.c_int32(-1)
        _lib.check(_lib.load().fa_bm_append_token(self._buf, seq, ctypes.byref(src), ctypes.byref(dst)),
                   "fa_bm_append_token")
        return src.value, dst.value

    def free_seq(self, seq: int) -> None:
        _lib.check(_lib.load().fa_bm_free_seq(self._buf, seq), "fa_bm_free_seq")

    def num_free_pages(self) -> int:
        return int(_lib.load().fa_bm_num_free_pages(self._buf))

    def seq_len(self, seq: int) -> int:
        return int(_lib.load().fa_bm_seq_len(self._buf, seq))

    def refcount(self, page: int) -> int:
        return int(_lib.load().fa_bm_page_refcount(self._buf, page))

    def block_table(self) -> Tuple[torch.Tensor, torch.Tensor]:
        """(block_table int32 [max_seqs, max_blocks], ctx_lens int32 [max_seqs]) on the host."""
        table = torch.empty((self.max_seqs, self.max_blocks), dtype=torch.int32)
        ctx = torch.empty((self.max_seqs,), dtype=torch.int32)
        _lib.check(_lib.load().fa_bm_block_table(self._buf, _ptr(table), _ptr(ctx)), "fa_bm_block_table")
        return table, ctx


@_on_device
def fa_copy_pages(kcache: torch.Tensor, vcache: torch.Tensor, src: torch.Tensor, dst: torch.Tensor) -> None:
    """Copy pages src[i] -> dst[i] of both caches (bf16 [P, H, page_size, d]); src, dst device int32 [n]."""
    _check_dev("kcache", kcache, torch.bfloat16)
    if kcache.dim() != 4:
        raise ValueError("kcache must be [P, H, page_size, d]")
    _check_dev("vcache", vcache, torch.bfloat16, kcache.shape)
    n = src.numel()
    _check_dev("src", src, torch.int32, (n,))
    _check_dev("dst", dst, torch.int32, (n,))
    P, H, ps, d = kcache.shape
    st = _lib.load().fa_copy_pages(_ptr(kcache), _ptr(vcache), _ptr(src), _ptr(dst), n, P, H, d, ps,
                                   _stream(kcache))
    _lib.check(st, "fa_copy_pages")


@_on_device
def fa_check_paged_tables(block_table: torch.Tensor, ctx_lens: torch.Tensor, page_size: int, num_pages: int,
                          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Check a block table and context lengths against the paged calls' contract
    on the device. Returns a device int32 tensor [2]: the number of sequences that
    break it, and the smallest such sequence index (-1 if none)."""
    _check_dev("block_table", block_table, torch.int32)
    if block_table.dim() != 2:
        raise ValueError("block_table must be [S, max_blocks]")
    S, max_blocks = block_table.shape
    _check_dev("ctx_lens", ctx_lens, torch.int32, (S,))
    if out is None:
        out = torch.empty((2,), dtype=torch.int32, device=block_table.device)
    _check_dev("out", out, torch.int32, (2,))
    st = _lib.load().fa_check_paged_tables(_ptr(block_table), _ptr(ctx_lens), S, max_blocks, int(page_size),
                                           int(num_pages), _ptr(out), _stream(block_table))
    _lib.check(st, "fa_check_paged_tables")
    return out


@_on_device
def fa_read_probe(src: torch.Tensor, sink: torch.Tensor) -> None:
    """Stream-read every byte of the contiguous device tensor src once (a
    measurement helper: the plain read rate of this GPU); XORs the data into
    sink, a device int32 tensor of one element."""
    if not isinstance(src, torch.Tensor) or src.device.type != "cuda" or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    _check_dev("sink", sink, torch.int32, (1,))
    st = _lib.load().fa_read_probe(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(src))
    _lib.check(st, "fa_read_probe")


def fa_status_str(status: int) -> str:
    return _lib.status_str(status)


def fa_version() -> int:
    return int(_lib.load().fa_version())

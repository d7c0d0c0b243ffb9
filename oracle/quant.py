"""Incoherent processing + FP8 block quantisation: plain fp64 CPU reference.

TEST INFRASTRUCTURE ONLY (see the package docstring): only the test suite,
the package smoke check and the benchmark's CPU leg use it; it shares no code
with the HIP library.

What it computes, written out from the definitions:
  y = x R               incoherent processing: Q and K are multiplied by one
                        random orthogonal matrix before quantisation, which
                        spreads outliers and keeps (QR)(KR)^T = QK^T
                        ("FlashAttention系列优化", FlashAttentionV3 / FP低精度);
                        R = identity (no rotation) for V
  s_b = max |y| / 448   block quantisation: one scale per block of 128 tokens
                        of one (batch, head), over all channels (same section;
                        91haoming.cn FlashAttention v1-v3 article, v3 FP8
                        part); s_b = 1 for an all-zero block; the last block of
                        a row holds the remaining tokens only. The scale is
                        stored as fp32: s_b is amax / 448 rounded to the
                        nearest fp32 (computed in fp64 and rounded once more to
                        fp32, which for a quotient gives the correctly rounded
                        fp32 result since 53 >= 2 * 24 + 2)
  code = E4M3FN(clamp(y / s_b, -448, 448)), with the stored s_b, nearest
                        value, ties to the even code (last mantissa bit 0):
                        decode(code) * s_b is then the grid point nearest y.
                        The pages fix no precision for this decision; it is
                        taken on y / s_b rounded to fp32, the precision of the
                        stored scale (rounding the fp64 quotient once more to
                        fp32 gives the correctly rounded fp32 quotient)
The E4M3FN format (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
exponent field 0 = subnormal, S.1111.111 = NaN, no infinities, largest
finite 448) is the OCP 8-bit floating point format (OFP8 specification,
2023); the decoder below is written from that definition and the encoder
picks the nearest decoded value.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
BLOCK = 128


def e4m3_decode_table() -> np.ndarray:
    """fp64 value of every byte 0..255 (NaN for the two NaN codes)."""
    out = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            out[c] = np.nan
        elif e == 0:
            out[c] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            out[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_TABLE = e4m3_decode_table()
_POS = _TABLE[:0x7F]            # codes 0x00 .. 0x7e: 0 .. 448, increasing


def e4m3_decode(codes) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3FN code of each finite |x| <= 448, ties to the even code."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_encode takes finite values with |x| <= 448")
    a = np.abs(x)
    hi = np.searchsorted(_POS, a, side="left")          # first value >= |x|
    hi = np.minimum(hi, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo).astype(np.uint8)
    neg = np.signbit(x)
    return np.where(neg, mag | 0x80, mag).astype(np.uint8)


def rotate_quantize(x, rot=None, block: int = BLOCK):
    """x [..., N, d] (any float dtype, taken as fp64), rot [d, d] or None.

    Returns (codes uint8 [..., N, d], scales fp64 [..., ceil(N / block)],
    y fp64 [..., N, d]).
    """
    x = np.asarray(x, dtype=np.float64)
    y = x if rot is None else x @ np.asarray(rot, dtype=np.float64)
    *lead, n, d = y.shape
    nb = (n + block - 1) // block
    scales = np.empty((*lead, nb), dtype=np.float64)
    codes = np.empty(y.shape, dtype=np.uint8)
    for b in range(nb):
        yb = y[..., b * block:(b + 1) * block, :]
        amax = np.abs(yb).max(axis=(-2, -1))
        s = np.where(amax > 0, amax / E4M3_MAX, 1.0).astype(np.float32).astype(np.float64)
        scales[..., b] = s
        q = (yb / s[..., None, None]).astype(np.float32).astype(np.float64)
        q = np.clip(q, -E4M3_MAX, E4M3_MAX)
        codes[..., b * block:(b + 1) * block, :] = e4m3_encode(q)
    return codes, scales, y


def dequantize(codes, scales, block: int = BLOCK) -> np.ndarray:
    """decode(code) * scale of its block, fp64."""
    v = e4m3_decode(codes)
    s = np.repeat(np.asarray(scales, dtype=np.float64), block, axis=-1)[..., : v.shape[-2]]
    return v * s[..., None]

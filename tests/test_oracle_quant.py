"""Pins of the FP8 quantisation oracle (oracle/quant.py).

- the E4M3FN decoder against the special values of the OCP FP8 specification
  (tests/golden/e4m3fn_values.txt) and against torch's float8_e4m3fn type for
  all 256 bytes (a library routine with the same definition);
- the encoder: a round trip of every finite code, torch's float8_e4m3fn cast
  (round to nearest even) on random values over all binades and on every exact
  midpoint between neighbouring values (ties go to the even code);
- the block structure: a pure-Python loop over the tokens of a ragged case;
- incoherent processing: the scores (QR)(KR)^T equal QK^T, rows keep their
  norm, the largest element of a block lands on code 448, the dequantised
  value is within half a step of y, and with outliers the rotation lowers the
  quantisation error of the scores (the pages' reason for the rotation);
- block scales lower the error of a tensor with one outlier block compared
  with one scale for the whole tensor (the pages' reason for block scales).
"""
import math
import os

import numpy as np
import torch

from oracle import quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3fn_values.txt")


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_encode(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decoder_special_values():
    n = 0
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        code, val = [t.strip() for t in line.split("|")]
        got = quant.e4m3_decode([int(code, 16)])[0]
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val)
            assert math.copysign(1.0, got) == math.copysign(1.0, float(val))
        n += 1
    assert n == 10


def test_decoder_matches_torch_all_bytes():
    codes = np.arange(256)
    a, b = quant.e4m3_decode(codes), _torch_decode(codes)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    ok = ~np.isnan(a)
    assert np.array_equal(a[ok], b[ok])
    assert np.array_equal(np.signbit(a[ok]), np.signbit(b[ok]))
    assert int(ok.sum()) == 254


def test_encoder_round_trip():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(quant.e4m3_encode(quant.e4m3_decode(codes)), codes)


def test_encoder_matches_torch_cast_random():
    rng = np.random.default_rng(3)
    mant = rng.uniform(1.0, 2.0, size=200000)
    expo = rng.integers(-12, 9, size=mant.size)
    x = mant * np.exp2(expo) * rng.choice([-1.0, 1.0], size=mant.size)
    x = np.clip(x, -448.0, 448.0).astype(np.float32)
    assert np.array_equal(quant.e4m3_encode(x.astype(np.float64)), _torch_encode(x))


def test_encoder_ties_to_even():
    pos = quant.e4m3_decode(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2          # exact in fp32 and fp64
    got = quant.e4m3_encode(mids)
    assert np.all(got % 2 == 0)
    assert np.array_equal(got, _torch_encode(mids.astype(np.float32)))
    assert np.array_equal(quant.e4m3_encode(-mids), got | 0x80)


def test_block_scales_by_token_loop():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 300, 8)) * 3
    codes, scales, _ = quant.rotate_quantize(x, None)
    assert scales.shape == (2, 3)
    for b in range(2):
        for blk in range(3):
            m = 0.0
            for t in range(blk * 128, min(300, blk * 128 + 128)):
                for c in range(8):
                    m = max(m, abs(x[b, t, c]))
            assert scales[b, blk] == float(np.float32(m / 448.0))
            t = min(299, blk * 128 + 7)
            assert codes[b, t, 3] == quant.e4m3_encode(np.clip(x[b, t, 3] / scales[b, blk], -448, 448))


def test_zero_block_has_unit_scale():
    x = np.zeros((1, 130, 4))
    x[0, 129, 1] = -2.0
    codes, scales, _ = quant.rotate_quantize(x, None)
    assert scales[0, 0] == 1.0 and np.all(codes[0, :128] == 0)
    assert codes[0, 129, 1] == 0xFE


def _haar(seed, n):
    g = np.random.default_rng(seed).standard_normal((n, n))
    qm, rm = np.linalg.qr(g)
    return qm * np.sign(np.diag(rm))[None, :]


def test_rotation_invariants_and_error_bound():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((2, 256, 64))
    k = rng.standard_normal((2, 256, 64))
    r = _haar(8, 64)
    cq, sq, yq = quant.rotate_quantize(q, r)
    _, _, yk = quant.rotate_quantize(k, r)
    np.testing.assert_allclose(yq @ np.swapaxes(yk, -1, -2), q @ np.swapaxes(k, -1, -2), rtol=0, atol=1e-11)
    np.testing.assert_allclose(np.linalg.norm(yq, axis=-1), np.linalg.norm(q, axis=-1), rtol=1e-13)
    # the element of largest magnitude of every block maps to +-448
    for b in range(2):
        for blk in range(2):
            blockv = yq[b, blk * 128:(blk + 1) * 128]
            i = np.unravel_index(np.argmax(np.abs(blockv)), blockv.shape)
            assert cq[b, blk * 128 + i[0], i[1]] & 0x7F == 0x7E
    # |dequantised - y| <= half the spacing of E4M3 at that magnitude, times the scale
    deq = quant.dequantize(cq, sq)
    s = np.repeat(sq, 128, axis=-1)[..., None]
    a = np.abs(yq / s)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    half_step = np.exp2(e - 3) / 2
    assert np.all(np.abs(deq - yq) <= half_step * s * (1 + 1e-12))


def test_rotation_reduces_score_error_with_outliers():
    rng = np.random.default_rng(11)
    d, n = 128, 512
    q = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    for x in (q, k):
        x[:, 5] *= 30.0                      # an outlier channel
    r = _haar(12, d)
    ref = q @ k.T
    errs = []
    for rot in (None, r):
        cq, sq, _ = quant.rotate_quantize(q, rot)
        ck, sk, _ = quant.rotate_quantize(k, rot)
        est = quant.dequantize(cq, sq) @ quant.dequantize(ck, sk).T
        errs.append(np.linalg.norm(est - ref) / np.linalg.norm(ref))
    assert errs[1] < 0.5 * errs[0]


def test_block_scales_beat_one_tensor_scale():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((1024, 64))
    x[:128] *= 1e5                           # one block far above the rest
    # E4M3's relative step is the same at every normal magnitude, so one scale
    # hurts only the values it pushes into the subnormals: the other blocks
    c, s, _ = quant.rotate_quantize(x, None)
    e_block = np.linalg.norm(quant.dequantize(c, s)[128:] - x[128:]) / np.linalg.norm(x[128:])
    c1, s1, _ = quant.rotate_quantize(x, None, block=1024)
    e_tensor = np.linalg.norm(quant.dequantize(c1, s1, block=1024)[128:] - x[128:]) / np.linalg.norm(x[128:])
    assert e_block < 0.05 and e_tensor > 0.5

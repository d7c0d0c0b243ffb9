"""Why the FP8 forward keeps P.V in bf16: P rounded to E4M3 breaks the parity
bound on the FP8 workload, P rounded to bf16 does not (CPU, fp64 arithmetic).

FlashAttention-3's FP8 path ("FlashAttention系列优化", FlashAttentionV3 /
FP低精度; 91haoming.cn article, FlashAttention v3 / FP8) quantises Q, K and V
per block; with P.V in FP8 the softmax weights P would be E4M3 too, with a
3-bit mantissa. This test takes the dequantised inputs of the FP8 workload
(B2 H16 N8192 d128, causal, outliers x20, Haar rotation, 128-token block
scales), computes exact scores and weights p = exp(s - rowmax) in fp64, and
forms O = (round(p) V) / l with round() either bf16 (what the kernel does) or
E4M3 after the most favourable scaling (p * 256, so the row max maps inside
E4M3's range), with l the exact sum. Everything else is exact, so the measured
error is the weight rounding alone (plus bf16 output rounding). Bound: the FP8
parity tolerance 8e-2 + half a bf16 ulp of |O|. The rows checked are the first
512 of one head (early causal rows average few keys, so one rounding error
weighs most there) plus a random sample.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_attention_106_amd import inputs


def _round(a, dtype):
    return torch.from_numpy(a.astype(np.float32)).to(dtype).to(torch.float32).numpy().astype(np.float64)


def _half_ulp_bf16(x):
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 8)


@pytest.fixture(scope="module")
def head():
    x = inputs.fp8_inputs(2, 2, 8192, 128, seed=4, causal=True)   # the FP8 workload's generator, 2 heads
    b, h = 1, 1
    q = oracle.dequant_e4m3(x.q8.numpy(), x.q_scale.numpy())[b, h]
    k = oracle.dequant_e4m3(x.k8.numpy(), x.k_scale.numpy())[b, h]
    v = oracle.dequant_e4m3(x.v8.numpy(), x.v_scale.numpy())[b, h]
    rows = np.r_[0:512, np.random.default_rng(0).choice(np.arange(512, 8192), 128, replace=False)]
    s = x.scale * (q[rows] @ k.T)
    s = np.where(np.arange(8192)[None, :] <= rows[:, None], s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    l = p.sum(axis=1, keepdims=True)
    return p, l, v, (p @ v) / l


def _error_over_bound(o, o_ref):
    err = np.abs(o - o_ref)
    return float(err.max()), float(np.max(err - (8e-2 + _half_ulp_bf16(o_ref))))


def test_p_in_bf16_meets_the_fp8_bound(head):
    p, l, v, o_ref = head
    o = _round((_round(p, torch.bfloat16) @ v) / l, torch.bfloat16)
    err, margin = _error_over_bound(o, o_ref)
    print("P in bf16: max|dO| = %.4f, margin to the bound %.4f" % (err, margin))
    assert margin <= 0


def test_p_in_e4m3_breaks_the_fp8_bound(head):
    p, l, v, o_ref = head
    o = _round((_round(p * 256.0, torch.float8_e4m3fn) / 256.0 @ v) / l, torch.bfloat16)
    err, margin = _error_over_bound(o, o_ref)
    rms = float(np.sqrt(np.mean((o - o_ref) ** 2)))
    print("P in E4M3: max|dO| = %.4f (rms %.4f), exceeds the bound by %.4f" % (err, rms, margin))
    assert margin > 0

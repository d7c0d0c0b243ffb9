"""Build libfa.so (gfx950 only) in-tree with hipcc.

    python -m exact_attention_106_amd.build

Each HIP source is compiled to an object in ``_build/`` in parallel, then
linked into ``exact_attention_106_amd/libfa.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")
# the prefill kernel template (fwd_prefill.h) is instantiated in five units
# that compile in parallel
SOURCES = ["api.hip", "fwd_f32.hip", "fwd_prefill_bf16.hip", "fwd_prefill_bf16_d64.hip", "fwd_prefill_fp8.hip",
           "fwd_prefill_fp8_d64.hip", "fwd_prefill_paged.hip", "decode.hip", "bwd.hip", "block_manager.hip", "fwd_sparse.hip", "fp8_quant.hip",
           "read_probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def common_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # packed fp32 VALU ops stay off in every HIP object
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Wno-unused-command-line-argument",
    ]


# per-source flags: the prefill kernel never produces NaN on purpose (masking
# uses -inf), and without NaN semantics max(max(a, b), c) is one v_max3
# backward and block-sparse forward: MFMA accumulators in VGPRs where they
# fit (the builtin MFMAs otherwise keep S in AGPRs and copy it out for the
# softmax, and shuffle O between AGPRs around the rescale branch; measured:
# the block-sparse forward runs 16 % faster this way, the paged prefill 9 %
# slower, so that one keeps the default)
PREFILL_FLAGS = ["-fno-honor-nans"]
EXTRA = {"fwd_prefill_bf16.hip": PREFILL_FLAGS, "fwd_prefill_bf16_d64.hip": PREFILL_FLAGS,
         "fwd_prefill_fp8.hip": PREFILL_FLAGS, "fwd_prefill_fp8_d64.hip": PREFILL_FLAGS,
         "fwd_prefill_paged.hip": PREFILL_FLAGS,
         "bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "fwd_sparse.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags() + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", str(os.cpu_count() or 8))))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB, file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()

"""ctypes loader for the in-tree libfa.so. Fails loudly when it is missing."""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfa.so")

FA_OK = 0
STATUS_NAMES = {
    0: "FA_OK", 1: "FA_ERR_NULL_PTR", 2: "FA_ERR_BAD_SHAPE", 3: "FA_ERR_UNSUPPORTED",
    4: "FA_ERR_WORKSPACE", 5: "FA_ERR_HIP",
}
# every symbol include/fa.h declares
EXPORTS = ("fa_fwd", "fa_fwd_f32", "fa_fwd_fp8", "fa_bwd_workspace_bytes", "fa_bwd",
           "fa_paged_decode_workspace_bytes", "fa_paged_decode", "fa_status_str", "fa_version")


class FaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lock = threading.Lock()
_lib = None


def load() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libfa.so is not built (%s); run `python -m exact_attention_106_amd.build`" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
        lib.fa_fwd.restype = i
        lib.fa_fwd_f32.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
        lib.fa_fwd_f32.restype = i
        lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
        lib.fa_fwd_fp8.restype = i
        lib.fa_bwd_workspace_bytes.argtypes = [i, i, i, i]
        lib.fa_bwd_workspace_bytes.restype = sz
        lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, sz, vp]
        lib.fa_bwd.restype = i
        lib.fa_paged_decode_workspace_bytes.argtypes = [i, i, i, i, i]
        lib.fa_paged_decode_workspace_bytes.restype = sz
        lib.fa_paged_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
        lib.fa_paged_decode.restype = i
        lib.fa_status_str.argtypes = [i]
        lib.fa_status_str.restype = ctypes.c_char_p
        lib.fa_version.argtypes = []
        lib.fa_version.restype = i
        _lib = lib
        return lib


def status_str(status: int) -> str:
    return load().fa_status_str(int(status)).decode()


def check(status: int, what: str) -> None:
    if status != FA_OK:
        raise FaError(status, "%s: %s" % (what, status_str(status)))

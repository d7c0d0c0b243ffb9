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
    4: "FA_ERR_WORKSPACE", 5: "FA_ERR_HIP", 6: "FA_ERR_NO_PAGES", 7: "FA_ERR_STATE",
    8: "FA_ERR_SCRATCH_LIMIT",
}
# every symbol include/fa.h declares
EXPORTS = ("fa_fwd", "fa_fwd_f32", "fa_fwd_fp8", "fa_quantize_fp8", "fa_quantize_fp8_qkv",
           "fa_fwd_block_sparse", "fa_bwd_workspace_bytes", "fa_bwd",
           "fa_paged_decode_workspace_bytes", "fa_paged_decode", "fa_noalloc_scratch_bytes",
           "fa_paged_decode_noalloc", "fa_paged_prefill",
           "fa_bm_state_bytes", "fa_bm_init",
           "fa_bm_add_seq", "fa_bm_fork", "fa_bm_append_token", "fa_bm_free_seq",
           "fa_bm_num_free_pages", "fa_bm_seq_len", "fa_bm_page_refcount", "fa_bm_block_table",
           "fa_copy_pages", "fa_check_paged_tables", "fa_read_probe", "fa_status_str", "fa_version")


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
        lib.fa_noalloc_scratch_bytes.argtypes = []
        lib.fa_noalloc_scratch_bytes.restype = sz
        lib.fa_paged_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
        lib.fa_paged_decode_noalloc.restype = i
        lib.fa_quantize_fp8.argtypes = [vp, vp, vp, vp, i, i, i, i, vp]
        lib.fa_quantize_fp8.restype = i
        lib.fa_quantize_fp8_qkv.argtypes = [vp] * 10 + [i, i, i, i, vp]
        lib.fa_quantize_fp8_qkv.restype = i
        lib.fa_fwd_block_sparse.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, f, ctypes.c_uint64, vp]
        lib.fa_fwd_block_sparse.restype = i
        lib.fa_paged_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
        lib.fa_paged_prefill.restype = i
        ip = ctypes.POINTER(ctypes.c_int32)
        lib.fa_bm_state_bytes.argtypes = [i, i, i]
        lib.fa_bm_state_bytes.restype = sz
        lib.fa_bm_init.argtypes = [vp, sz, i, i, i, i]
        lib.fa_bm_init.restype = i
        lib.fa_bm_add_seq.argtypes = [vp, i, i]
        lib.fa_bm_add_seq.restype = i
        lib.fa_bm_fork.argtypes = [vp, i, i]
        lib.fa_bm_fork.restype = i
        lib.fa_bm_append_token.argtypes = [vp, i, ip, ip]
        lib.fa_bm_append_token.restype = i
        lib.fa_bm_free_seq.argtypes = [vp, i]
        lib.fa_bm_free_seq.restype = i
        lib.fa_bm_num_free_pages.argtypes = [vp]
        lib.fa_bm_num_free_pages.restype = i
        lib.fa_bm_seq_len.argtypes = [vp, i]
        lib.fa_bm_seq_len.restype = i
        lib.fa_bm_page_refcount.argtypes = [vp, i]
        lib.fa_bm_page_refcount.restype = i
        lib.fa_bm_block_table.argtypes = [vp, vp, vp]
        lib.fa_bm_block_table.restype = i
        lib.fa_copy_pages.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp]
        lib.fa_copy_pages.restype = i
        lib.fa_check_paged_tables.argtypes = [vp, vp, i, i, i, i, vp, vp]
        lib.fa_check_paged_tables.restype = i
        lib.fa_read_probe.argtypes = [vp, ctypes.c_size_t, vp, vp]
        lib.fa_read_probe.restype = i
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

"""ctypes loader for libsrt.so: argument types of every C-ABI entry point.

Loading needs no GPU (the HIP runtime initialises lazily).  If the library is
missing the import of the binding fails loudly; there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# always the in-tree build next to this file: no environment override, so
# what the tests and the benchmark load is what build.py produced
LIB_PATH = os.path.join(HERE, "libsrt.so")

c_int, c_ll, c_double, c_float, c_void_p, c_size_t = C.c_int, C.c_longlong, C.c_double, C.c_float, C.c_void_p, C.c_size_t
c_char_p = C.c_char_p

# name -> argtypes (every function returns int status, except the three string/version helpers)
SIGNATURES = {
    "srt_abi_version": [],
    "srt_status_string": [c_int],
    "srt_last_error": [],
    "srt_rope_inv_freq": [c_int, c_double, c_double, c_double, c_double, c_double, c_int,
                          C.POINTER(c_double), C.POINTER(c_double), C.POINTER(C.c_byte)],
    "srt_rope_inv_freq_dynamic_ntk": [c_double, c_ll, c_double, c_int, C.POINTER(c_double), C.POINTER(c_double)],
    "srt_rope_inv_freq_factors": [c_double, C.POINTER(c_double), c_int, C.POINTER(c_double)],
    "srt_rope_cos_sin": [C.POINTER(c_double), c_int, c_double, c_ll, c_void_p, c_void_p],
    "srt_rope_apply": [c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int, c_ll, c_void_p, c_ll, c_int,
                       c_void_p],
    "srt_attn_prefill": [c_void_p, c_void_p, c_void_p, c_int,
                         c_int, c_int, c_int, c_int, c_int, c_int,
                         c_ll, c_ll, c_ll, c_ll, c_int, c_int, c_int, c_float,
                         c_void_p, c_ll, c_int,
                         c_void_p, c_int, c_ll, c_void_p, c_ll, c_void_p, c_void_p],
    "srt_attn_merge_states": [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_ll,
                              c_void_p, c_int, c_ll, c_void_p, c_ll,
                              c_int, c_int, c_int, c_int, c_void_p],
    "srt_attn_decode_workspace_size": [c_int, c_int, c_int, c_int, C.POINTER(c_size_t)],
    "srt_attn_decode_splitk": [c_void_p, c_void_p, c_void_p, c_int,
                               c_int, c_int, c_int, c_int, c_int, c_void_p,
                               c_int, c_float, c_void_p, c_ll, c_int, c_int, c_int,
                               c_void_p, c_size_t, c_void_p, c_void_p, c_void_p],
    "srt_attn_decode_splitk_noalloc": [c_void_p, c_void_p, c_void_p, c_int,
                                       c_int, c_int, c_int, c_int, c_int, c_void_p,
                                       c_int, c_float, c_void_p, c_ll, c_int, c_int, c_int,
                                       c_void_p, c_void_p, c_void_p],
    "srt_attn_decode_noalloc_max_workspace": [],
    "srt_attn_backward_workspace_size": [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                         C.POINTER(c_size_t)],
    "srt_attn_backward": [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int,
                          c_int, c_int, c_int, c_int, c_int, c_int,
                          c_ll, c_ll, c_int, c_int, c_int, c_float,
                          c_void_p, c_ll, c_int, c_void_p, c_size_t,
                          c_void_p, c_void_p, c_void_p, c_void_p],
    "srt_attn_ring_workspace_size": [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                     C.POINTER(c_size_t)],
    "srt_attn_ring_prefill": [c_void_p, c_void_p, c_void_p, c_int,
                              c_int, c_int, c_int, c_int, c_int,
                              c_int, c_int, c_int, c_int, c_int, c_float,
                              c_void_p, c_ll, c_int,
                              c_void_p, c_size_t, c_void_p, c_void_p, c_void_p],
}

_lib = None
ABI_VERSION = 2          # srt_abi_version() of the library these signatures describe


def load(path: str = LIB_PATH):
    """Load libsrt.so once and declare the argument types of its exports."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libsrt.so not built at {path}: run `python scaled_rope_tiled_amd/build.py`")
    lib = C.CDLL(path)
    lib.srt_abi_version.restype = c_int
    if lib.srt_abi_version() != ABI_VERSION:
        raise ImportError(f"{path} implements ABI {lib.srt_abi_version()}, this binding ABI {ABI_VERSION}: rebuild it")
    for name, args in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = (c_char_p if name in ("srt_status_string", "srt_last_error")
                      else c_size_t if name == "srt_attn_decode_noalloc_max_workspace" else c_int)
    _lib = lib
    return lib


class SrtError(RuntimeError):
    def __init__(self, status: int, fn: str):
        lib = load()
        msg = lib.srt_last_error().decode() or lib.srt_status_string(status).decode()
        super().__init__(f"{fn}: {lib.srt_status_string(status).decode()} ({status}): {msg}")
        self.status = status


def check(status: int, fn: str) -> None:
    if status != 0:
        raise SrtError(status, fn)

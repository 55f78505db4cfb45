"""ctypes loader for libpagedkv.so (built in-tree by paged_kv_cache_40_amd.build).

There is no fallback: if the library is missing or does not load, every entry
point raises.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedkv.so")

PA_F32, PA_F16 = 0, 1
PA_OK = 0
PA_SWAP_OUT, PA_SWAP_IN = 0, 1
PA_DECODE_SHARED_BLOCKS = 1
PA_DECODE_GROUP_SHIFT = 8  # group size g of the grouped decode in flag bits 8..11
PA_CHECK_OK = 0xFFFFFFFFFFFFFFFF
PA_NOALLOC_WORKSPACE_BYTES = 256 << 20  # the device array behind pa_decode_noalloc
# pa_check_kind values
CHECK_KINDS = {1: "START_LOC", 2: "QUERY_COUNT", 3: "CONTEXT_LEN", 4: "BLOCK_ID",
               5: "SLOT_REUSED", 6: "PAIR_ID", 7: "DEST_REUSED", 8: "DEST_IS_SOURCE"}

_c_int, _c_i32, _c_i64, _c_size = ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_vp = ctypes.c_void_p

# name -> (restype, argtypes); mirrors include/pa.h
SIGNATURES = {
    "pa_write_kv": (_c_int, [_vp, _vp, _c_i64, _vp, _vp, _vp, _c_i32, _vp, _vp, _c_i32, _c_i32,
                             _c_i32, _c_i32, _c_i32, _c_i32, _vp]),
    "pa_decode_workspace_bytes": (_c_size, [_c_i32, _c_i32, _c_i32, _c_i32]),
    "pa_decode": (_c_int, [_vp, _vp, _vp, _vp, _c_i64, _vp, _c_i32, _vp, _vp, _c_i32, _c_i32,
                           _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _c_size, _vp]),
    "pa_decode_ext": (_c_int, [_vp, _vp, _vp, _vp, _c_i64, _vp, _c_i32, _vp, _vp, _c_i32, _c_i32,
                               _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _c_size, _c_i32,
                               _vp, ctypes.c_uint32, _vp]),
    "pa_decode_noalloc": (_c_int, [_vp, _vp, _vp, _vp, _c_i64, _vp, _c_i32, _vp, _vp, _c_i32,
                                   _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                   _vp, ctypes.c_uint32, _vp]),
    "pa_copy_blocks": (_c_int, [_vp, _vp, _c_i64, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                _vp]),
    "pa_swap_blocks": (_c_int, [_vp, _vp, _c_i64, _vp, _vp, _c_i64, _vp, _c_i32, _c_i32, _c_i32,
                                _c_i32, _c_i32, _c_i32, _vp]),
    "pa_check_workspace_bytes": (_c_size, [_c_i64]),
    "pa_check_attention": (_c_int, [_vp, _c_i64, _vp, _c_i32, _vp, _vp, _c_i32, _c_i32, _c_i32,
                                    _c_i32, _c_i32, _c_i32, _vp]),
    "pa_check_write": (_c_int, [_vp, _vp, _c_size, _c_i64, _vp, _c_i32, _vp, _vp, _c_i32, _c_i32,
                                _c_i32, _vp]),
    "pa_check_pairs": (_c_int, [_vp, _vp, _c_size, _c_i64, _c_i64, _vp, _c_i32, _c_i32, _vp]),
    "pa_strerror": (ctypes.c_char_p, [_c_int]),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library once and attach the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -m paged_kv_cache_40_amd.build` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load().pa_strerror(int(status)).decode()


def check(status: int, what: str) -> None:
    if status != PA_OK:
        raise RuntimeError(f"{what}: {strerror(status)} (status {status})")

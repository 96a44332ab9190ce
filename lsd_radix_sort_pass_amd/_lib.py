"""ctypes loader for librs.so (the C ABI declared in include/rs.h and
include/rs_prof.h).  Fails loudly when the library has not been built: there
is no fallback path."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librs.so")

RS_SUCCESS = 0
RS_ERROR_INVALID_VALUE = 1
RS_ERROR_INSUFFICIENT_TEMP = 2
RS_ERROR_LAUNCH = 3
RS_ERROR_SCRATCH_LIMIT = 4

RS_KERNEL_FILL = 0
RS_KERNEL_HIST = 1
RS_KERNEL_SCAN = 2
RS_KERNEL_PASS = 3
RS_KERNEL_COPY = 4
RS_KERNEL_SMALL = 5
RS_KERNEL_KINDS = 6

# Every function the two public headers declare, with its ctypes signature.
_VP = ctypes.c_void_p
_SZ = ctypes.c_size_t
_I = ctypes.c_int
_FP = ctypes.POINTER(ctypes.c_float)
SIGNATURES = {
    "rs_temp_bytes": (_SZ, [_SZ, _I, _I, _I]),
    "rs_sort_keys_u32": (_I, [_VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_sort_keys_i32": (_I, [_VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_sort_keys_f32": (_I, [_VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_sort_pairs_u32": (_I, [_VP, _VP, _VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_sort_pairs_i32": (_I, [_VP, _VP, _VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_sort_pairs_f32": (_I, [_VP, _VP, _VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_temp_bytes64": (_SZ, [_SZ, _I, _I, _I]),
    "rs_sort_keys_u64": (_I, [_VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_sort_keys_i64": (_I, [_VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_sort_keys_f64": (_I, [_VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_sort_pairs_u64": (_I, [_VP, _VP, _VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_sort_pairs_i64": (_I, [_VP, _VP, _VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_sort_pairs_f64": (_I, [_VP, _VP, _VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_temp_bytes_ex": (_SZ, [_SZ, _I, _I, _I, _I]),
    "rs_sort_keys_u16": (_I, [_VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_sort_keys_i16": (_I, [_VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_sort_keys_f16": (_I, [_VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_sort_pairs_u16": (_I, [_VP, _VP, _VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_sort_pairs_i16": (_I, [_VP, _VP, _VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_sort_pairs_f16": (_I, [_VP, _VP, _VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_sort_pairs_u16_v64": (_I, [_VP, _VP, _VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_sort_pairs_i16_v64": (_I, [_VP, _VP, _VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_sort_pairs_f16_v64": (_I, [_VP, _VP, _VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_sort_pairs_u32_v64": (_I, [_VP, _VP, _VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_sort_pairs_i32_v64": (_I, [_VP, _VP, _VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_sort_pairs_f32_v64": (_I, [_VP, _VP, _VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_sort_pairs_u64_v64": (_I, [_VP, _VP, _VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_sort_pairs_i64_v64": (_I, [_VP, _VP, _VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_sort_pairs_f64_v64": (_I, [_VP, _VP, _VP, _VP, _SZ, _I, _I, _VP, _SZ, _VP]),
    "rs_temp_bytes_morton30": (_SZ, [_SZ]),
    "rs_sort_morton30": (_I, [_VP, _SZ, _FP, _FP, _VP, _VP, _VP, _SZ, _VP]),
    "rs_sort_keys_u32_noalloc": (_I, [_VP, _VP, _SZ, _I, _I, _VP]),
    "rs_status_string": (ctypes.c_char_p, [_I]),
    "rs_prof_enable": (_I, [_I]),
    "rs_prof_reset": (None, []),
    "rs_prof_summary": (_I, [_I, ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_double)]),
    "rs_copy_u32": (_I, [_VP, _VP, _SZ, _VP]),
    "rs_prof_small_path": (_I, [_I]),
    "rs_prof_header_offset": (ctypes.c_size_t, [_I]),
    "rs_prof_tile_items": (_I, [_I]),
    "rs_prof_samples": (_SZ, [_I, _I, ctypes.POINTER(ctypes.c_double), _SZ]),
    "rs_prof_force_giveup": (_I, [_I]),
    "rs_prof_ranker": (_I, [_I]),
    "rs_prof_lds_rank_probe": (_I, [_VP, _VP, _I, _I, _I, _VP]),
}

_lib = None


class LibraryNotBuilt(RuntimeError):
    pass


def load():
    """Load librs.so (once).  Raises LibraryNotBuilt if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryNotBuilt(
            f"{LIB_PATH} not found: build it with `python -m lsd_radix_sort_pass_amd.build` "
            "(or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().rs_status_string(code).decode()

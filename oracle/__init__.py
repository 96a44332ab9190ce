"""CPU oracle for the stable LSD radix sort -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the GPU library and
its Python binding) never imports, links or calls it, and the two share no
code: the only thing both sides use is the seeded input generator module,
which holds none of the sort's arithmetic.

The arithmetic lives in ``oracle.cpp`` (plain C++17, built with g++); this
module is ctypes marshalling around it plus the build step.  Page citations
are in ``oracle.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")

KEY_U32 = 0
KEY_I32 = 1
KEY_F32 = 2
KEY_U64 = 3
KEY_I64 = 4
KEY_F64 = 5
KEY_U16 = 6
KEY_I16 = 7
KEY_F16 = 8

_KIND_OF_DTYPE = {
    np.dtype(np.uint32): KEY_U32,
    np.dtype(np.int32): KEY_I32,
    np.dtype(np.float32): KEY_F32,
    np.dtype(np.uint64): KEY_U64,
    np.dtype(np.int64): KEY_I64,
    np.dtype(np.float64): KEY_F64,
    np.dtype(np.uint16): KEY_U16,
    np.dtype(np.int16): KEY_I16,
    np.dtype(np.float16): KEY_F16,
}

_lib = None


def build() -> str:
    """Compile liboracle.so with g++ (always recompiles)."""
    cmd = [
        "g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-Wall", "-Wextra",
        "-o", _LIB + ".tmp", _SRC,
    ]
    subprocess.run(cmd, check=True, cwd=_HERE)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    u32p = ctypes.POINTER(ctypes.c_uint32)
    lib.oracle_ordered_key.argtypes = [ctypes.c_int, ctypes.c_uint32]
    lib.oracle_ordered_key.restype = ctypes.c_uint32
    lib.oracle_lsd_sort.argtypes = [ctypes.c_int, u32p, u32p, ctypes.c_size_t,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, u32p, u32p]
    lib.oracle_lsd_sort.restype = ctypes.c_int
    lib.oracle_split_sort.argtypes = [ctypes.c_int, u32p, u32p, ctypes.c_size_t,
                                      ctypes.c_int, ctypes.c_int, u32p, u32p]
    lib.oracle_split_sort.restype = ctypes.c_int
    lib.oracle_decimal_pass.argtypes = [u32p, ctypes.c_size_t, ctypes.c_int, u32p]
    lib.oracle_decimal_pass.restype = ctypes.c_int
    u64p = ctypes.POINTER(ctypes.c_uint64)
    lib.oracle_ordered_key64.argtypes = [ctypes.c_int, ctypes.c_uint64]
    lib.oracle_ordered_key64.restype = ctypes.c_uint64
    lib.oracle_lsd_sort64.argtypes = [ctypes.c_int, u64p, u32p, ctypes.c_size_t,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, u64p, u32p]
    lib.oracle_lsd_sort64.restype = ctypes.c_int
    lib.oracle_split_sort64.argtypes = [ctypes.c_int, u64p, u32p, ctypes.c_size_t,
                                        ctypes.c_int, ctypes.c_int, u64p, u32p]
    lib.oracle_split_sort64.restype = ctypes.c_int
    vp = ctypes.c_void_p
    lib.oracle_ordered_key_any.argtypes = [ctypes.c_int, ctypes.c_uint64]
    lib.oracle_ordered_key_any.restype = ctypes.c_uint64
    lib.oracle_lsd_sort_any.argtypes = [ctypes.c_int, vp, vp, ctypes.c_int, ctypes.c_size_t,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp]
    lib.oracle_lsd_sort_any.restype = ctypes.c_int
    lib.oracle_split_sort_any.argtypes = [ctypes.c_int, vp, vp, ctypes.c_int, ctypes.c_size_t,
                                          ctypes.c_int, ctypes.c_int, vp, vp]
    lib.oracle_split_sort_any.restype = ctypes.c_int
    fp = ctypes.POINTER(ctypes.c_float)
    lib.oracle_morton_scale.argtypes = [ctypes.c_float, ctypes.c_float]
    lib.oracle_morton_scale.restype = ctypes.c_float
    lib.oracle_morton30.argtypes = [fp, ctypes.c_size_t, fp, fp, u32p]
    lib.oracle_morton30.restype = ctypes.c_int
    _lib = lib
    return lib


def _u32_view(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype.itemsize != 4:
        raise TypeError(f"expected a 32-bit array, got {a.dtype}")
    return a.view(np.uint32)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32))


def kind_of(dtype) -> int:
    return _KIND_OF_DTYPE[np.dtype(dtype)]


def ordered_key(kind: int, bits: int) -> int:
    """Order-preserving unsigned key of one 32-bit (kinds 0-2), 64-bit
    (kinds 3-5) or 16-bit (kinds 6-8) pattern."""
    if kind >= KEY_U16:
        return int(_load().oracle_ordered_key_any(kind, bits & 0xFFFF))
    if kind >= KEY_U64:
        return int(_load().oracle_ordered_key64(kind, bits & 0xFFFFFFFFFFFFFFFF))
    return int(_load().oracle_ordered_key(kind, bits & 0xFFFFFFFF))


def _run_sort_any(fn_name, keys, values, begin_bit, end_bit, extra):
    """Any key width (16/32/64) with no, 32-bit or 64-bit values."""
    kind = kind_of(keys.dtype)
    n = keys.size
    kout = np.empty_like(keys)
    vin = vout = None
    val_bytes = 0
    if values is not None:
        vin = np.ascontiguousarray(values)
        if vin.size != n or vin.dtype.itemsize not in (4, 8):
            raise ValueError("values must be n 4- or 8-byte elements")
        val_bytes = vin.dtype.itemsize
        vout = np.empty_like(vin)
    p = lambda a: None if a is None else ctypes.c_void_p(a.ctypes.data)
    rc = getattr(_load(), fn_name)(kind, p(keys), p(vin), val_bytes, n, begin_bit, end_bit, *extra, p(kout), p(vout))
    if rc != 0:
        raise ValueError(f"{fn_name} failed with code {rc}")
    return kout if values is None else (kout, vout)


def _run_sort(fn_name, keys, values, begin_bit, end_bit, extra):
    keys = np.ascontiguousarray(keys)
    if keys.dtype.itemsize == 2 or (values is not None and np.asarray(values).dtype.itemsize == 8):
        return _run_sort_any(fn_name + "_any", keys, values, begin_bit, end_bit, extra)
    kind = kind_of(keys.dtype)
    wide = keys.dtype.itemsize == 8
    if wide:
        fn_name += "64"
        kin = keys.view(np.uint64)
        kptr = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))
    else:
        kin = _u32_view(keys)
        kptr = _ptr
    n = kin.size
    kout = np.empty(n, dtype=kin.dtype)
    vin = vout = None
    if values is not None:
        vin = _u32_view(values)
        if vin.size != n:
            raise ValueError("keys and values differ in length")
        vout = np.empty(n, dtype=np.uint32)
    fn = getattr(_load(), fn_name)
    rc = fn(kind, kptr(kin), _ptr(vin), n, begin_bit, end_bit, *extra, kptr(kout), _ptr(vout))
    if rc != 0:
        raise ValueError(f"{fn_name} failed with code {rc}")
    kout = kout.view(keys.dtype)
    if values is not None:
        vout = vout.view(np.asarray(values).dtype)
        return kout, vout
    return kout


def _key_bits(keys) -> int:
    return 8 * np.asarray(keys).dtype.itemsize


def lsd_sort(keys, values=None, begin_bit=0, end_bit=None, radix_bits=8):
    """Stable LSD radix sort (counting-sort passes).  Returns sorted keys, or
    (keys, values) when values are given.  Keys: uint16/int16/float16,
    uint32/int32/float32 or uint64/int64/float64 (end_bit defaults to the key
    width); values: any 4- or 8-byte dtype.  The original bit patterns are
    returned, permuted."""
    if end_bit is None:
        end_bit = _key_bits(keys)
    return _run_sort("oracle_lsd_sort", keys, values, begin_bit, end_bit, (radix_bits,))


def split_sort(keys, values=None, begin_bit=0, end_bit=None):
    """Same result via one-bit two-bucket splits (independent algorithm)."""
    if end_bit is None:
        end_bit = _key_bits(keys)
    return _run_sort("oracle_split_sort", keys, values, begin_bit, end_bit, ())


def decimal_pass(values, place: int) -> np.ndarray:
    """One stable pass on decimal digit (x // 10**place) % 10."""
    vin = np.ascontiguousarray(values, dtype=np.uint32)
    out = np.empty_like(vin)
    rc = _load().oracle_decimal_pass(_ptr(vin), vin.size, place, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_decimal_pass failed with code {rc}")
    return out


def morton30(points, lo=(0.0, 0.0, 0.0), hi=(1.0, 1.0, 1.0)) -> np.ndarray:
    """30-bit Morton codes (uint32) of an (n, 3) float32 array of points over
    the box [lo, hi); see oracle_morton30 in oracle.h for the definition."""
    pts = np.ascontiguousarray(points, dtype=np.float32)
    if pts.ndim != 2 or pts.shape[1] != 3:
        raise ValueError("points must have shape (n, 3)")
    lo_a = np.ascontiguousarray(lo, dtype=np.float32)
    hi_a = np.ascontiguousarray(hi, dtype=np.float32)
    codes = np.empty(pts.shape[0], dtype=np.uint32)
    fp = ctypes.POINTER(ctypes.c_float)
    rc = _load().oracle_morton30(pts.ctypes.data_as(fp), pts.shape[0], lo_a.ctypes.data_as(fp),
                                 hi_a.ctypes.data_as(fp), _ptr(codes))
    if rc != 0:
        raise ValueError(f"oracle_morton30 failed with code {rc}")
    return codes


def std_sort(keys, stable: bool = False) -> np.ndarray:
    """CPU context (not a reference): std::sort / std::stable_sort of a copy
    of uint32 or int32 keys in their native order."""
    a = np.array(keys, copy=True)
    if a.dtype not in (np.dtype(np.uint32), np.dtype(np.int32)):
        raise TypeError("std_sort takes uint32 or int32 keys")
    lib = _load()
    lib.oracle_std_sort.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    lib.oracle_std_sort.restype = ctypes.c_int
    rc = lib.oracle_std_sort(kind_of(a.dtype), a.ctypes.data, a.size, 1 if stable else 0)
    if rc != 0:
        raise ValueError(f"oracle_std_sort failed with code {rc}")
    return a


def morton_scale(lo: float, hi: float) -> float:
    """The float32 quantisation scale 1024 / (hi - lo)."""
    return float(_load().oracle_morton_scale(lo, hi))

"""MI355X (gfx950) stable LSD radix sort -- Python binding.

Thin marshalling layer over the C ABI in include/rs.h: every step of the sort
runs in the HIP kernels of librs.so.  PyTorch is used only for device memory
(tensors) and streams.

    import torch, lsd_radix_sort_pass_amd as rs
    k = torch.randint(0, 2**31, (1 << 20,), dtype=torch.int32, device="cuda")
    s = rs.sort_keys(k)                              # int32 ascending, stable
    ks, vs = rs.sort_pairs(k.view(torch.uint32), torch.arange(k.numel(),
                           device="cuda", dtype=torch.int32))

Key dtypes: torch.uint16/int16/float16, torch.uint32/int32/float32 and
torch.uint64/int64/float64 (the float order puts every NaN and both
infinities last, -0.0 before +0.0).  Pairs: any of those key dtypes with a
32- or 64-bit value dtype.  begin_bit/end_bit select a bit range of the
order-preserving key (end_bit defaults to the key width).
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib

__all__ = [
    "RadixSortError", "key_bits", "temp_bytes", "temp_bytes_morton30", "sort_morton30", "alloc_temp", "sort_keys", "sort_pairs",
    "copy_u32", "prof_enable", "prof_reset", "prof_summary", "prof_small_path", "library_path",
    "error_word", "skipped_passes", "order_flag", "prof_tile_items", "sort_keys_u32_noalloc",
    "NOALLOC_MAX_KEYS", "DeviceGuardError", "prof_samples", "prof_force_giveup", "lds_rank_probe", "prof_ranker",
]

TEMP_ALIGN = 256

_KEYS_FN = {
    torch.uint16: "rs_sort_keys_u16",
    torch.int16: "rs_sort_keys_i16",
    torch.float16: "rs_sort_keys_f16",
    torch.uint32: "rs_sort_keys_u32",
    torch.int32: "rs_sort_keys_i32",
    torch.float32: "rs_sort_keys_f32",
    torch.uint64: "rs_sort_keys_u64",
    torch.int64: "rs_sort_keys_i64",
    torch.float64: "rs_sort_keys_f64",
}
_PAIRS_FN = {
    torch.uint16: "rs_sort_pairs_u16",
    torch.int16: "rs_sort_pairs_i16",
    torch.float16: "rs_sort_pairs_f16",
    torch.uint32: "rs_sort_pairs_u32",
    torch.int32: "rs_sort_pairs_i32",
    torch.float32: "rs_sort_pairs_f32",
    torch.uint64: "rs_sort_pairs_u64",
    torch.int64: "rs_sort_pairs_i64",
    torch.float64: "rs_sort_pairs_f64",
}

_WORD_DTYPES = (torch.uint32, torch.int32, torch.float32)
_DWORD_DTYPES = (torch.uint64, torch.int64, torch.float64)
_VALUE_DTYPES = _WORD_DTYPES + _DWORD_DTYPES
_KEY_DTYPES = tuple(_KEYS_FN)


def key_bits(dtype: torch.dtype) -> int:
    """Width in bits of a supported key dtype."""
    if dtype not in _KEYS_FN:
        raise TypeError(f"unsupported key dtype {dtype}")
    if dtype in _DWORD_DTYPES:
        return 64
    return 16 if dtype in (torch.uint16, torch.int16, torch.float16) else 32


class RadixSortError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {_lib.status_string(code)} (rs_status {code})")


class DeviceGuardError(RuntimeError):
    """A sort's bounded device-side wait gave up (the error word in temp is
    non-zero): its output is invalid."""

    def __init__(self, word: int, where: str):
        self.word = word
        super().__init__(f"{where}: a device-side wait gave up (error word {word:#x}); the output is invalid")


def _check_guard(temp: torch.Tensor, device, stream, where: str) -> None:
    s = torch.cuda.current_stream(device) if stream is None else stream
    s.synchronize()
    word = int(temp[:4].view(torch.int32).item())
    if word != 0:
        raise DeviceGuardError(word, where)


def library_path() -> str:
    return _lib.LIB_PATH


def temp_bytes(n: int, with_values: bool = False, begin_bit: int = 0, end_bit: Optional[int] = None,
               key_dtype: torch.dtype = torch.uint32, value_bytes: int = 4) -> int:
    """Temp bytes of a sort of n keys of key_dtype (with values of
    value_bytes bytes, 4 or 8, if with_values)."""
    kb = key_bits(key_dtype)
    end_bit = kb if end_bit is None else end_bit
    return int(_lib.load().rs_temp_bytes_ex(n, kb // 8, value_bytes if with_values else 0, begin_bit, end_bit))


def alloc_temp(n: int, with_values: bool = False, begin_bit: int = 0, end_bit: Optional[int] = None,
               device=None, key_dtype: torch.dtype = torch.uint32, value_bytes: int = 4) -> torch.Tensor:
    """A uint8 device tensor large enough (and 256-byte aligned) for a sort."""
    nbytes = temp_bytes(n, with_values, begin_bit, end_bit, key_dtype, value_bytes)
    t = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    if t.data_ptr() % TEMP_ALIGN:
        raise RuntimeError("device allocator returned a temp buffer that is not 256-byte aligned")
    return t


def _check_words(t: torch.Tensor, name: str, dtypes=_WORD_DTYPES) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if t.dtype not in dtypes:
        names = ", ".join(str(d).replace("torch.", "") for d in dtypes)
        raise TypeError(f"{name} must be one of {names} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_handle(device, stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _temp_for(n, with_values, begin_bit, end_bit, device, temp, key_dtype, value_bytes=4):
    if temp is None:
        return alloc_temp(n, with_values, begin_bit, end_bit, device, key_dtype, value_bytes)
    if temp.device != device:
        raise ValueError("temp must be on the same device as the keys")
    return temp


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _temp_args(temp: torch.Tensor):
    nbytes = temp.numel() * temp.element_size()
    return ctypes.c_void_p(temp.data_ptr()), nbytes


def sort_keys(keys: torch.Tensor, begin_bit: int = 0, end_bit: Optional[int] = None,
              out: Optional[torch.Tensor] = None, temp: Optional[torch.Tensor] = None,
              stream: Optional[torch.cuda.Stream] = None, check: bool = False) -> torch.Tensor:
    """Stable ascending sort of a 1-D device tensor of 16-, 32- or 64-bit keys.

    Returns `out` (allocated if None; pass `out=keys` to sort in place).
    check=True waits for the stream and raises DeviceGuardError if a
    device-side wait of the sort gave up (the output is then invalid)."""
    _check_words(keys, "keys", _KEY_DTYPES)
    n = keys.numel()
    end_bit = key_bits(keys.dtype) if end_bit is None else end_bit
    if out is None:
        out = torch.empty_like(keys)
    else:
        _check_words(out, "out", _KEY_DTYPES)
        if out.dtype != keys.dtype or out.numel() != n or out.device != keys.device:
            raise ValueError("out must match keys in dtype, size and device")
    temp = _temp_for(n, False, begin_bit, end_bit, keys.device, temp, keys.dtype)
    tptr, tbytes = _temp_args(temp)
    fn = getattr(_lib.load(), _KEYS_FN[keys.dtype])
    code = fn(_ptr(keys), _ptr(out), n, begin_bit, end_bit, tptr, tbytes,
              _stream_handle(keys.device, stream))
    if code != _lib.RS_SUCCESS:
        raise RadixSortError(code, _KEYS_FN[keys.dtype])
    if check and n > 1 and begin_bit != end_bit:
        _check_guard(temp, keys.device, stream, _KEYS_FN[keys.dtype])
    return out


NOALLOC_MAX_KEYS = 1 << 22      # RS_NOALLOC_MAX_KEYS in include/rs.h


def sort_keys_u32_noalloc(keys: torch.Tensor, begin_bit: int = 0, end_bit: int = 32,
                          out: torch.Tensor = None, stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """rs_sort_keys_u32_noalloc: the uint32 keys-only sort with the library's
    fixed per-device scratch instead of a temp buffer (at most
    NOALLOC_MAX_KEYS keys).  The C call allocates nothing; pass `out` to
    keep this wrapper from allocating the result.  Calls that overlap on one
    GPU race on the shared scratch."""
    _check_words(keys, "keys", (torch.uint32,))
    n = keys.numel()
    if out is None:
        out = torch.empty_like(keys)
    else:
        _check_words(out, "out", (torch.uint32,))
        if out.numel() != n or out.device != keys.device:
            raise ValueError("out must match keys in size and device")
    code = _lib.load().rs_sort_keys_u32_noalloc(_ptr(keys), _ptr(out), n, begin_bit, end_bit,
                                                _stream_handle(keys.device, stream))
    if code != _lib.RS_SUCCESS:
        raise RadixSortError(code, "rs_sort_keys_u32_noalloc")
    return out


def sort_pairs(keys: torch.Tensor, values: torch.Tensor, begin_bit: int = 0,
               end_bit: Optional[int] = None,
               keys_out: Optional[torch.Tensor] = None, values_out: Optional[torch.Tensor] = None,
               temp: Optional[torch.Tensor] = None,
               stream: Optional[torch.cuda.Stream] = None,
               check: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """Stable ascending sort of 16-, 32- or 64-bit keys (uint, int or
    float) carrying 32- or 64-bit values (any 4- or 8-byte dtype of
    uint/int/float).  check=True as for sort_keys."""
    _check_words(keys, "keys", _KEY_DTYPES)
    _check_words(values, "values", _VALUE_DTYPES)
    n = keys.numel()
    end_bit = key_bits(keys.dtype) if end_bit is None else end_bit
    if values.numel() != n or values.device != keys.device:
        raise ValueError("values must match keys in size and device")
    keys_out = torch.empty_like(keys) if keys_out is None else keys_out
    values_out = torch.empty_like(values) if values_out is None else values_out
    _check_words(keys_out, "keys_out", _KEY_DTYPES)
    _check_words(values_out, "values_out", _VALUE_DTYPES)
    if keys_out.dtype != keys.dtype or keys_out.numel() != n or values_out.numel() != n:
        raise ValueError("outputs must match the inputs in dtype and size")
    if values_out.element_size() != values.element_size():
        raise ValueError("values_out must have the values' element size")
    vb = values.element_size()
    temp = _temp_for(n, True, begin_bit, end_bit, keys.device, temp, keys.dtype, vb)
    tptr, tbytes = _temp_args(temp)
    name = _PAIRS_FN[keys.dtype] + ("_v64" if vb == 8 else "")
    code = getattr(_lib.load(), name)(_ptr(keys), _ptr(keys_out), _ptr(values), _ptr(values_out),
                                      n, begin_bit, end_bit, tptr, tbytes,
                                      _stream_handle(keys.device, stream))
    if code != _lib.RS_SUCCESS:
        raise RadixSortError(code, name)
    if check and n > 1 and begin_bit != end_bit:
        _check_guard(temp, keys.device, stream, name)
    return keys_out, values_out


def temp_bytes_morton30(n: int) -> int:
    return int(_lib.load().rs_temp_bytes_morton30(n))


def sort_morton30(points: torch.Tensor, box_lo=(0.0, 0.0, 0.0), box_hi=(1.0, 1.0, 1.0),
                  codes_out: Optional[torch.Tensor] = None, index_out: Optional[torch.Tensor] = None,
                  temp: Optional[torch.Tensor] = None,
                  stream: Optional[torch.cuda.Stream] = None,
                  check: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """30-bit Morton codes of an (n, 3) float32 device tensor of points over
    the box [box_lo, box_hi), sorted, with the index of each code's point
    (stable).  Returns (codes uint32, index uint32).  check=True as for
    sort_keys."""
    if not isinstance(points, torch.Tensor) or points.device.type != "cuda":
        raise ValueError("points must be a device tensor")
    if points.dtype != torch.float32 or points.dim() != 2 or points.shape[1] != 3 or not points.is_contiguous():
        raise ValueError("points must be a contiguous (n, 3) float32 tensor")
    n = points.shape[0]
    codes_out = torch.empty(n, dtype=torch.uint32, device=points.device) if codes_out is None else codes_out
    index_out = torch.empty(n, dtype=torch.uint32, device=points.device) if index_out is None else index_out
    _check_words(codes_out, "codes_out")
    _check_words(index_out, "index_out")
    if codes_out.numel() != n or index_out.numel() != n:
        raise ValueError("outputs must hold n elements")
    if temp is None:
        temp = torch.empty(max(temp_bytes_morton30(n), 1), dtype=torch.uint8, device=points.device)
        if temp.data_ptr() % TEMP_ALIGN:
            raise RuntimeError("device allocator returned a temp buffer that is not 256-byte aligned")
    tptr, tbytes = _temp_args(temp)
    lo = (ctypes.c_float * 3)(*[float(v) for v in box_lo])
    hi = (ctypes.c_float * 3)(*[float(v) for v in box_hi])
    code = _lib.load().rs_sort_morton30(_ptr(points), n, lo, hi, _ptr(codes_out), _ptr(index_out),
                                        tptr, tbytes, _stream_handle(points.device, stream))
    if code != _lib.RS_SUCCESS:
        raise RadixSortError(code, "rs_sort_morton30")
    if check and n > 0:
        _check_guard(temp, points.device, stream, "rs_sort_morton30")
    return codes_out, index_out


def error_word(temp: torch.Tensor) -> int:
    """The device guard word at temp offset 0 (0 after a successful sort).
    Reads device memory: synchronises with the current stream."""
    return int(temp[:4].view(torch.int32).item())


def _header_word(temp: torch.Tensor, which: int, index: int = 0) -> int:
    off = int(_lib.load().rs_prof_header_offset(which)) + 4 * index
    return int(temp[off:off + 4].view(torch.int32).item())


def skipped_passes(temp: torch.Tensor, passes: int) -> list:
    """Per-pass skip flags a multi-launch sort (more than 65536 keys) left in
    temp: 1 for a pass that moved nothing and was skipped.  Reads device
    memory: synchronises with the current stream."""
    return [_header_word(temp, 1, p) for p in range(int(passes))]


def order_flag(temp: torch.Tensor) -> int:
    """0 when the last multi-launch sort found its keys already in sub-key
    order (every pass skipped), else 1.  Synchronises like skipped_passes."""
    return _header_word(temp, 2)


def copy_u32(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """Plain device copy of 32-bit words (used to calibrate byte counters)."""
    _check_words(src, "src")
    _check_words(dst, "dst")
    if src.numel() != dst.numel():
        raise ValueError("size mismatch")
    code = _lib.load().rs_copy_u32(_ptr(src), _ptr(dst), src.numel(), _stream_handle(src.device, stream))
    if code != _lib.RS_SUCCESS:
        raise RadixSortError(code, "rs_copy_u32")


def prof_enable(on: bool = True) -> bool:
    return bool(_lib.load().rs_prof_enable(1 if on else 0))


def prof_small_path(mode: int) -> int:
    """One-launch path for small inputs (test hook): 0 off, 1 on (default),
    2 on with a single workgroup.  Returns the previous mode."""
    return int(_lib.load().rs_prof_small_path(int(mode)))


def prof_tile_items(items: int) -> int:
    """Pass tiles of keys-only 32-bit sorts (test hook): 0 chosen per size
    (the default), 16 or 28 keys per thread forced.  Returns the previous
    setting."""
    return int(_lib.load().rs_prof_tile_items(int(items)))


def prof_reset() -> None:
    _lib.load().rs_prof_reset()


def prof_samples(kind: int, sub: int = -1) -> list:
    """Milliseconds of every recorded launch of one kernel kind (pass
    launches: of pass index `sub`; sub < 0 for all), in launch order."""
    lib = _lib.load()
    count = int(lib.rs_prof_samples(kind, sub, None, 0))
    buf = (ctypes.c_double * max(count, 1))()
    got = int(lib.rs_prof_samples(kind, sub, buf, count))
    return [float(buf[i]) for i in range(min(got, count))]


def prof_ranker(mode: int) -> int:
    """Local ranker (test and measurement hook): 0 LDS-atomic (default), 1
    ballot match ranker (32-bit keys; see rs_prof_ranker).  Returns the
    previous mode."""
    return int(_lib.load().rs_prof_ranker(int(mode)))


def prof_force_giveup(on: bool) -> bool:
    """Test hook: force a look-back give-up in every multi-launch sort (see
    rs_prof_force_giveup).  Returns the previous setting."""
    return bool(_lib.load().rs_prof_force_giveup(1 if on else 0))


def lds_rank_probe(digits: torch.Tensor, slots: int, unit: int, stream=None) -> torch.Tensor:
    """Run rs_prof_lds_rank_probe on a device tensor of uint32 digits (a
    multiple of 1024 * slots words) and return what each LDS add returned."""
    _check_words(digits, "digits", (torch.uint32,))
    per_block = 1024 * int(slots)
    if digits.numel() == 0 or digits.numel() % per_block:
        raise ValueError(f"digits must hold a positive multiple of {per_block} words")
    ranks = torch.empty_like(digits)
    code = _lib.load().rs_prof_lds_rank_probe(_ptr(digits), _ptr(ranks), digits.numel() // per_block, int(slots),
                                              int(unit), _stream_handle(digits.device, stream))
    if code != _lib.RS_SUCCESS:
        raise RadixSortError(code, "rs_prof_lds_rank_probe")
    return ranks


def prof_summary(kind: int) -> Tuple[int, float]:
    """(launches, total milliseconds) recorded for one kernel kind."""
    launches = ctypes.c_uint64(0)
    ms = ctypes.c_double(0.0)
    code = _lib.load().rs_prof_summary(kind, ctypes.byref(launches), ctypes.byref(ms))
    if code != _lib.RS_SUCCESS:
        raise RadixSortError(code, "rs_prof_summary")
    return int(launches.value), float(ms.value)

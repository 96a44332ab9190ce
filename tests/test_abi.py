"""C-ABI boundary checks that need no GPU: the library loads, exports every
function the public headers declare, and rejects bad arguments on the host
before making any HIP call.  (Pointers below are fake addresses: every call
here must return before touching them.)"""
import ctypes
import os
import re

import pytest

from lsd_radix_sort_pass_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("rs.h", "rs_prof.h")]

OK, INVALID, INSUFFICIENT = _lib.RS_SUCCESS, _lib.RS_ERROR_INVALID_VALUE, _lib.RS_ERROR_INSUFFICIENT_TEMP
TEMP = 0x7F0000000000          # fake, 256-byte aligned device addresses
KIN, KOUT, VIN, VOUT = 0x100000000, 0x200000000, 0x300000000, 0x400000000


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def declared_functions():
    names = []
    for h in HEADERS:
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names += re.findall(r"^[A-Za-z_][\w \t\*]*?\b(rs_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert "rs_sort_keys_u32" in names and "rs_sort_pairs_u32" in names
    assert set(names) == set(_lib.SIGNATURES), "binding and headers disagree"
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in (0, 1, 2, 3):
        assert lib.rs_status_string(code)
    assert b"unknown" in lib.rs_status_string(99)


def test_temp_bytes(lib):
    tb = lib.rs_temp_bytes
    assert tb(0, 0, 0, 32) == 0 and tb(1, 1, 0, 32) == 0 and tb(1000, 0, 7, 7) == 0
    assert tb(1000, 0, 0, 33) == 0 and tb(1000, 0, 9, 8) == 0 and tb(1000, 0, -1, 8) == 0
    assert tb(2**32, 0, 0, 32) == 0
    for n in [2, 1000, 8192, 8193, 1 << 20, (1 << 28) + 3]:
        k = tb(n, 0, 0, 32)
        p = tb(n, 1, 0, 32)
        assert k >= 4 * n and p >= 8 * n and p > k
        assert k % 256 == 0 and p % 256 == 0
        assert tb(n + 8192, 0, 0, 32) > k
    # fewer bits -> fewer passes -> no more scan state
    assert tb(1 << 20, 0, 0, 16) <= tb(1 << 20, 0, 0, 32)
    # from 2^30 - 2^16 on, 64-bit status words (twice the scan state)
    lim = (1 << 30) - (1 << 16)
    assert tb(lim, 0, 0, 32) - 4 * lim > tb(lim - 1, 0, 0, 32) - 4 * (lim - 1) + 100_000


def _keys(lib, fn, kin, kout, n, b, e, temp, tbytes):
    return getattr(lib, fn)(kin, kout, n, b, e, temp, tbytes, None)


@pytest.mark.parametrize("fn", ["rs_sort_keys_u32", "rs_sort_keys_i32", "rs_sort_keys_f32"])
def test_keys_validation(lib, fn):
    n = 10000
    need = lib.rs_temp_bytes(n, 0, 0, 32)
    call = lambda *a: _keys(lib, fn, *a)
    assert call(KIN, KOUT, 0, 0, 32, None, 0) == OK                 # n = 0: nothing to do
    assert call(None, KOUT, n, 0, 32, TEMP, need) == INVALID
    assert call(KIN, None, n, 0, 32, TEMP, need) == INVALID
    assert call(KIN, KOUT, n, -1, 32, TEMP, need) == INVALID
    assert call(KIN, KOUT, n, 0, 33, TEMP, need) == INVALID
    assert call(KIN, KOUT, n, 9, 8, TEMP, need) == INVALID
    assert call(KIN, KOUT, 2**32, 0, 32, TEMP, 2**40) == INVALID
    assert call(KIN, KIN + 4, n, 0, 32, TEMP, need) == INVALID     # partial overlap
    assert call(KIN, KOUT, n, 0, 32, None, need) == INVALID          # no temp
    assert call(KIN, KOUT, n, 0, 32, TEMP + 4, need) == INVALID      # misaligned temp
    assert call(KIN, KOUT, n, 0, 32, TEMP, need - 1) == INSUFFICIENT
    assert call(KIN, KOUT, n, 0, 32, KIN + 256, 2 * need) == INVALID  # temp overlaps keys
    assert call(KIN, KIN, 1, 0, 32, None, 0) == OK                   # trivial, in place: no work
    assert call(KIN, KIN, n, 5, 5, None, 0) == OK                    # empty bit range, in place


def test_pairs_validation(lib):
    n = 10000
    need = lib.rs_temp_bytes(n, 1, 0, 32)
    f = lib.rs_sort_pairs_u32
    call = lambda kin, kout, vin, vout, nn=n, b=0, e=32, t=TEMP, tb=need: f(kin, kout, vin, vout, nn, b, e, t, tb, None)
    assert call(KIN, KOUT, None, VOUT) == INVALID
    assert call(KIN, KOUT, VIN, None) == INVALID
    assert call(KIN, KOUT, VIN, VIN + 8) == INVALID                   # values partial overlap
    assert call(KIN, KOUT, KIN + 16, VOUT) == INVALID                 # values overlap keys
    assert call(KIN, KOUT, VIN, KOUT) == INVALID                      # vals_out is keys_out
    assert call(KIN, KOUT, VIN, VOUT, tb=lib.rs_temp_bytes(n, 0, 0, 32)) == INSUFFICIENT
    assert call(KIN, KOUT, VIN, VOUT, t=VIN) == INVALID               # temp overlaps values
    assert call(KIN, KIN, VIN, VIN, nn=1, t=None, tb=0) == OK


def test_prof_hooks_without_gpu(lib):
    prev = lib.rs_prof_enable(0)
    assert prev in (0, 1)
    assert lib.rs_prof_enable(0) == 0
    lib.rs_prof_reset()
    launches, ms = ctypes.c_uint64(5), ctypes.c_double(5.0)
    assert lib.rs_prof_summary(_lib.RS_KERNEL_PASS, ctypes.byref(launches), ctypes.byref(ms)) == OK
    assert launches.value == 0 and ms.value == 0.0
    assert lib.rs_prof_summary(99, ctypes.byref(launches), ctypes.byref(ms)) == INVALID
    assert lib.rs_copy_u32(KIN, KOUT, 0, None) == OK
    assert lib.rs_copy_u32(KIN, KIN + 4, 100, None) == INVALID
    assert lib.rs_copy_u32(None, KOUT, 100, None) == INVALID


def test_header_offsets(lib):
    """The inspection words of a sort's temp header: error word at 0, the
    per-pass skip flags and the order flag after it, inside the first 256
    bytes, 4-byte aligned, not overlapping (up to 8 skip flags)."""
    err, skip, order = (lib.rs_prof_header_offset(i) for i in range(3))
    assert err == 0
    assert skip % 4 == 0 and order % 4 == 0
    assert 4 <= skip and skip + 4 * 8 <= order and order + 4 <= 512
    bad = ctypes.c_size_t(-1).value
    assert lib.rs_prof_header_offset(3) >= order + 4 and lib.rs_prof_header_offset(3) % 256 == 0
    mode, bounds = lib.rs_prof_header_offset(4), lib.rs_prof_header_offset(5)
    assert order + 4 <= mode and mode % 16 == 0 and mode + 32 <= bounds and bounds % 4 == 0
    assert bounds + 4 * 8 * 7 <= lib.rs_prof_header_offset(3)
    assert lib.rs_prof_header_offset(6) == bad and lib.rs_prof_header_offset(-1) == bad


def test_tile_items_hook(lib):
    """16 or 28 keys per thread are forced, anything else means automatic;
    the previous setting is returned."""
    prev = lib.rs_prof_tile_items(16)
    try:
        assert lib.rs_prof_tile_items(28) == 16
        assert lib.rs_prof_tile_items(5) == 28
        assert lib.rs_prof_tile_items(0) == 0
    finally:
        lib.rs_prof_tile_items(prev)


def test_temp_bytes_covers_both_tiles(lib):
    """Keys-only 32-bit sorts may run either tile size; temp covers the one
    with more tiles (more status words), so it is at least the pairs-free
    layout of 16384-key tiles: 2 status regions of (tiles + 8) x 256 words."""
    n = 1 << 24
    tb = lib.rs_temp_bytes(n, 0, 0, 32)
    short_tiles = (n + 16383) // 16384
    assert tb >= 4 * n + 2 * (short_tiles + 8) * 256 * 4


def test_temp_bytes64(lib):
    tb = lib.rs_temp_bytes64
    assert tb(0, 0, 0, 64) == 0 and tb(1, 1, 0, 64) == 0 and tb(1000, 0, 40, 40) == 0
    assert tb(1000, 0, 0, 65) == 0 and tb(1000, 0, 9, 8) == 0 and tb(1000, 0, -1, 8) == 0
    assert tb(2**32, 0, 0, 64) == 0
    for n in [2, 1000, 14336, 14337, 1 << 20, (1 << 27) + 3]:
        k = tb(n, 0, 0, 64)
        p = tb(n, 1, 0, 64)
        assert k >= 8 * n and p >= 12 * n and p > k
        assert k % 256 == 0 and p % 256 == 0
        # a 32-bit range of a 64-bit key still needs a 64-bit alternate buffer
        assert tb(n, 0, 0, 32) >= 8 * n
        assert tb(n, 0, 0, 32) >= lib.rs_temp_bytes(n, 0, 0, 32)
        if n >= 1000:
            assert tb(n, 0, 0, 32) > lib.rs_temp_bytes(n, 0, 0, 32)
    assert tb(1 << 20, 0, 0, 16) <= tb(1 << 20, 0, 0, 64)
    # the 32-bit call rejects a 64-bit bit range
    assert lib.rs_temp_bytes(1000, 0, 0, 64) == 0


@pytest.mark.parametrize("fn", ["rs_sort_keys_u64", "rs_sort_keys_i64", "rs_sort_keys_f64"])
def test_keys64_validation(lib, fn):
    n = 10000
    need = lib.rs_temp_bytes64(n, 0, 0, 64)
    call = lambda *a: _keys(lib, fn, *a)
    assert call(KIN, KOUT, 0, 0, 64, None, 0) == OK
    assert call(None, KOUT, n, 0, 64, TEMP, need) == INVALID
    assert call(KIN, KOUT, n, 0, 65, TEMP, need) == INVALID
    assert call(KIN, KOUT, n, 40, 39, TEMP, need) == INVALID
    assert call(KIN + 4, KOUT, n, 0, 64, TEMP, need) == INVALID      # keys not 8-byte aligned
    assert call(KIN, KOUT + 4, n, 0, 64, TEMP, need) == INVALID
    assert call(KIN, KIN + 8, n, 0, 64, TEMP, need) == INVALID       # partial overlap
    assert call(KIN, KOUT, n, 0, 64, TEMP, need - 1) == INSUFFICIENT
    # the 32-bit temp size is too small for 64-bit keys
    assert call(KIN, KOUT, n, 0, 32, TEMP, lib.rs_temp_bytes(n, 0, 0, 32)) == INSUFFICIENT
    assert call(KIN, KOUT, n, 0, 64, KIN + 8 * n - 256, 2 * need) == INVALID  # temp overlaps keys
    assert call(KIN, KIN, 1, 0, 64, None, 0) == OK
    assert call(KIN, KIN, n, 63, 63, None, 0) == OK


@pytest.mark.parametrize("fn", ["rs_sort_pairs_u64", "rs_sort_pairs_i64", "rs_sort_pairs_f64"])
def test_pairs64_validation(lib, fn):
    n = 10000
    need = lib.rs_temp_bytes64(n, 1, 0, 64)
    f = getattr(lib, fn)
    call = lambda kin, kout, vin, vout, nn=n, b=0, e=64, t=TEMP, tb=need: f(kin, kout, vin, vout, nn, b, e, t, tb, None)
    assert call(KIN, KOUT, None, VOUT) == INVALID
    assert call(KIN, KOUT, VIN + 2, VOUT) == INVALID                  # values not 4-byte aligned
    assert call(KIN, KOUT, KIN + 8 * n - 8, VOUT) == INVALID          # values overlap the keys' last element
    assert call(KIN, KOUT, VIN, VOUT, tb=lib.rs_temp_bytes64(n, 0, 0, 64)) == INSUFFICIENT
    assert call(KIN, KIN, VIN, VIN, nn=1, t=None, tb=0) == OK


def test_32bit_keys_must_be_aligned(lib):
    n = 10000
    need = lib.rs_temp_bytes(n, 0, 0, 32)
    assert lib.rs_sort_keys_u32(KIN + 2, KOUT, n, 0, 32, TEMP, need, None) == INVALID


def test_morton_validation(lib):
    import ctypes as C
    f = lib.rs_sort_morton30
    box = lambda *v: (C.c_float * 3)(*v)
    lo, hi = box(0, 0, 0), box(1, 1, 1)
    n = 5000
    need = lib.rs_temp_bytes_morton30(n)
    assert lib.rs_temp_bytes_morton30(0) == 0 and lib.rs_temp_bytes_morton30(1) > 0
    assert need >= 8 * n and need % 256 == 0
    call = lambda xyz=KIN, nn=n, l=lo, h=hi, co=KOUT, io=VOUT, t=TEMP, tb=need: f(xyz, nn, l, h, co, io, t, tb, None)
    assert call(nn=0) == OK
    assert call(l=None) == INVALID
    assert call(h=box(1, 0, 1)) == INVALID                          # hi <= lo on y
    assert call(h=box(1, float("inf"), 1)) == INVALID
    assert call(l=box(float("nan"), 0, 0)) == INVALID
    assert call(l=box(-3e38, 0, 0), h=box(3e38, 1, 1)) == INVALID   # the width overflows single precision
    assert call(xyz=None) == INVALID
    assert call(xyz=KIN + 2) == INVALID                             # not 4-byte aligned
    assert call(co=KIN + 4) == INVALID                              # codes overlap the points
    assert call(io=KOUT + 8) == INVALID                             # index overlaps the codes
    assert call(t=TEMP + 4) == INVALID
    assert call(tb=need - 1) == INSUFFICIENT
    assert call(t=KIN + 256, tb=need) == INVALID                    # temp overlaps the points
    assert call(nn=2**32) == INVALID


def test_temp_bytes_ex(lib):
    tb = lib.rs_temp_bytes_ex
    assert tb(1000, 3, 0, 0, 16) == 0 and tb(1000, 2, 2, 0, 16) == 0   # bad key / value sizes
    assert tb(1000, 2, 0, 0, 17) == 0 and tb(1, 2, 0, 0, 16) == 0
    for n in [1000, 8193, 1 << 20]:
        k16, k32, k64 = tb(n, 2, 0, 0, 16), tb(n, 4, 0, 0, 32), tb(n, 8, 0, 0, 64)
        assert k16 >= 2 * n and k16 < k32 < k64
        assert tb(n, 4, 0, 0, 32) == lib.rs_temp_bytes(n, 0, 0, 32)
        assert tb(n, 4, 4, 0, 32) == lib.rs_temp_bytes(n, 1, 0, 32)
        assert tb(n, 8, 4, 0, 64) == lib.rs_temp_bytes64(n, 1, 0, 64)
        assert tb(n, 4, 8, 0, 32) >= 12 * n and tb(n, 4, 8, 0, 32) > tb(n, 4, 4, 0, 32)
        assert tb(n, 8, 8, 0, 64) >= 16 * n


@pytest.mark.parametrize("fn", ["rs_sort_keys_u16", "rs_sort_keys_i16", "rs_sort_keys_f16"])
def test_keys16_validation(lib, fn):
    n = 10001
    need = lib.rs_temp_bytes_ex(n, 2, 0, 0, 16)
    call = lambda *a: _keys(lib, fn, *a)
    assert call(KIN, KOUT, n, 0, 17, TEMP, need) == INVALID
    assert call(KIN + 1, KOUT, n, 0, 16, TEMP, need) == INVALID       # keys not 2-byte aligned
    assert call(KIN, KIN + 2, n, 0, 16, TEMP, need) == INVALID        # partial overlap
    assert call(KIN, KOUT, n, 0, 16, TEMP, need - 1) == INSUFFICIENT
    assert call(KIN, KIN, n, 7, 7, None, 0) == OK


@pytest.mark.parametrize("fn", ["rs_sort_pairs_u16_v64", "rs_sort_pairs_f32_v64", "rs_sort_pairs_f64_v64"])
def test_pairs_v64_validation(lib, fn):
    n = 10000
    kb = {"u16": 2, "f32": 4, "f64": 8}[fn.split("_")[3]]
    need = lib.rs_temp_bytes_ex(n, kb, 8, 0, 8 * kb)
    f = getattr(lib, fn)
    call = lambda kin, kout, vin, vout, t=TEMP, tb=need: f(kin, kout, vin, vout, n, 0, 8 * kb, t, tb, None)
    assert call(KIN, KOUT, VIN + 4, VOUT) == INVALID                  # values not 8-byte aligned
    assert call(KIN, KOUT, VIN, VOUT + 4) == INVALID
    assert call(KIN, KOUT, VIN, VIN + 8) == INVALID                   # values partial overlap
    assert call(KIN, KOUT, KIN + kb * n - 8, VOUT) == INVALID         # values overlap keys
    assert call(KIN, KOUT, VIN, VOUT, tb=lib.rs_temp_bytes_ex(n, kb, 4, 0, 8 * kb)) == INSUFFICIENT


def _header_macro(name):
    src = open(HEADERS[0]).read()
    m = re.search(r"#define\s+" + name + r"\s+\(\(size_t\)(\d+)\s*<<\s*(\d+)\)", src)
    assert m, name
    return int(m.group(1)) << int(m.group(2))


def test_noalloc_limits(lib):
    """rs_sort_keys_u32_noalloc: the scratch holds the temp storage of the
    largest allowed sort (every bit range); larger inputs, bad bit ranges
    and NULL pointers are rejected on the host, and trivial calls need no
    scratch."""
    max_keys = _header_macro("RS_NOALLOC_MAX_KEYS")
    scratch = _header_macro("RS_NOALLOC_SCRATCH_BYTES")
    assert max_keys == (1 << 22)
    for b, e in [(0, 32), (0, 8), (3, 29), (24, 32)]:
        assert 0 < lib.rs_temp_bytes(max_keys, 0, b, e) <= scratch
    f = lib.rs_sort_keys_u32_noalloc
    assert f(KIN, KOUT, max_keys + 1, 0, 32, None) == _lib.RS_ERROR_SCRATCH_LIMIT
    assert f(KIN, KOUT, 2**32, 0, 32, None) == _lib.RS_ERROR_SCRATCH_LIMIT
    assert f(KIN, KOUT, 1000, 0, 33, None) == INVALID
    assert f(KIN, KOUT, 1000, 9, 8, None) == INVALID
    assert f(None, KOUT, 1000, 0, 32, None) == INVALID
    assert f(KIN, KIN + 4, 1000, 0, 32, None) == INVALID             # partial overlap
    assert f(KIN, KOUT, 0, 0, 32, None) == OK
    assert f(KIN, KIN, 1, 0, 32, None) == OK                         # trivial, in place
    assert f(KIN, KIN, 1000, 4, 4, None) == OK
    assert b"scratch" in lib.rs_status_string(_lib.RS_ERROR_SCRATCH_LIMIT)


def test_measurement_hooks_validation(lib):
    """The per-launch samples, the forced give-up switch and the LDS probe
    reject bad arguments on the host."""
    buf = (ctypes.c_double * 4)()
    assert lib.rs_prof_samples(99, -1, buf, 4) == 0
    assert lib.rs_prof_samples(_lib.RS_KERNEL_PASS, 0, None, 0) == 0
    prev = lib.rs_prof_force_giveup(1)
    try:
        assert lib.rs_prof_force_giveup(0) == 1
    finally:
        lib.rs_prof_force_giveup(prev)
    prev = lib.rs_prof_ranker(1)
    try:
        assert lib.rs_prof_ranker(7) == 1 and lib.rs_prof_ranker(0) == 0
    finally:
        lib.rs_prof_ranker(prev)
    probe = lib.rs_prof_lds_rank_probe
    assert probe(None, KOUT, 1, 28, 4, None) == INVALID
    assert probe(KIN, None, 1, 28, 4, None) == INVALID
    assert probe(KIN, KOUT, 0, 28, 4, None) == INVALID
    assert probe(KIN, KOUT, 65536, 28, 4, None) == INVALID
    assert probe(KIN, KOUT, 1, 12, 4, None) == INVALID
    assert probe(KIN, KOUT, 1, 28, 2, None) == INVALID
    assert probe(KIN, KIN + 4, 1, 8, 1, None) == INVALID              # overlapping arrays

"""Pins for the CPU oracle (no GPU).

Each test ties the oracle to something other than itself:
  * the worked decimal example printed on the wandres.dev page
    ("La idea y el requisito de estabilidad"), stored in tests/golden/;
  * closed-form ordered-key values worked out by hand from IEEE-754 and
    two's-complement bit patterns;
  * numpy's stable sorts / Python's stable ``sorted`` using the NATIVE order
    of the key type (never the oracle's transform), which fixes the int rule
    of the wandres.dev page and the float policy of the Silicon Studio page
    (NaN and +-Inf last, -0.0 before +0.0);
  * brute force over every short sequence of an edge-value alphabet;
  * the one-bit two-bucket formula of the Silicon Studio page
    ("アルゴリズムの詳細") as an independent algorithm;
  * invariance of the result under the digit width.
"""
import itertools
import math
import os
import struct

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.txt")


def _golden_rows():
    rows = {}
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            label, *vals = line.split()
            rows[label] = [int(v) for v in vals]
    return rows


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def bits_f32(u: int) -> float:
    return struct.unpack("<f", struct.pack("<I", u))[0]


# --------------------------------------------------------------------------
# Worked example (wandres.dev, "La idea y el requisito de estabilidad")
# --------------------------------------------------------------------------

def test_worked_example_decimal_passes():
    rows = _golden_rows()
    cur = np.array(rows["input"], dtype=np.uint32)
    for place, label in enumerate(["units", "tens", "hundreds"]):
        cur = oracle.decimal_pass(cur, place)
        assert cur.tolist() == rows[label], f"after the {label} pass"


@pytest.mark.parametrize("radix_bits", [1, 2, 3, 4, 8, 11, 16])
def test_worked_example_binary_digits_reach_final_line(radix_bits):
    rows = _golden_rows()
    keys = np.array(rows["input"], dtype=np.uint32)
    out = oracle.lsd_sort(keys, radix_bits=radix_bits)
    assert out.tolist() == rows["hundreds"]
    assert oracle.split_sort(keys).tolist() == rows["hundreds"]


def test_worked_example_order_of_equal_units_kept():
    # 802 and 002 share the units digit and 802 comes first in the input:
    # the page stresses that a stable pass keeps 802 ahead of 002.
    rows = _golden_rows()
    units = oracle.decimal_pass(np.array(rows["input"], dtype=np.uint32), 0).tolist()
    assert units.index(802) < units.index(2)


# --------------------------------------------------------------------------
# Ordered keys: closed-form values
# --------------------------------------------------------------------------

def test_u32_key_is_identity():
    for v in [0, 1, 0x7FFFFFFF, 0x80000000, 0xFFFFFFFF, 0x12345678]:
        assert oracle.ordered_key(oracle.KEY_U32, v) == v


def test_i32_key_closed_form():
    # Two's complement: INT_MIN has pattern 0x80000000 and must map to the
    # smallest key, -1 (0xFFFFFFFF) sits just below 0, INT_MAX is the largest.
    assert oracle.ordered_key(oracle.KEY_I32, 0x80000000) == 0x00000000
    assert oracle.ordered_key(oracle.KEY_I32, 0xFFFFFFFF) == 0x7FFFFFFF
    assert oracle.ordered_key(oracle.KEY_I32, 0x00000000) == 0x80000000
    assert oracle.ordered_key(oracle.KEY_I32, 0x7FFFFFFF) == 0xFFFFFFFF
    # -2 < -1 (the Silicon Studio int rule would invert this pair).
    assert oracle.ordered_key(oracle.KEY_I32, 0xFFFFFFFE) < oracle.ordered_key(oracle.KEY_I32, 0xFFFFFFFF)


def test_f32_key_closed_form():
    K = lambda u: oracle.ordered_key(oracle.KEY_F32, u)
    assert K(0x7F800000) == 0xFFFFFFFF           # +Inf
    assert K(0xFF800000) == 0xFFFFFFFF           # -Inf
    assert K(0x7FC00000) == 0xFFFFFFFF           # quiet NaN
    assert K(0xFFC12345) == 0xFFFFFFFF           # negative NaN with payload
    assert K(0x7F800001) == 0xFFFFFFFF           # signalling NaN
    assert K(f32_bits(-1.0)) == 0x407FFFFF       # ~0xBF800000
    assert K(0x80000000) == 0x7FFFFFFF           # -0.0
    assert K(0x00000000) == 0x80000000           # +0.0
    assert K(0x00000001) == 0x80000001           # smallest denormal
    assert K(0x80000001) == 0x7FFFFFFE           # -smallest denormal
    assert K(f32_bits(1.0)) == 0xBF800000
    assert K(0x7F7FFFFF) == 0xFF7FFFFF           # FLT_MAX
    assert K(0xFF7FFFFF) == 0x00800000           # -FLT_MAX


def test_f32_key_orders_like_values_on_a_ladder():
    # Strictly increasing finite floats (the appendix argument of the
    # Silicon Studio page) must give strictly increasing keys.
    ladder = [-3.4028235e38, -1e10, -2.0, -1.0, -1e-30, -1e-45, -0.0, 0.0,
              1e-45, 1e-38, 1e-30, 0.5, 1.0, 1.0000001, 2.0, 1e10, 3.4028235e38]
    keys = [oracle.ordered_key(oracle.KEY_F32, f32_bits(x)) for x in ladder]
    assert keys == sorted(keys) and len(set(keys)) == len(keys)


# --------------------------------------------------------------------------
# Native-order references (never use the oracle's transform)
# --------------------------------------------------------------------------

def native_f32_perm(keys: np.ndarray) -> np.ndarray:
    """Stable permutation under the Silicon Studio float policy written with
    IEEE comparisons: finite values by value, -0.0 before +0.0, every NaN and
    +-Inf after all finite values in input order."""
    special = np.isnan(keys) | np.isinf(keys)
    val = np.where(special, np.float32(0), keys).astype(np.float64)
    zero_pos = np.where(special, 0, np.where(np.signbit(keys), 0, 1))
    return np.lexsort((zero_pos, val, special.astype(np.int8)))


def native_perm(keys: np.ndarray, begin_bit: int = 0, end_bit: int = 32) -> np.ndarray:
    if keys.dtype == np.float32:
        assert (begin_bit, end_bit) == (0, 32)
        return native_f32_perm(keys)
    width = end_bit - begin_bit
    if keys.dtype == np.uint32:
        sub = (keys.astype(np.uint64) >> np.uint64(begin_bit)) & np.uint64((1 << width) - 1)
    elif keys.dtype == np.int32:
        if end_bit == 32:
            # Dropping the low bits of a signed value keeps its order:
            # floor(x / 2^b) == arithmetic shift.
            sub = keys.astype(np.int64) >> np.int64(begin_bit)
        else:
            # Below bit 31 the ordered key has the same bits as x.
            sub = (keys.astype(np.int64) & np.int64(0xFFFFFFFF)) >> np.int64(begin_bit)
            sub &= np.int64((1 << width) - 1)
    else:
        raise TypeError(keys.dtype)
    return np.argsort(sub, kind="stable")


def _inputs(dtype, n, seed):
    rng = np.random.default_rng(seed)
    if dtype == np.uint32:
        return [rng.integers(0, 2**32, n, dtype=np.uint32),
                rng.integers(0, 7, n, dtype=np.uint32),
                (rng.integers(0, 2**32, n, dtype=np.uint32)
                 & rng.integers(0, 2**32, n, dtype=np.uint32)
                 & rng.integers(0, 2**32, n, dtype=np.uint32))]
    if dtype == np.int32:
        return [rng.integers(-(2**31), 2**31, n, dtype=np.int32),
                rng.integers(-3, 4, n, dtype=np.int32),
                np.array(([-2**31, 2**31 - 1, -1, 0, 1, -2] * n)[:n], dtype=np.int32)]
    if dtype == np.float32:
        g = rng.normal(0, 1000, n).astype(np.float32)
        b = g.view(np.uint32)
        idx = rng.choice(n, size=min(n, 64), replace=False)
        specials = np.array([0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC0BEEF, 0x7F800001,
                             0x80000000, 0x00000000, 0x00000001, 0x80000001, 0x7F7FFFFF,
                             0xFF7FFFFF, 0x00800000], dtype=np.uint32)
        b[idx] = specials[rng.integers(0, specials.size, idx.size)]
        small = rng.integers(-4, 5, n).astype(np.float32)
        return [g, small]
    raise TypeError(dtype)


@pytest.mark.parametrize("dtype", [np.uint32, np.int32, np.float32])
@pytest.mark.parametrize("n", [0, 1, 2, 3, 17, 1000, 1 << 16])
def test_lsd_matches_native_stable_sort(dtype, n):
    for i, keys in enumerate(_inputs(dtype, n, seed=7 + n)):
        vals = np.arange(n, dtype=np.uint32)
        k, v = oracle.lsd_sort(keys, vals)
        perm = native_perm(keys)
        assert np.array_equal(v, perm.astype(np.uint32)), f"input {i}"
        assert np.array_equal(k.view(np.uint32), keys.view(np.uint32)[perm]), f"input {i}"


@pytest.mark.parametrize("dtype", [np.uint32, np.int32])
@pytest.mark.parametrize("bits", [(0, 32), (0, 4), (4, 8), (1, 31), (28, 32), (0, 30),
                                  (8, 16), (5, 5), (13, 32), (0, 1), (31, 32)])
def test_lsd_bit_ranges_match_native(dtype, bits):
    b, e = bits
    for keys in _inputs(dtype, 5000, seed=99 + b + 37 * e):
        vals = np.arange(keys.size, dtype=np.uint32)
        k, v = oracle.lsd_sort(keys, vals, begin_bit=b, end_bit=e)
        perm = native_perm(keys, b, e)
        assert np.array_equal(v, perm.astype(np.uint32))
        assert np.array_equal(k, keys[perm])


def test_large_random_matches_numpy():
    rng = np.random.default_rng(2024)
    n = 1 << 20
    for keys in [rng.integers(0, 2**32, n, dtype=np.uint32),
                 rng.integers(-(2**31), 2**31, n, dtype=np.int32)]:
        k = oracle.lsd_sort(keys)
        assert np.array_equal(k, np.sort(keys, kind="stable"))
    f = rng.normal(0, 1, n).astype(np.float32)
    k = oracle.lsd_sort(f)
    assert np.array_equal(k.view(np.uint32), f.view(np.uint32)[native_f32_perm(f)])


# --------------------------------------------------------------------------
# Brute force over short sequences of edge values
# --------------------------------------------------------------------------

U32_ALPHABET = [0, 1, 0x7FFFFFFF, 0x80000000, 0xFFFFFFFE, 0xFFFFFFFF, 0x0F, 0xF0]
F32_ALPHABET_A = [0xFF800000, f32_bits(-1.0), 0x80000000, 0x00000000, 0x00000001,
                  f32_bits(1.0), 0x7F800000, 0x7FC00000]
F32_ALPHABET_B = [0xFFC0BEEF, 0xFF7FFFFF, 0x80000001, 0x7F7FFFFF, 0x7FC00001,
                  0x80000000, f32_bits(2.0), 0x00000000]


def _f32_native_key(u):
    x = bits_f32(u)
    if math.isnan(x) or math.isinf(x):
        return (1, 0.0, 0)
    return (0, x, 0 if math.copysign(1.0, x) < 0 else 1)


def _native_key(dtype, begin_bit, end_bit):
    width = end_bit - begin_bit
    if dtype == np.float32:
        return _f32_native_key
    if dtype == np.uint32:
        return lambda u: (u >> begin_bit) & ((1 << width) - 1)
    # int32 given as its bit pattern
    def signed(u):
        return u - (1 << 32) if u & 0x80000000 else u
    if end_bit == 32:
        return lambda u: signed(u) >> begin_bit
    return lambda u: (u >> begin_bit) & ((1 << width) - 1)


def _brute(dtype, alphabet, max_len, bit_ranges, sorter):
    checked = 0
    for begin_bit, end_bit in bit_ranges:
        key = _native_key(dtype, begin_bit, end_bit)
        for length in range(0, max_len + 1):
            for seq in itertools.product(range(len(alphabet)), repeat=length):
                pats = [alphabet[s] for s in seq]
                keys = np.array(pats, dtype=np.uint32).view(dtype)
                vals = np.arange(length, dtype=np.uint32)
                k, v = sorter(keys, vals, begin_bit, end_bit)
                expect = sorted(range(length), key=lambda i: key(pats[i]))
                assert v.tolist() == expect, (seq, begin_bit, end_bit)
                assert k.view(np.uint32).tolist() == [pats[i] for i in expect]
                checked += 1
    return checked


def _lsd(keys, vals, b, e):
    return oracle.lsd_sort(keys, vals, begin_bit=b, end_bit=e)


def _split(keys, vals, b, e):
    return oracle.split_sort(keys, vals, begin_bit=b, end_bit=e)


@pytest.mark.parametrize("sorter", [_lsd, _split], ids=["lsd", "split"])
def test_brute_force_u32(sorter):
    assert _brute(np.uint32, U32_ALPHABET, 5, [(0, 32)], sorter) > 30000
    _brute(np.uint32, U32_ALPHABET, 4, [(0, 4), (4, 8), (1, 31), (28, 32), (3, 3)], sorter)


def test_brute_force_i32():
    _brute(np.int32, U32_ALPHABET, 5, [(0, 32)], _lsd)
    _brute(np.int32, U32_ALPHABET, 4, [(4, 32), (0, 4), (0, 31)], _lsd)


def test_brute_force_f32():
    _brute(np.float32, F32_ALPHABET_A, 5, [(0, 32)], _lsd)
    _brute(np.float32, F32_ALPHABET_B, 4, [(0, 32)], _lsd)
    _brute(np.float32, F32_ALPHABET_A, 3, [(0, 32)], _split)


# --------------------------------------------------------------------------
# Independent algorithms and digit-width invariance
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [np.uint32, np.int32, np.float32])
def test_split_formula_equals_counting_sort(dtype):
    for keys in _inputs(dtype, 1 << 14, seed=5):
        vals = np.arange(keys.size, dtype=np.uint32)
        bit_ranges = [(0, 32)] if dtype == np.float32 else [(0, 32), (3, 19), (0, 30)]
        for b, e in bit_ranges:
            k1, v1 = oracle.lsd_sort(keys, vals, begin_bit=b, end_bit=e)
            k2, v2 = oracle.split_sort(keys, vals, begin_bit=b, end_bit=e)
            assert np.array_equal(v1, v2) and np.array_equal(k1.view(np.uint32), k2.view(np.uint32))


@pytest.mark.parametrize("dtype", [np.uint32, np.int32, np.float32])
def test_result_independent_of_digit_width(dtype):
    keys = _inputs(dtype, 20000, seed=11)[0]
    vals = np.arange(keys.size, dtype=np.uint32)
    ref = oracle.lsd_sort(keys, vals, radix_bits=8)
    for r in [1, 3, 4, 5, 7, 11, 16]:
        k, v = oracle.lsd_sort(keys, vals, radix_bits=r)
        assert np.array_equal(v, ref[1]) and np.array_equal(k.view(np.uint32), ref[0].view(np.uint32))


def test_stability_values_increase_within_equal_keys():
    rng = np.random.default_rng(3)
    keys = rng.integers(0, 16, 1 << 16, dtype=np.uint32)
    vals = np.arange(keys.size, dtype=np.uint32)
    k, v = oracle.lsd_sort(keys, vals)
    assert np.all(np.diff(k.astype(np.int64)) >= 0)
    same = k[1:] == k[:-1]
    assert np.all(v[1:][same] > v[:-1][same])


def test_identity_cases():
    keys = np.array([5, 3, 9, 3], dtype=np.uint32)
    assert oracle.lsd_sort(keys, begin_bit=7, end_bit=7).tolist() == [5, 3, 9, 3]
    same = np.full(100, 42, dtype=np.uint32)
    k, v = oracle.lsd_sort(same, np.arange(100, dtype=np.uint32))
    assert v.tolist() == list(range(100))


def test_invalid_arguments_rejected():
    keys = np.zeros(4, dtype=np.uint32)
    for b, e in [(-1, 32), (0, 33), (9, 8)]:
        with pytest.raises(ValueError):
            oracle.lsd_sort(keys, begin_bit=b, end_bit=e)
    with pytest.raises(ValueError):
        oracle.lsd_sort(keys, radix_bits=0)
    with pytest.raises(ValueError):
        oracle.lsd_sort(keys, radix_bits=17)

"""Pins for the CPU oracle's 64-bit keys (no GPU).

The Silicon Studio page ("符号付型、浮動小数点型に対する radix sort") ends by
noting that 64-bit types take the same procedure as its 32-bit rules.  Each
test ties the 64-bit oracle to something other than itself: closed-form
ordered keys worked out by hand from IEEE-754 binary64 and two's complement,
numpy / Python stable sorts in the NATIVE order of the type, brute force over
every short sequence of edge values, the one-bit two-bucket formula as an
independent algorithm, and invariance under the digit width."""
import itertools
import math
import struct

import numpy as np
import pytest

import oracle


def f64_bits(x: float) -> int:
    return struct.unpack("<Q", struct.pack("<d", x))[0]


def bits_f64(u: int) -> float:
    return struct.unpack("<d", struct.pack("<Q", u))[0]


ALL = 0xFFFFFFFFFFFFFFFF


def test_u64_key_is_identity():
    for u in [0, 1, 0x7FFFFFFFFFFFFFFF, 0x8000000000000000, ALL]:
        assert oracle.ordered_key(oracle.KEY_U64, u) == u


def test_i64_key_closed_form():
    K = lambda u: oracle.ordered_key(oracle.KEY_I64, u)
    assert K(0x8000000000000000) == 0                      # INT64_MIN
    assert K(ALL) == 0x7FFFFFFFFFFFFFFF                    # -1
    assert K(0) == 0x8000000000000000
    assert K(1) == 0x8000000000000001
    assert K(0x7FFFFFFFFFFFFFFF) == ALL                    # INT64_MAX


def test_f64_key_closed_form():
    K = lambda u: oracle.ordered_key(oracle.KEY_F64, u)
    assert K(0x7FF0000000000000) == ALL                    # +Inf
    assert K(0xFFF0000000000000) == ALL                    # -Inf
    assert K(0x7FF8000000000000) == ALL                    # quiet NaN
    assert K(0xFFF8000000001234) == ALL                    # negative NaN with payload
    assert K(0x7FF0000000000001) == ALL                    # signalling NaN
    assert K(f64_bits(-1.0)) == 0x400FFFFFFFFFFFFF         # ~0xBFF0000000000000
    assert K(0x8000000000000000) == 0x7FFFFFFFFFFFFFFF     # -0.0
    assert K(0x0000000000000000) == 0x8000000000000000     # +0.0
    assert K(0x0000000000000001) == 0x8000000000000001     # smallest denormal
    assert K(0x8000000000000001) == 0x7FFFFFFFFFFFFFFE     # -smallest denormal
    assert K(f64_bits(1.0)) == 0xBFF0000000000000
    assert K(0x7FEFFFFFFFFFFFFF) == 0xFFEFFFFFFFFFFFFF     # DBL_MAX
    assert K(0xFFEFFFFFFFFFFFFF) == 0x0010000000000000     # -DBL_MAX


def test_f64_key_orders_like_values_on_a_ladder():
    ladder = [-1.7976931348623157e308, -1e100, -2.0, -1.0, -1e-300, -5e-324, -0.0, 0.0,
              5e-324, 1e-308, 1e-300, 0.5, 1.0, 1.0000000000000002, 2.0, 1e100, 1.7976931348623157e308]
    keys = [oracle.ordered_key(oracle.KEY_F64, f64_bits(x)) for x in ladder]
    assert keys == sorted(keys) and len(set(keys)) == len(keys)


def native_f64_perm(keys: np.ndarray) -> np.ndarray:
    """Stable permutation under the Silicon Studio float policy written with
    IEEE comparisons: finite values by value, -0.0 before +0.0, every NaN and
    +-Inf after all finite values in input order."""
    special = np.isnan(keys) | np.isinf(keys)
    val = np.where(special, 0.0, keys)
    zero_pos = np.where(special, 0, np.where(np.signbit(keys), 0, 1))
    return np.lexsort((zero_pos, val, special.astype(np.int8)))


def native_sub(keys: np.ndarray, begin_bit: int, end_bit: int) -> list:
    """Python-int sub-keys in the native order of the type."""
    width = end_bit - begin_bit
    raw = keys.view(np.uint64).tolist()
    if keys.dtype == np.int64 and end_bit == 64:
        # Dropping low bits of a signed value keeps its order (floor division).
        return [(u - (1 << 64) if u >> 63 else u) >> begin_bit for u in raw]
    # uint64, or int64 below bit 63 (the ordered key has the raw bits there).
    return [(u >> begin_bit) & ((1 << width) - 1) for u in raw]


def _inputs(dtype, n, seed):
    rng = np.random.default_rng(seed)
    if dtype == np.uint64:
        return [rng.integers(0, 2**64, n, dtype=np.uint64), rng.integers(0, 7, n, dtype=np.uint64),
                rng.integers(0, 2**64, n, dtype=np.uint64) & rng.integers(0, 2**64, n, dtype=np.uint64)]
    if dtype == np.int64:
        return [rng.integers(-(2**63), 2**63, n, dtype=np.int64), rng.integers(-3, 4, n, dtype=np.int64),
                np.array(([-2**63, 2**63 - 1, -1, 0, 1, -2] * n)[:n], dtype=np.int64)]
    g = rng.normal(0, 1e6, n)
    b = g.view(np.uint64)
    idx = rng.choice(n, size=min(n, 64), replace=False)
    specials = np.array([0x7FF0000000000000, 0xFFF0000000000000, 0x7FF8000000000000, 0xFFF8000000001234,
                         0x7FF0000000000001, 0x8000000000000000, 0, 1, 0x8000000000000001,
                         0x7FEFFFFFFFFFFFFF, 0xFFEFFFFFFFFFFFFF], dtype=np.uint64)
    b[idx] = specials[rng.integers(0, specials.size, idx.size)]
    return [g, rng.integers(-4, 5, n).astype(np.float64)]


@pytest.mark.parametrize("dtype", [np.uint64, np.int64, np.float64])
@pytest.mark.parametrize("n", [0, 1, 2, 3, 17, 1000, 1 << 14])
def test_lsd64_matches_native_stable_sort(dtype, n):
    for keys in _inputs(dtype, n, seed=n + 3):
        vals = np.arange(n, dtype=np.uint32)
        k, v = oracle.lsd_sort(keys, vals)
        perm = native_f64_perm(keys) if dtype == np.float64 else np.argsort(keys, kind="stable")
        assert np.array_equal(v, perm.astype(np.uint32))
        assert np.array_equal(k.view(np.uint64), keys.view(np.uint64)[perm])


@pytest.mark.parametrize("dtype", [np.uint64, np.int64])
@pytest.mark.parametrize("bits", [(0, 64), (0, 8), (56, 64), (3, 61), (32, 64), (0, 32), (63, 64), (7, 7)])
def test_lsd64_bit_ranges_match_native(dtype, bits):
    b, e = bits
    for keys in _inputs(dtype, 3000, seed=b * 64 + e):
        vals = np.arange(keys.size, dtype=np.uint32)
        _, v = oracle.lsd_sort(keys, vals, begin_bit=b, end_bit=e)
        sub = native_sub(keys, b, e)
        expect = sorted(range(keys.size), key=lambda i: sub[i])  # Python's sort is stable
        assert v.tolist() == expect


U64_ALPHABET = [0, 1, 0x7FFFFFFFFFFFFFFF, 0x8000000000000000, 0xFFFFFFFFFFFFFFFE, ALL,
                0x00000000FFFFFFFF, 0xFFFFFFFF00000000]
F64_ALPHABET = [0xFFF0000000000000, f64_bits(-1.0), 0x8000000000000000, 0, 1, f64_bits(1.0),
                0x7FF0000000000000, 0x7FF8000000000000]


def _native64(dtype):
    if dtype == np.float64:
        def key(u):
            x = bits_f64(u)
            if math.isnan(x) or math.isinf(x):
                return (1, 0.0, 0)
            return (0, x, 0 if math.copysign(1.0, x) < 0 else 1)
        return key
    if dtype == np.int64:
        return lambda u: u - (1 << 64) if u >> 63 else u
    return lambda u: u


@pytest.mark.parametrize("dtype,alphabet", [(np.uint64, U64_ALPHABET), (np.int64, U64_ALPHABET),
                                            (np.float64, F64_ALPHABET)])
def test_brute_force_64(dtype, alphabet):
    key = _native64(dtype)
    for length in range(0, 5):
        for seq in itertools.product(range(len(alphabet)), repeat=length):
            pats = [alphabet[s] for s in seq]
            keys = np.array(pats, dtype=np.uint64).view(dtype)
            vals = np.arange(length, dtype=np.uint32)
            k, v = oracle.lsd_sort(keys, vals)
            expect = sorted(range(length), key=lambda i: key(pats[i]))
            assert v.tolist() == expect, seq
            assert k.view(np.uint64).tolist() == [pats[i] for i in expect]


@pytest.mark.parametrize("dtype", [np.uint64, np.int64, np.float64])
def test_split64_equals_counting_sort_and_width_invariance(dtype):
    for keys in _inputs(dtype, 1 << 12, seed=11):
        vals = np.arange(keys.size, dtype=np.uint32)
        k8, v8 = oracle.lsd_sort(keys, vals)
        ks, vs = oracle.split_sort(keys, vals)
        assert np.array_equal(v8, vs) and np.array_equal(k8.view(np.uint64), ks.view(np.uint64))
        for r in [1, 4, 11, 16]:
            kr, vr = oracle.lsd_sort(keys, vals, radix_bits=r)
            assert np.array_equal(vr, v8)


def test_invalid_64_arguments_rejected():
    keys = np.arange(10, dtype=np.uint64)
    with pytest.raises(ValueError):
        oracle.lsd_sort(keys, begin_bit=0, end_bit=65)
    with pytest.raises(ValueError):
        oracle.lsd_sort(keys, begin_bit=9, end_bit=8)

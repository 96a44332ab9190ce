"""Pins for the oracle's 16-bit keys and 64-bit values (no GPU).

The Silicon Studio page ("符号付型、浮動小数点型に対する radix sort") ends by
noting that 16- and 64-bit types take the same procedure as its 32-bit
rules.  Each test ties the oracle to something other than itself:
ordered keys worked out by hand from IEEE-754 binary16 and two's
complement, numpy stable sorts in the NATIVE order of the type (the float
policy written with IEEE comparisons: NaN and both infinities last, -0.0
before +0.0), brute force over short sequences of edge values, the one-bit
split as an independent algorithm, invariance under the digit width, and
64-bit payloads that must follow the native stable permutation."""
import itertools
import math

import numpy as np
import pytest

import oracle


def K(kind, bits):
    return oracle.ordered_key(kind, bits)


def test_f16_key_closed_form():
    f = oracle.KEY_F16
    assert K(f, 0x0000) == 0x8000            # +0
    assert K(f, 0x8000) == 0x7FFF            # -0
    assert K(f, 0x3C00) == 0xBC00            # 1.0
    assert K(f, 0xBC00) == 0x43FF            # -1.0
    assert K(f, 0x7BFF) == 0xFBFF            # 65504, the largest finite half
    assert K(f, 0xFBFF) == 0x0400            # -65504
    assert K(f, 0x0001) == 0x8001            # smallest subnormal
    assert K(f, 0x8001) == 0x7FFE
    for special in (0x7C00, 0xFC00, 0x7E00, 0xFE01, 0x7C01):
        assert K(f, special) == 0xFFFF       # +-Inf and NaNs: the maximum


def test_i16_u16_key_closed_form():
    assert K(oracle.KEY_I16, 0x8000) == 0    # -32768
    assert K(oracle.KEY_I16, 0xFFFF) == 0x7FFF  # -1
    assert K(oracle.KEY_I16, 0x0000) == 0x8000
    assert K(oracle.KEY_I16, 0x7FFF) == 0xFFFF  # 32767
    for u in (0, 1, 0x7FFF, 0x8000, 0xFFFF):
        assert K(oracle.KEY_U16, u) == u


def test_f16_keys_order_like_values():
    """Every finite half, in value order, gets a strictly increasing key
    (equal values -0/+0 excepted, where -0 comes first)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    finite = np.isfinite(vals)
    order = np.lexsort((~np.signbit(vals[finite]), vals[finite]))   # value, then -0 before +0
    keys = np.array([K(oracle.KEY_F16, int(b)) for b in bits[finite][order]])
    assert np.all(np.diff(keys) > 0)


def native_perm(keys, begin_bit, end_bit):
    width = end_bit - begin_bit
    if keys.dtype == np.float16:
        assert (begin_bit, end_bit) == (0, 16)
        special = np.isnan(keys) | np.isinf(keys)
        val = np.where(special, 0, keys).astype(np.float64)
        zero_pos = np.where(special, 0, np.where(np.signbit(keys), 0, 1))
        return np.lexsort((zero_pos, val, special.astype(np.int8)))
    if keys.dtype.kind == "u":
        sub = (keys.astype(np.uint64) >> np.uint64(begin_bit)) & np.uint64((1 << width) - 1)
        return np.argsort(sub, kind="stable")
    # signed: the sub-key of the ordered key, from the value with an arithmetic shift
    bits = 8 * keys.dtype.itemsize
    v = keys.astype(np.int64) + (1 << (bits - 1))                  # value - min, i.e. the ordered key
    sub = (v >> begin_bit) & ((1 << width) - 1)
    return np.argsort(sub, kind="stable")


def rand_keys(dtype, n, rng):
    if dtype == np.float16:
        x = (rng.standard_normal(n) * 100).astype(np.float16)
        sp = rng.random(n)
        x[sp < 0.02] = np.inf
        x[(sp >= 0.02) & (sp < 0.04)] = -np.inf
        x[(sp >= 0.04) & (sp < 0.06)] = np.nan
        x[(sp >= 0.06) & (sp < 0.08)] = -0.0
        x[(sp >= 0.08) & (sp < 0.10)] = 0.0
        x[(sp >= 0.10) & (sp < 0.12)] = np.float16(6e-8)            # subnormals
        return x
    info = np.iinfo(dtype)
    return rng.integers(info.min, int(info.max) + 1, n, dtype=dtype)


@pytest.mark.parametrize("dtype", [np.uint16, np.int16, np.float16])
@pytest.mark.parametrize("n", [0, 1, 7, 1000, 5000])
def test_16bit_matches_native_stable_sort(dtype, n):
    rng = np.random.default_rng(n + 5)
    keys = rand_keys(dtype, n, rng)
    vals = rng.integers(0, 2**32, n, dtype=np.uint32)
    perm = native_perm(keys, 0, 16)
    ok, ov = oracle.lsd_sort(keys, vals)
    assert np.array_equal(ok.view(np.uint16), keys[perm].view(np.uint16))
    assert np.array_equal(ov, vals[perm])


@pytest.mark.parametrize("dtype", [np.uint16, np.int16])
@pytest.mark.parametrize("bits", [(0, 8), (8, 16), (3, 13), (15, 16), (0, 1)])
def test_16bit_bit_ranges(dtype, bits):
    b, e = bits
    rng = np.random.default_rng(b * 17 + e)
    keys = rand_keys(dtype, 3000, rng)
    vals = np.arange(3000, dtype=np.uint32)
    ok, ov = oracle.lsd_sort(keys, vals, b, e)
    assert np.array_equal(ov, native_perm(keys, b, e).astype(np.uint32))


EDGE_F16 = [0.0, -0.0, 1.0, -1.0, 65504.0, -65504.0, 6e-8, float("inf"), float("-inf"), float("nan")]


def _f16_native_key(x):
    if math.isnan(x) or math.isinf(x):
        return (1, 0.0, 0)
    return (0, x, 0 if math.copysign(1.0, x) < 0 else 1)


@pytest.mark.parametrize("length", [1, 2, 3, 4])
def test_brute_force_f16_i16(length):
    for seq in itertools.product(range(len(EDGE_F16)), repeat=length):
        keys = np.array([EDGE_F16[i] for i in seq], dtype=np.float16)
        vals = np.arange(length, dtype=np.uint64) * np.uint64(0x100000001)
        want = sorted(range(length), key=lambda i: _f16_native_key(float(keys[i])))
        ok, ov = oracle.lsd_sort(keys, vals)
        assert ov.tolist() == [int(vals[i]) for i in want]
    ints = [-32768, -1, 0, 1, 32767]
    for seq in itertools.product(ints, repeat=min(length, 3)):
        keys = np.array(seq, dtype=np.int16)
        want = sorted(range(len(seq)), key=lambda i: seq[i])
        _, ov = oracle.lsd_sort(keys, np.arange(len(seq), dtype=np.uint32))
        assert ov.tolist() == want


@pytest.mark.parametrize("kdtype", [np.uint16, np.float16, np.uint32, np.int32, np.float32, np.uint64,
                                    np.int64, np.float64])
@pytest.mark.parametrize("vdtype", [np.uint64, np.int64, np.float64])
def test_64bit_values_follow_the_stable_permutation(kdtype, vdtype):
    """64-bit payloads (any bit pattern, NaN payloads included) move with
    their keys: the output values are the input values under the native
    stable permutation of the keys."""
    rng = np.random.default_rng(41)
    n = 2000
    if kdtype in (np.float32, np.float64):
        keys = (rng.standard_normal(n) * 50).astype(kdtype)
        keys[rng.random(n) < 0.05] = np.nan
    elif kdtype in (np.uint16, np.float16):
        keys = rand_keys(kdtype, n, rng)
    else:
        keys = rng.integers(np.iinfo(kdtype).min, int(np.iinfo(kdtype).max) + 1, n, dtype=kdtype)
    keys = np.concatenate([keys, keys[:300]])                       # equal keys: order by index
    vals = rng.integers(0, 2**64, keys.size, dtype=np.uint64).view(vdtype)
    width = 8 * keys.dtype.itemsize
    if kdtype in (np.float32, np.float64):
        special = np.isnan(keys) | np.isinf(keys)
        val = np.where(special, 0, keys).astype(np.float64)
        perm = np.lexsort((np.where(special, 0, np.where(np.signbit(keys), 0, 1)), val, special))
    elif keys.dtype.kind == "i":
        perm = np.argsort(keys, kind="stable")
    else:
        perm = native_perm(keys, 0, width) if kdtype in (np.uint16, np.float16) else np.argsort(keys, kind="stable")
    ok, ov = oracle.lsd_sort(keys, vals)
    assert np.array_equal(ov.view(np.uint64), vals[perm].view(np.uint64))
    assert np.array_equal(ok.view(np.uint8), keys[perm].view(np.uint8))


@pytest.mark.parametrize("dtype", [np.uint16, np.int16, np.float16])
def test_split_sort_and_width_invariance_16(dtype):
    rng = np.random.default_rng(8)
    keys = rand_keys(dtype, 1500, rng)
    vals = rng.integers(0, 2**64, 1500, dtype=np.uint64)
    ref_k, ref_v = oracle.split_sort(keys, vals)
    for r in (1, 3, 5, 8, 11, 16):
        k, v = oracle.lsd_sort(keys, vals, radix_bits=r)
        assert np.array_equal(k.view(np.uint16), ref_k.view(np.uint16)) and np.array_equal(v, ref_v)


def test_invalid_arguments_rejected():
    keys = np.zeros(4, dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.lsd_sort(keys, None, 0, 17)
    with pytest.raises(ValueError):
        oracle.lsd_sort(keys, np.zeros(4, dtype=np.uint8))

"""GPU parity for 64-bit keys (uint64, int64, float64; 32-bit values): the
HIP sort through the C ABI against the CPU oracle, bit-exact for keys and
values, at sizes spanning several tiles with ragged tails, over bit ranges up
to 64, in place, on the float and integer edge patterns, with passes that
move nothing, and (property-checked) on the 64-bit status path."""
import sys

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
rs = pytest.importorskip("lsd_radix_sort_pass_amd")

pytestmark = pytest.mark.gpu

# Keys per pass tile of the library's launch configuration for 64-bit keys.
KEY_TILE = 14336
PAIR_TILE = 11264

DTYPES = [np.uint64, np.int64, np.float64]


def note(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def assert_parity(keys, values=None, begin_bit=0, end_bit=64, in_place=False):
    note(f"dtype={keys.dtype} n={keys.size} pairs={values is not None} bits=[{begin_bit},{end_bit}) "
         f"in_place={in_place}")
    dk = to_dev(keys)
    if values is None:
        gk = rs.sort_keys(dk, begin_bit, end_bit, out=dk if in_place else None)
        gv = None
    else:
        dv = to_dev(values)
        gk, gv = rs.sort_pairs(dk, dv, begin_bit, end_bit,
                               keys_out=dk if in_place else None, values_out=dv if in_place else None)
    torch.cuda.synchronize()
    gk = gk.cpu().numpy().view(np.uint64)
    if values is None:
        ok = oracle.lsd_sort(keys, None, begin_bit, end_bit)
    else:
        ok, ov = oracle.lsd_sort(keys, values, begin_bit, end_bit)
        gv = gv.cpu().numpy()
    ob = ok.view(np.uint64)
    if not np.array_equal(gk, ob):
        bad = np.flatnonzero(gk != ob)
        raise AssertionError(f"keys differ at {bad.size} positions, first {bad[:8].tolist()}: "
                             f"gpu {[hex(x) for x in gk[bad[:4]]]} oracle {[hex(x) for x in ob[bad[:4]]]}")
    if values is not None and not np.array_equal(gv, ov):
        bad = np.flatnonzero(gv != ov)
        raise AssertionError(f"values differ at {bad.size} positions, first {bad[:8].tolist()}")


def rand_keys(dtype, n, seed):
    rng = np.random.default_rng(seed)
    if dtype == np.uint64:
        return rng.integers(0, 2**64, n, dtype=np.uint64)
    if dtype == np.int64:
        return rng.integers(-(2**63), 2**63, n, dtype=np.int64)
    # mixed signs and magnitudes over many exponents, a few specials
    x = rng.standard_normal(n) * np.exp2(rng.integers(-60, 60, n))
    sp = rng.random(n)
    x[sp < 0.002] = np.inf
    x[(sp >= 0.002) & (sp < 0.004)] = -np.inf
    x[(sp >= 0.004) & (sp < 0.006)] = np.nan
    x[(sp >= 0.006) & (sp < 0.008)] = -0.0
    x[(sp >= 0.008) & (sp < 0.010)] = 0.0
    return x.astype(np.float64)


SIZES = [2, 3, 64, 100, 4097, PAIR_TILE - 1, PAIR_TILE, PAIR_TILE + 1, KEY_TILE - 1, KEY_TILE, KEY_TILE + 1,
         3 * KEY_TILE + 1234, 11 * PAIR_TILE + 4321]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n", SIZES)
def test_keys64_random(dtype, n):
    assert_parity(rand_keys(dtype, n, seed=n + 64))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n", SIZES)
def test_pairs64_random(dtype, n):
    keys = rand_keys(dtype, n, seed=n + 65)
    assert_parity(keys, np.arange(n, dtype=np.uint32))


@pytest.mark.parametrize("bits", [(0, 32), (32, 64), (7, 61), (60, 64), (0, 8), (24, 40), (63, 64), (1, 64),
                                  (0, 63), (5, 45)])
def test_bit_ranges64(bits):
    b, e = bits
    n = 3 * KEY_TILE + 99
    vals = np.random.default_rng(b * 64 + e).integers(0, 2**32, n, dtype=np.uint32)
    assert_parity(rand_keys(np.uint64, n, seed=b * 65 + e), vals, b, e)
    assert_parity(rand_keys(np.int64, n, seed=e), None, b, e)
    assert_parity(rand_keys(np.float64, n, seed=b + 7), vals, b, e)


@pytest.mark.parametrize("dtype", DTYPES)
def test_in_place64(dtype):
    n = 4 * KEY_TILE + 5
    keys = rand_keys(dtype, n, seed=17)
    for b, e in [(0, 64), (0, 40), (8, 16)]:
        assert_parity(keys, None, b, e, in_place=True)
        assert_parity(keys, np.arange(n, dtype=np.uint32), b, e, in_place=True)


def test_edge_patterns64():
    n = 5 * KEY_TILE + 3
    rng = np.random.default_rng(55)
    ones = np.uint64(0xFFFFFFFFFFFFFFFF)
    cases = [
        np.full(n, ones, dtype=np.uint64),                              # all bits set
        np.zeros(n, dtype=np.uint64),
        np.arange(n, dtype=np.uint64),
        np.arange(n, dtype=np.uint64)[::-1].copy(),
        (np.arange(n, dtype=np.uint64) % np.uint64(2)) * ones,
        rng.integers(0, 3, n, dtype=np.uint64) << np.uint64(56),
        rng.integers(0, 2**64, n, dtype=np.uint64) | np.uint64(0xFF),     # low digit all 255
        rng.integers(0, 2**32, n, dtype=np.uint64),                     # high half zero: 4 passes move nothing
    ]
    for keys in cases:
        assert_parity(keys, np.arange(n, dtype=np.uint32))
    ints = np.array([-(2**63), 2**63 - 1, -1, 0, 1, -(2**32), 2**32, -(2**31) - 1], dtype=np.int64)
    assert_parity(ints[rng.integers(0, ints.size, n)], np.arange(n, dtype=np.uint32))
    specials = np.array([0x7FF0000000000000, 0xFFF0000000000000, 0x7FF8000000000000, 0xFFF80000DEADBEEF,
                         0x7FF0000000000001, 0x8000000000000000, 0x0000000000000000, 0x0000000000000001,
                         0x8000000000000001, 0x000FFFFFFFFFFFFF, 0x800FFFFFFFFFFFFF, 0x7FEFFFFFFFFFFFFF,
                         0xFFEFFFFFFFFFFFFF, 0x3FF0000000000000, 0xBFF0000000000000], dtype=np.uint64)
    f = specials[rng.integers(0, specials.size, n)].view(np.float64)
    assert_parity(f)
    assert_parity(f, np.arange(n, dtype=np.uint32))


def test_trivial_calls64():
    for n in [0, 1]:
        keys = rand_keys(np.uint64, n, seed=1)
        assert_parity(keys)
        assert_parity(keys, np.arange(n, dtype=np.uint32))
    keys = rand_keys(np.float64, 1000, seed=2)
    assert_parity(keys, np.arange(1000, dtype=np.uint32), 40, 40)


@pytest.mark.parametrize("case", ["small_ints", "high_const", "low_const", "all_equal", "one_byte"])
def test_trivial_passes64(case):
    """Passes in which every key has the same digit are skipped (the number
    that run decides which buffers the rest use and whether a copy follows)."""
    n = 3 * KEY_TILE + 1001
    rng = np.random.default_rng(400 + len(case))
    r = rng.integers(0, 2**64, n, dtype=np.uint64)
    keys = {
        "small_ints": r >> np.uint64(40),                                              # 5 of 8 passes trivial
        "high_const": (r & np.uint64(0xFFFFFFFF)) | np.uint64(0xABCD123400000000),
        "low_const": (r & np.uint64(0xFFFFFF0000000000)) | np.uint64(0x42),
        "all_equal": np.full(n, 0x0123456789ABCDEF, dtype=np.uint64),
        "one_byte": (r & np.uint64(0x0000FF0000000000)) | np.uint64(0x1200000000000034),
    }[case]
    vals = rng.integers(0, 2**32, n, dtype=np.uint32)
    for b, e in [(0, 64), (8, 64), (0, 48), (4, 60)]:
        assert_parity(keys, None, b, e)
        assert_parity(keys, vals, b, e)
        assert_parity(keys, None, b, e, in_place=True)
        assert_parity(keys, vals, b, e, in_place=True)
    small = rng.integers(-1000, 1000, n, dtype=np.int64)                                # signed, ordered top bytes constant
    assert_parity(small, vals)
    halves = np.where(rng.random(n) < 0.5, 2.0, -2.0)
    assert_parity(halves, np.arange(n, dtype=np.uint32), in_place=True)


@pytest.mark.parametrize("pattern", ["two_values", "all_equal", "runs"])
def test_stability64(pattern):
    n = 7 * PAIR_TILE + 4097
    rng = np.random.default_rng(800 + len(pattern))
    if pattern == "two_values":
        keys = rng.integers(0, 2, n, dtype=np.uint64) * np.uint64(0x0101010101010101)
    elif pattern == "all_equal":
        keys = np.full(n, 0x1234567890ABCDEF, dtype=np.uint64)
    else:
        keys = np.repeat(rng.integers(0, 2**64, n // 100 + 1, dtype=np.uint64), 100)[:n]
    values = np.arange(n, dtype=np.uint32)
    assert_parity(keys, values)
    assert_parity(keys, values, 8, 56)


def test_wide_status_sizes64():
    """For 64-bit keys, n >= 2^29 takes the library's 64-bit status words and
    store addresses.  The oracle is too slow at this size, so the result is
    checked through properties that together fix the stable sort uniquely:
    keys non-decreasing, values a permutation of 0..n-1, each output key equal
    to the input key its value names, equal keys in increasing value order;
    the keys-only sort must then match the pairs sort's keys."""
    n = (1 << 29) + (1 << 18) + 41
    note(f"wide status 64-bit n={n}")
    g = torch.Generator(device="cuda")
    g.manual_seed(4321)
    lo = torch.randint(0, 1 << 20, (n,), dtype=torch.int64, device="cuda", generator=g)
    golden = 0x9E3779B97F4A7C15 - (1 << 64)  # the 64-bit golden-ratio constant as a signed value
    keys = lo * golden  # about 500 copies of each key, spread over all 64 bits (the product wraps)
    del lo
    sign = torch.tensor(-(2**63), dtype=torch.int64, device="cuda")
    vals = torch.arange(n, dtype=torch.int32, device="cuda").view(torch.uint32)
    ko, vo = rs.sort_pairs(keys.view(torch.uint64), vals)
    torch.cuda.synchronize()
    ko = ko.view(torch.int64)
    chunk = 1 << 27
    seen = torch.zeros(n, dtype=torch.uint8, device="cuda")
    for s in range(0, n, chunk):
        e = min(n, s + chunk + 1)
        k = ko[s:e] ^ sign  # signed order of this view = unsigned order of the keys
        v = vo[s:e].view(torch.int32).to(torch.int64)
        assert bool((k[1:] >= k[:-1]).all()), f"keys out of order in [{s}, {e})"
        same = k[1:] == k[:-1]
        assert bool((v[1:][same] > v[:-1][same]).all()), f"equal keys out of input order in [{s}, {e})"
        assert bool((keys[v] == ko[s:e]).all()), "key/value mismatch"
        seen[v[: min(chunk, n - s)]] = 1
    assert bool(seen.all()), "values are not a permutation"
    del seen, vo, vals
    ko2 = rs.sort_keys(keys.view(torch.uint64))
    torch.cuda.synchronize()
    assert torch.equal(ko2.view(torch.int64), ko)




@pytest.mark.parametrize("dtype", DTYPES)
def test_already_sorted64(dtype):
    """Sorted 64-bit keys skip every pass; an inversion at the wave edge, the
    tile edge or the very end is still sorted."""
    n = 5 * KEY_TILE + 555  # above the one-launch path's limit (the flag is the multi-launch path's)
    keys = oracle.lsd_sort(rand_keys(dtype, n, seed=77))  # in ordered-key order (-Inf, NaN last, -0 < +0)
    for i, is_sorted in [(None, True), (63, False), (KEY_TILE - 1, False), (n - 2, False)]:
        k = keys.copy()
        if i is not None:
            k[i], k[i + 1] = k[i + 1], k[i]
            if oracle.ordered_key(oracle.kind_of(k.dtype), int(k[i:i + 1].view(np.uint64)[0])) == \
               oracle.ordered_key(oracle.kind_of(k.dtype), int(k[i + 1:i + 2].view(np.uint64)[0])):
                continue  # equal keys: swapping them changes nothing
        temp = rs.alloc_temp(n, True, 0, 64, device="cuda", key_dtype=to_dev(k[:1]).dtype)
        note(f"sorted64 {k.dtype} swap {i}")
        ko, vo = rs.sort_pairs(to_dev(k), to_dev(np.arange(n, dtype=np.uint32)), temp=temp)
        torch.cuda.synchronize()
        flag = rs.order_flag(temp)
        assert flag == (0 if is_sorted else 1)
        ek, ev = oracle.lsd_sort(k, np.arange(n, dtype=np.uint32))
        assert np.array_equal(ko.cpu().numpy().view(np.uint64), ek.view(np.uint64))
        assert np.array_equal(vo.cpu().numpy(), ev)

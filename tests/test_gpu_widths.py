"""GPU parity for 16-bit keys (uint16, int16, float16) and for 64-bit values
with every key width: the HIP sort through the C ABI against the CPU
oracle, bit-exact for keys and values, on both the one-launch path (up to
65536 keys) and the multi-launch path, around the tile sizes of each
combination, over bit ranges, in place, with float specials, passes that
move nothing, already-sorted input, heavy duplicates, and (property
checked) the 64-bit status path that 64-bit values take from 2^29 keys."""
import sys

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
rs = pytest.importorskip("lsd_radix_sort_pass_amd")

pytestmark = pytest.mark.gpu

SMALL_MAX = 65536   # largest input of the one-launch path

TORCH_OF = {np.dtype(np.uint16): torch.uint16, np.dtype(np.int16): torch.int16,
            np.dtype(np.float16): torch.float16}


def note(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def word_view(a):
    return a.view({2: np.uint16, 4: np.uint32, 8: np.uint64}[a.dtype.itemsize])


def run(keys, values=None, b=0, e=None, in_place=False):
    e = 8 * keys.dtype.itemsize if e is None else e
    note(f"widths dtype={keys.dtype} n={keys.size} values={None if values is None else values.dtype} "
         f"bits=[{b},{e}) in_place={in_place}")
    dk = torch.from_numpy(np.ascontiguousarray(keys)).to("cuda")
    vb = 0 if values is None else values.dtype.itemsize
    temp = rs.alloc_temp(keys.size, values is not None, b, e, device="cuda", key_dtype=dk.dtype,
                         value_bytes=vb or 4)
    if values is None:
        ko = rs.sort_keys(dk, b, e, out=dk if in_place else None, temp=temp)
    else:
        dv = torch.from_numpy(np.ascontiguousarray(values)).to("cuda")
        ko, vo = rs.sort_pairs(dk, dv, b, e, keys_out=dk if in_place else None,
                               values_out=dv if in_place else None, temp=temp)
    torch.cuda.synchronize()
    assert rs.error_word(temp) == 0
    if values is None:
        ek = oracle.lsd_sort(keys, None, b, e)
    else:
        ek, ev = oracle.lsd_sort(keys, values, b, e)
        got_v = vo.cpu().numpy()
        if not np.array_equal(word_view(got_v), word_view(ev)):
            bad = np.flatnonzero(word_view(got_v) != word_view(ev))
            raise AssertionError(f"values differ at {bad.size} positions, first {bad[:6].tolist()}")
    got_k = ko.cpu().numpy()
    if not np.array_equal(word_view(got_k), word_view(ek)):
        bad = np.flatnonzero(word_view(got_k) != word_view(ek))
        raise AssertionError(f"keys differ at {bad.size} positions, first {bad[:6].tolist()}: "
                             f"gpu {word_view(got_k)[bad[:4]].tolist()} oracle {word_view(ek)[bad[:4]].tolist()}")


def keys_of(dtype, n, seed):
    rng = np.random.default_rng(seed)
    if dtype == np.float16:
        x = (rng.standard_normal(n) * 300).astype(np.float16)
        sp = rng.random(n)
        x[sp < 0.01] = np.inf
        x[(sp >= 0.01) & (sp < 0.02)] = -np.inf
        x[(sp >= 0.02) & (sp < 0.03)] = np.nan
        x[(sp >= 0.03) & (sp < 0.04)] = -0.0
        x[(sp >= 0.04) & (sp < 0.05)] = np.float16(3e-7)   # subnormal
        return x
    if dtype == np.float32:
        return (rng.standard_normal(n) * 1000).astype(np.float32)
    if dtype == np.float64:
        return rng.standard_normal(n) * 1e6
    info = np.iinfo(dtype)
    return rng.integers(info.min, int(info.max) + 1, n, dtype=dtype)


def payload64(n, seed, dtype=np.uint64):
    return np.random.default_rng(seed).integers(0, 2**64, n, dtype=np.uint64).view(dtype)


K16 = [np.uint16, np.int16, np.float16]
SIZES16 = [2, 3, 100, 4097, SMALL_MAX, SMALL_MAX + 1, 17407, 28672 + 1, 3 * 28672 + 77, 7 * 17408 + 5, 3 * 11264 + 7]


@pytest.mark.parametrize("dtype", K16)
@pytest.mark.parametrize("n", SIZES16)
def test_16bit_keys_and_pairs(dtype, n):
    keys = keys_of(dtype, n, seed=n + 160)
    run(keys)
    run(keys, np.arange(n, dtype=np.uint32))
    run(keys, payload64(n, n))


@pytest.mark.parametrize("dtype", K16)
@pytest.mark.parametrize("bits", [(0, 8), (8, 16), (3, 13), (15, 16), (0, 1)])
def test_16bit_bit_ranges_in_place(dtype, bits):
    b, e = bits
    for n in (20000, 150000):                     # one-launch and multi-launch paths
        keys = keys_of(dtype, n, seed=b * 16 + e + n)
        run(keys, None, b, e)
        run(keys, np.arange(n, dtype=np.uint32), b, e, in_place=True)
        run(keys, payload64(n, e), b, e, in_place=True)


def test_f16_specials_and_duplicates():
    n = 200000
    rng = np.random.default_rng(7)
    specials = np.array([0x7C00, 0xFC00, 0x7E00, 0xFE01, 0x7C01, 0x8000, 0x0000, 0x0001, 0x8001, 0x7BFF,
                         0xFBFF, 0x3C00, 0xBC00], dtype=np.uint16)
    f = specials[rng.integers(0, specials.size, n)].view(np.float16)
    run(f)
    run(f, np.arange(n, dtype=np.uint32))
    run(f[:40000], payload64(40000, 3), in_place=True)
    run(np.full(n, 7, dtype=np.uint16), np.arange(n, dtype=np.uint32))       # every pass trivial
    run((rng.integers(0, 256, n, dtype=np.uint16)), np.arange(n, dtype=np.uint32))  # high byte trivial
    run(np.sort(keys_of(np.uint16, n, 9)), payload64(n, 9))                   # already sorted


KEYS_ALL = [np.uint16, np.int16, np.float16, np.uint32, np.int32, np.float32, np.uint64, np.int64, np.float64]


@pytest.mark.parametrize("kdtype", KEYS_ALL)
@pytest.mark.parametrize("n", [2, 1000, 8193, SMALL_MAX, SMALL_MAX + 3, 11264 * 3 + 11, 8192 * 9 + 1])
def test_64bit_values(kdtype, n):
    keys = keys_of(kdtype, n, seed=n + 640)
    run(keys, payload64(n, n + 1))
    run(keys, payload64(n, n + 2, np.float64))           # NaN payloads among the bit patterns


@pytest.mark.parametrize("kdtype", [np.uint32, np.float64, np.int16])
def test_64bit_values_in_place_ranges_duplicates(kdtype):
    n = 5 * 11264 + 999 + SMALL_MAX
    rng = np.random.default_rng(11)
    keys = keys_of(kdtype, n, seed=12)
    width = 8 * keys.dtype.itemsize
    for b, e in [(0, width), (0, 8), (width - 8, width), (3, width - 3)]:
        run(keys, payload64(n, b + e), b, e, in_place=True)
    dup = keys[rng.integers(0, 20, n)]                       # 20 distinct keys
    run(dup, np.arange(n, dtype=np.uint64))
    run(dup[:30000], np.arange(30000, dtype=np.uint64), in_place=True)


def test_64bit_values_wide_status():
    """From 2^29 keys, 64-bit values take the 64-bit status words and store
    addresses.  Checked by properties (the oracle is too slow here): keys
    non-decreasing, values a permutation of 0..n-1 (as 64-bit values), each
    output key the input key its value names, equal keys in increasing
    value order; the keys-only sort must give the same keys."""
    n = (1 << 29) + (1 << 16) + 3
    note(f"wide 64-bit values n={n}")
    g = torch.Generator(device="cuda")
    g.manual_seed(99)
    keys = (torch.randint(0, 1 << 20, (n,), dtype=torch.int32, device="cuda", generator=g) * 4099).view(torch.uint32)
    vals = torch.arange(n, dtype=torch.int64, device="cuda")
    ko, vo = rs.sort_pairs(keys, vals)
    torch.cuda.synchronize()
    sign = torch.tensor(-(2**31), dtype=torch.int32, device="cuda")
    chunk = 1 << 27
    seen = torch.zeros(n, dtype=torch.uint8, device="cuda")
    for s in range(0, n, chunk):
        e = min(n, s + chunk + 1)
        k = ko[s:e].view(torch.int32) ^ sign
        v = vo[s:e]
        assert bool((k[1:] >= k[:-1]).all()), f"keys out of order in [{s}, {e})"
        same = k[1:] == k[:-1]
        assert bool((v[1:][same] > v[:-1][same]).all()), f"equal keys out of input order in [{s}, {e})"
        assert bool((keys.view(torch.int32)[v] == ko[s:e].view(torch.int32)).all()), "key/value mismatch"
        seen[v[: min(chunk, n - s)]] = 1
    assert bool(seen.all()), "values are not a permutation"
    del seen, vo, vals
    ko2 = rs.sort_keys(keys)
    torch.cuda.synchronize()
    assert torch.equal(ko2.view(torch.int32), ko.view(torch.int32))


@pytest.mark.parametrize("kdtype", [np.uint16, np.uint32, np.uint64])
@pytest.mark.parametrize("shift", [0, 1, 3])
def test_skipped_passes_copy_at_any_alignment(kdtype, shift):
    """When every pass is skipped the output is a copy of the input, made
    with 16-byte accesses when both buffers allow it and element by element
    otherwise: views shifted by 0, 1 or 3 elements, sizes with a ragged
    tail, keys only and pairs, in place (the odd-count copy back) and not."""
    n = 5 * 28672 + 13
    rng = np.random.default_rng(int(shift) + 8 * np.dtype(kdtype).itemsize)
    keys = np.sort(keys_of(kdtype, n, seed=shift))                 # already in order
    vals = rng.integers(0, 2**32, n + shift, dtype=np.uint32)
    note(f"skipped-pass copy dtype={np.dtype(kdtype)} shift={shift} n={n}")
    padded = np.concatenate([np.zeros(shift, dtype=kdtype), keys])
    for in_place in (False, True):
        dk = torch.from_numpy(padded.copy()).to("cuda")[shift:]
        dv = torch.from_numpy(vals.copy()).to("cuda")[shift:]
        ko = rs.sort_keys(dk, out=dk if in_place else None)
        torch.cuda.synchronize()
        assert np.array_equal(word_view(ko.cpu().numpy()), word_view(keys))
        dk = torch.from_numpy(padded.copy()).to("cuda")[shift:]
        ko, vo = rs.sort_pairs(dk, dv, keys_out=dk if in_place else None, values_out=dv if in_place else None)
        torch.cuda.synchronize()
        assert np.array_equal(word_view(ko.cpu().numpy()), word_view(keys))
        assert np.array_equal(vo.cpu().numpy(), vals[shift:])
    # one pass skipped, one run: in place with an odd executed count copies back
    low = (keys_of(np.uint32, n, seed=5) & np.uint32(0xFF)).astype(kdtype)
    run(low, np.arange(n, dtype=np.uint32), in_place=True)


@pytest.mark.parametrize("dtype", [np.uint16, np.int16, np.uint64, np.float64])
@pytest.mark.parametrize("where", ["none", "in_lane", "lane_end", "wave_end", "row_end", "last"])
def test_order_check_wide_and_narrow_layouts(dtype, where):
    """The histogram kernel's order check loads V = 16 / key bytes
    consecutive keys per lane (8 for 16-bit keys, 2 for 64-bit keys):
    sorted keys skip every pass, and one descent inside a lane's run, at a
    run's end, at the end of a wave's part of a row, at a row's end or at
    the input's end is found."""
    dtype = np.dtype(dtype)
    v = 16 // dtype.itemsize
    n = 3 * SMALL_MAX + 777
    rng = np.random.default_rng(700 + v + len(where))
    if dtype.kind == "f":
        keys = np.sort(rng.standard_normal(n) * 100.0).astype(dtype)
    else:
        info = np.iinfo(dtype)
        keys = np.sort(rng.integers(info.min, info.max, n, dtype=dtype, endpoint=True))
    at = {"none": None, "in_lane": 0, "lane_end": v - 1, "wave_end": 64 * v - 1, "row_end": 1024 * v - 1,
          "last": n - 2}[where]
    if at is not None:
        # the key after `at` one step below it: the only descent
        if dtype.kind == "f":
            keys[at + 1] = np.nextafter(keys[at], dtype.type(-np.inf))
        else:
            if keys[at] == np.iinfo(dtype).min:
                keys[at] += dtype.type(1)
            keys[at + 1] = keys[at] - dtype.type(1)
    note(f"order check dtype={dtype} where={where} at={at}")
    dk = torch.from_numpy(keys.copy()).to("cuda")
    temp = rs.alloc_temp(n, False, 0, 8 * dtype.itemsize, device="cuda", key_dtype=dk.dtype)
    out = rs.sort_keys(dk, temp=temp)
    torch.cuda.synchronize()
    assert rs.order_flag(temp) == (0 if at is None else 1)
    assert np.array_equal(word_view(out.cpu().numpy()), word_view(oracle.lsd_sort(keys)))

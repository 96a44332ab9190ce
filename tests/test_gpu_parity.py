"""GPU parity: the HIP sort (through the C ABI) against the CPU oracle,
bit-exact for keys and values, on seeded inputs shaped like the workloads,
at sizes spanning several tiles with a ragged tail, at full workload sizes,
and on edge cases."""
import sys

import numpy as np
import pytest

import oracle
from lsd_radix_sort_pass_amd import workloads

torch = pytest.importorskip("torch")
rs = pytest.importorskip("lsd_radix_sort_pass_amd")

pytestmark = pytest.mark.gpu

# Keys per pass tile of the library's launch configuration: keys-only sorts
# and key-value sorts use different tile sizes.
KEY_TILE = 28672
PAIR_TILE = 17408
TILE = KEY_TILE

NP_TO_TORCH = {np.dtype(np.uint32): torch.uint32, np.dtype(np.int32): torch.int32,
               np.dtype(np.float32): torch.float32}


def note(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def gpu_sort(keys, values=None, begin_bit=0, end_bit=32, in_place=False, temp=None):
    dk = to_dev(keys)
    if values is None:
        out = rs.sort_keys(dk, begin_bit, end_bit, out=dk if in_place else None, temp=temp)
        torch.cuda.synchronize()
        return out.cpu().numpy(), None
    dv = to_dev(values)
    ko, vo = rs.sort_pairs(dk, dv, begin_bit, end_bit,
                           keys_out=dk if in_place else None, values_out=dv if in_place else None,
                           temp=temp)
    torch.cuda.synchronize()
    return ko.cpu().numpy(), vo.cpu().numpy()


def assert_parity(keys, values=None, begin_bit=0, end_bit=32, **kw):
    note(f"dtype={keys.dtype} n={keys.size} pairs={values is not None} bits=[{begin_bit},{end_bit}) {kw}")
    gk, gv = gpu_sort(keys, values, begin_bit, end_bit, **kw)
    if values is None:
        ok = oracle.lsd_sort(keys, None, begin_bit, end_bit)
    else:
        ok, ov = oracle.lsd_sort(keys, values, begin_bit, end_bit)
    word = {2: np.uint16, 4: np.uint32, 8: np.uint64}[keys.dtype.itemsize]
    gb, ob = gk.view(word), ok.view(word)
    if not np.array_equal(gb, ob):
        bad = np.flatnonzero(gb != ob)
        raise AssertionError(f"keys differ at {bad.size} positions, first {bad[:8].tolist()}: "
                             f"gpu {gb[bad[:8]].tolist()} oracle {ob[bad[:8]].tolist()}")
    if values is not None:
        if not np.array_equal(gv, ov):
            bad = np.flatnonzero(gv != ov)
            raise AssertionError(f"values differ at {bad.size} positions, first {bad[:8].tolist()}")


def rand_keys(dtype, n, seed):
    rng = np.random.default_rng(seed)
    if dtype == np.uint32:
        return rng.integers(0, 2**32, n, dtype=np.uint32)
    if dtype == np.int32:
        return rng.integers(-(2**31), 2**31, n, dtype=np.int32)
    return workloads.make("gauss_f32_2^24", n=n, seed=seed)[0]


SIZES = [2, 3, 64, 100, 4097, PAIR_TILE - 1, PAIR_TILE, PAIR_TILE + 1, KEY_TILE - 1, KEY_TILE, KEY_TILE + 1,
         3 * KEY_TILE + 1234, 17 * PAIR_TILE + 4321]


@pytest.mark.parametrize("dtype", [np.uint32, np.int32, np.float32])
@pytest.mark.parametrize("n", SIZES)
def test_keys_random(dtype, n):
    assert_parity(rand_keys(dtype, n, seed=n))


@pytest.mark.parametrize("dtype", [np.uint32, np.int32, np.float32])
@pytest.mark.parametrize("n", SIZES)
def test_pairs_random(dtype, n):
    keys = rand_keys(dtype, n, seed=n + 1)
    assert_parity(keys, np.arange(n, dtype=np.uint32))


@pytest.mark.parametrize("dtype", [np.int32, np.float32])
def test_pairs_signed_and_float_bit_ranges(dtype):
    n = 3 * PAIR_TILE + 555
    keys = rand_keys(dtype, n, seed=91)
    vals = np.random.default_rng(92).integers(0, 2**32, n, dtype=np.uint32)  # arbitrary payloads
    for b, e in [(0, 32), (0, 8), (24, 32), (3, 29), (31, 32)]:
        assert_parity(keys, vals, b, e)
    assert_parity(keys, vals, 0, 32, in_place=True)


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_workload_shapes_small(name):
    n = 9 * TILE + 777
    keys, values, b, e = workloads.make(name, n=n)
    assert_parity(keys, values, b, e)


@pytest.mark.parametrize("bits", [(0, 8), (8, 16), (3, 29), (0, 30), (24, 32), (0, 1),
                                  (5, 13), (16, 32), (31, 32), (0, 24), (1, 32)])
def test_bit_ranges(bits):
    b, e = bits
    n = 5 * TILE + 99
    keys = rand_keys(np.uint32, n, seed=b * 64 + e)
    assert_parity(keys, np.arange(n, dtype=np.uint32), b, e)
    assert_parity(rand_keys(np.int32, n, seed=e), None, b, e)
    assert_parity(rand_keys(np.float32, n, seed=b), None, b, e)


@pytest.mark.parametrize("bits", [(0, 32), (0, 24), (8, 16), (0, 30)])
def test_in_place(bits):
    b, e = bits
    n = 4 * TILE + 5
    keys = rand_keys(np.uint32, n, seed=7)
    assert_parity(keys, None, b, e, in_place=True)
    assert_parity(keys, np.arange(n, dtype=np.uint32), b, e, in_place=True)


def test_edge_patterns():
    n = 6 * TILE + 3
    rng = np.random.default_rng(5)
    cases = [
        np.full(n, 0xFFFFFFFF, dtype=np.uint32),          # real keys equal to a pad sentinel
        np.zeros(n, dtype=np.uint32),
        np.arange(n, dtype=np.uint32),
        np.arange(n, dtype=np.uint32)[::-1].copy(),
        (np.arange(n, dtype=np.uint32) % 2) * np.uint32(0xFFFFFFFF),
        rng.integers(0, 3, n, dtype=np.uint32) << np.uint32(24),
        rng.integers(0, 2**32, n, dtype=np.uint32) | np.uint32(0xFF),   # low digit all 255
    ]
    for keys in cases:
        assert_parity(keys, np.arange(n, dtype=np.uint32))
    specials = np.array([0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC0BEEF, 0x7F800001,
                         0x80000000, 0x00000000, 0x00000001, 0x80000001], dtype=np.uint32)
    f = specials[rng.integers(0, specials.size, n)].view(np.float32)
    assert_parity(f)


def test_trivial_calls():
    for n in [0, 1]:
        keys = rand_keys(np.uint32, n, seed=1)
        assert_parity(keys)
        assert_parity(keys, np.arange(n, dtype=np.uint32))
    keys = rand_keys(np.uint32, 1000, seed=2)
    assert_parity(keys, np.arange(1000, dtype=np.uint32), 9, 9)


def test_unaligned_views_and_reused_temp():
    n = 3 * TILE + 17
    base = rand_keys(np.uint32, n + 1, seed=9)
    dk = to_dev(base)[1:]                       # 4-byte aligned, not 16
    temp = rs.alloc_temp(n, True, 0, 32, device=dk.device)
    temp.fill_(0xAB)                            # garbage scan state must not matter
    note("unaligned view, dirty temp")
    out = rs.sort_keys(dk, temp=temp)
    torch.cuda.synchronize()
    expect = oracle.lsd_sort(base[1:])
    assert np.array_equal(out.cpu().numpy(), expect)
    assert rs.error_word(temp) == 0
    vals = np.arange(n, dtype=np.uint32)
    for _ in range(3):                          # repeat: deterministic, temp reused
        ko, vo = rs.sort_pairs(dk, to_dev(vals), temp=temp)
        torch.cuda.synchronize()
        ek, ev = oracle.lsd_sort(base[1:], vals)
        assert np.array_equal(ko.cpu().numpy(), ek) and np.array_equal(vo.cpu().numpy(), ev)
        assert rs.error_word(temp) == 0


@pytest.mark.parametrize("swap", [None, 63, 4095, 9727])
def test_unaligned_view_order_check(swap):
    """Sorted keys in a view that is not 16-byte aligned (the histogram then
    loads them one by one in its 16-byte layout): no pass runs, and one
    inversion at a lane end or a row end of that layout is still found."""
    n = 3 * KEY_TILE + 4321
    rng = np.random.default_rng(77)
    base = np.sort(rng.integers(0, 2**32, n + 1, dtype=np.uint32))
    keys = base[1:].copy()
    if swap is not None:
        if keys[swap] == keys[swap + 1]:
            keys[swap + 1] += np.uint32(1)
        keys[swap], keys[swap + 1] = keys[swap + 1], keys[swap]
    padded = np.concatenate([base[:1], keys])
    dk = to_dev(padded)[1:]
    note(f"unaligned view order check swap={swap}")
    temp = rs.alloc_temp(n, False, 0, 32, device=dk.device)
    out = rs.sort_keys(dk, temp=temp)
    torch.cuda.synchronize()
    assert rs.order_flag(temp) == (0 if swap is None else 1)
    assert np.array_equal(out.cpu().numpy(), oracle.lsd_sort(keys))


def test_stream_ordering():
    n = 2 * TILE + 3
    keys = rand_keys(np.int32, n, seed=4)
    s = torch.cuda.Stream()
    dk = to_dev(keys)
    torch.cuda.synchronize()
    note("side stream")
    with torch.cuda.stream(s):
        out = rs.sort_keys(dk)
    s.synchronize()
    assert np.array_equal(out.cpu().numpy(), oracle.lsd_sort(keys))


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_workload_full_size(name):
    keys, values, b, e = workloads.make(name)
    assert_parity(keys, values, b, e)


STABILITY_PATTERNS = ["two_values", "all_equal", "one_hot_digit", "runs", "skewed_bytes"]


@pytest.mark.parametrize("pattern", STABILITY_PATTERNS)
def test_stability_heavy_duplicates(pattern):
    """Equal keys must keep their input order (values carry the input index):
    whole waves, slots and tiles of one digit stress the within-wave rank
    order."""
    n = 7 * 2 * TILE + 4097
    rng = np.random.default_rng(700 + STABILITY_PATTERNS.index(pattern))
    if pattern == "two_values":
        keys = rng.integers(0, 2, n, dtype=np.uint32) * np.uint32(0x01010101)
    elif pattern == "all_equal":
        keys = np.full(n, 0x12345678, dtype=np.uint32)
    elif pattern == "one_hot_digit":
        keys = (np.uint32(1) << rng.integers(0, 32, n, dtype=np.uint32)).astype(np.uint32)
    elif pattern == "runs":
        keys = np.repeat(rng.integers(0, 2**32, n // 100 + 1, dtype=np.uint32), 100)[:n]
    else:
        keys = (rng.integers(0, 4, n, dtype=np.uint32) * np.uint32(0x40404040)) ^ np.uint32(0x00FF0000)
    values = np.arange(n, dtype=np.uint32)
    assert_parity(keys, values)
    assert_parity(keys, values, 8, 24)


def _ordered_i32(t):
    """Signed view whose order is the unsigned order of the 32-bit words."""
    return t.view(torch.int32) ^ torch.tensor(-(2**31), dtype=torch.int32, device=t.device)


def test_wide_status_sizes():
    """n >= 2^30 takes the library's 64-bit status words and 64-bit store
    addresses.  The CPU oracle is too slow at this size, so the result is
    checked through properties that together fix the stable sort uniquely:
    output keys non-decreasing; output values a permutation of 0..n-1; each
    output key equal to the input key its value points to; equal keys in
    increasing value order.  The keys-only sort must then match the pairs
    sort's keys bit for bit."""
    n = (1 << 30) + (1 << 20) + 37
    note(f"wide status n={n}")
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    keys = torch.randint(0, 1 << 20, (n,), dtype=torch.int32, device="cuda", generator=g)
    keys = (keys * 4099).view(torch.uint32)  # duplicates (about 1000 per key) spread over all digits
    vals = torch.arange(n, dtype=torch.int32, device="cuda").view(torch.uint32)
    ko, vo = rs.sort_pairs(keys, vals)
    torch.cuda.synchronize()
    chunk = 1 << 28
    seen = torch.zeros(n, dtype=torch.uint8, device="cuda")
    for s in range(0, n, chunk):
        e = min(n, s + chunk + 1)
        k = _ordered_i32(ko[s:e])
        v = vo[s:e].view(torch.int32).to(torch.int64)
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


def _trivial_cases(n, rng):
    r = lambda: rng.integers(0, 2**32, n, dtype=np.uint32)
    return {
        "low_byte_const": (r() & np.uint32(0xFFFFFF00)) | np.uint32(0x5A),          # pass 0 moves nothing
        "high_byte_const": r() & np.uint32(0x00FFFFFF),                            # last pass moves nothing
        "middle_const": (r() & np.uint32(0xFF0000FF)) | np.uint32(0x00ABCD00),       # passes 1 and 2
        "all_equal": np.full(n, 0xDEADBEEF, dtype=np.uint32),                       # no pass runs
        "one_varying_byte": (r() & np.uint32(0x0000FF00)) | np.uint32(0x12000034),   # only pass 1 runs
    }


@pytest.mark.parametrize("case", ["low_byte_const", "high_byte_const", "middle_const", "all_equal", "one_varying_byte"])
def test_trivial_passes_skipped(case):
    """Passes in which every key has the same digit are skipped; the buffers
    the remaining passes use, and the final copy, depend on how many run."""
    n = 3 * KEY_TILE + 1001
    rng = np.random.default_rng(300 + len(case))
    keys = _trivial_cases(n, rng)[case]
    vals = rng.integers(0, 2**32, n, dtype=np.uint32)
    for b, e in [(0, 32), (8, 32), (0, 16), (4, 28)]:
        assert_parity(keys, None, b, e)
        assert_parity(keys, vals, b, e)
        assert_parity(keys, None, b, e, in_place=True)
        assert_parity(keys, vals, b, e, in_place=True)


@pytest.mark.parametrize("case", ["low_byte_const", "high_byte_const", "middle_const", "one_varying_byte"])
def test_skip_flags_match_constant_digits(case):
    """The library's per-pass skip flags are set exactly for the passes
    whose digit is the same for every key (the keys are not in order, so
    the already-sorted exit does not apply)."""
    n = 3 * KEY_TILE + 1001
    rng = np.random.default_rng(300 + len(case))
    keys = _trivial_cases(n, rng)[case]
    assert np.any(keys[1:] < keys[:-1])
    temp = rs.alloc_temp(n, False, 0, 32, device="cuda")
    out = rs.sort_keys(to_dev(keys), temp=temp)
    torch.cuda.synchronize()
    want = [int(np.unique((keys >> np.uint32(8 * p)) & np.uint32(0xFF)).size == 1) for p in range(4)]
    assert rs.skipped_passes(temp, 4) == want and rs.order_flag(temp) == 1
    assert np.array_equal(out.cpu().numpy(), oracle.lsd_sort(keys))


def test_trivial_passes_signed_and_float():
    n = 2 * KEY_TILE + 77
    rng = np.random.default_rng(41)
    small = rng.integers(0, 1 << 20, n, dtype=np.int32)                            # ordered top byte constant
    assert_parity(small)
    assert_parity(small, np.arange(n, dtype=np.uint32), in_place=True)
    ones = np.full(n, 1.0, dtype=np.float32)                                         # every pass trivial
    assert_parity(ones)
    assert_parity(ones, np.arange(n, dtype=np.uint32))
    halves = np.where(rng.random(n) < 0.5, np.float32(2.0), np.float32(-2.0)).astype(np.float32)
    assert_parity(halves, np.arange(n, dtype=np.uint32), in_place=True)


# The library's order flag (rs.order_flag) lets the tests see that the
# already-sorted path is taken exactly when the input is in sub-key order.
# The flag belongs to the multi-launch path: inputs of more than 65536 keys.


def _sorted_cases(n, rng):
    base = np.sort(rng.integers(0, 2**32, n, dtype=np.uint32))
    cases = {"sorted": (base, True), "sorted_dups": (np.sort(rng.integers(0, 100, n, dtype=np.uint32)), True),
             "descending": (base[::-1].copy(), False), "all_equal": (np.full(n, 7, dtype=np.uint32), True)}
    # one adjacent inversion at places the kernels split the keys: wave
    # edges, the histogram's 1024-key units and its workgroup chunks (here
    # 14336 keys: each 28672-key pass-0 segment split in two), pass tiles,
    # the two ends (and, in a unit's layout of 4 consecutive keys per lane
    # and 256-key rows, in-lane pairs, lane ends and row ends)
    for i in [0, 63, 1023, 16383, KEY_TILE - 1, PAIR_TILE - 1, n // 2, n - 2, 5 * 1024 + 63, 7 * 1024 + 1023,
              16384 + 15 * 1024 + 9 * 64 + 63, 4098, 2 * 4096 + 5 * 256 + 255, 3 * 4096 + 255,
              14 * 1024 - 1, KEY_TILE + 14 * 1024 - 1]:
        k = base.copy()
        if k[i] == k[i + 1]:
            k[i + 1] += np.uint32(1)
        k[i], k[i + 1] = k[i + 1], k[i]
        cases[f"swap_{i}"] = (k, False)
    return cases


@pytest.mark.parametrize("case", ["sorted", "sorted_dups", "descending", "all_equal", "swap_0", "swap_63",
                                  "swap_1023", "swap_16383", f"swap_{KEY_TILE - 1}", f"swap_{PAIR_TILE - 1}",
                                  "swap_mid", "swap_last", "swap_5183", "swap_8191", "swap_32383",
                                  "swap_4098", "swap_9727", "swap_12543", "swap_14335", "swap_43007"])
def test_already_sorted_inputs(case):
    """An input already in sub-key order skips every pass; one adjacent
    inversion anywhere must still be sorted."""
    n = 3 * KEY_TILE + 4321
    rng = np.random.default_rng(900)
    cases = _sorted_cases(n, rng)
    name = {"swap_mid": f"swap_{n // 2}", "swap_last": f"swap_{n - 2}"}.get(case, case)
    keys, is_sorted = cases[name]
    vals = np.arange(n, dtype=np.uint32)
    for pairs in (False, True):
        for in_place in (False, True):
            note(f"sorted check {case} pairs={pairs} in_place={in_place}")
            temp = rs.alloc_temp(n, pairs, 0, 32, device="cuda")
            dk = to_dev(keys)
            if pairs:
                dv = to_dev(vals)
                ko, vo = rs.sort_pairs(dk, dv, keys_out=dk if in_place else None,
                                       values_out=dv if in_place else None, temp=temp)
            else:
                ko = rs.sort_keys(dk, out=dk if in_place else None, temp=temp)
            torch.cuda.synchronize()
            flag = rs.order_flag(temp)
            assert flag == (0 if is_sorted else 1), f"unsorted flag {flag} for {case}"
            if pairs:
                ek, ev = oracle.lsd_sort(keys, vals)
                assert np.array_equal(ko.cpu().numpy(), ek) and np.array_equal(vo.cpu().numpy(), ev)
            else:
                assert np.array_equal(ko.cpu().numpy(), oracle.lsd_sort(keys))


def test_sorted_by_sub_key_only():
    """Keys whose bits [8, 16) never decrease (other bits random) are in
    order for that bit range: the sort returns them unchanged; for the full
    range they are not sorted."""
    n = 3 * KEY_TILE + 999  # above the one-launch path's limit (the flag is the multi-launch path's)
    rng = np.random.default_rng(901)
    mid = np.sort(rng.integers(0, 256, n, dtype=np.uint32))
    keys = (rng.integers(0, 2**32, n, dtype=np.uint32) & np.uint32(0xFFFF00FF)) | (mid << np.uint32(8))
    for b, e, is_sorted in [(8, 16, True), (8, 12, False), (0, 32, False), (12, 16, False)]:
        temp = rs.alloc_temp(n, True, b, e, device="cuda")
        note(f"sub-key order bits [{b},{e})")
        ko, vo = rs.sort_pairs(to_dev(keys), to_dev(np.arange(n, dtype=np.uint32)), b, e, temp=temp)
        torch.cuda.synchronize()
        flag = rs.order_flag(temp)
        ek, ev = oracle.lsd_sort(keys, np.arange(n, dtype=np.uint32), b, e)
        assert np.array_equal(ko.cpu().numpy(), ek) and np.array_equal(vo.cpu().numpy(), ev)
        if is_sorted:
            assert flag == 0 and np.array_equal(ek, keys)
        elif not np.array_equal(ek, keys):
            assert flag == 1


def test_sorted_floats_signed_zero_and_nan():
    """numpy's float order treats -0.0 and +0.0 as equal and puts NaN last;
    the ordered key puts -0.0 first and NaN/Inf at the maximum, so such an
    input is already sorted only without +0.0 before -0.0."""
    n = KEY_TILE + 777
    rng = np.random.default_rng(902)
    x = np.sort(np.concatenate([rng.standard_normal(n - 40), np.zeros(20), -np.zeros(20)]).astype(np.float32))
    assert_parity(x)
    assert_parity(x, np.arange(n, dtype=np.uint32))
    y = np.sort(rng.standard_normal(n).astype(np.float32))
    y[-5:] = np.float32(np.inf)
    y[-3:] = np.float32(np.nan)          # Inf and NaN share the maximum key: in order
    assert_parity(y)
    i64 = np.sort(rng.integers(-(2**63), 2**63, n, dtype=np.int64))
    assert_parity(i64, None, 0, 64)
    assert_parity(i64[::-1].copy(), np.arange(n, dtype=np.uint32), 0, 64)


@pytest.mark.parametrize("dtype", [np.uint32, np.float32])
def test_blocks_of_one_digit(dtype):
    """A large share of equal keys gathers into contiguous blocks after the
    first pass, where every key of a wave has the same digit; those waves
    rank with one counter add.  Values are the input index, so the order
    inside the blocks is checked too, and the blocks are cut by tile and
    segment boundaries at several sizes."""
    rng = np.random.default_rng(55)
    for n in (7 * KEY_TILE + 3001, 23 * PAIR_TILE + 17):
        if dtype == np.uint32:
            keys = rng.integers(0, 2**32, n, dtype=np.uint32)
            keys[rng.random(n) < 0.4] = np.uint32(0xC0FFEE11)
        else:
            keys = (rng.standard_normal(n) * 100).astype(np.float32)
            sp = rng.random(n)
            keys[sp < 0.02] = np.inf
            keys[(sp >= 0.02) & (sp < 0.04)] = -np.inf
            keys[(sp >= 0.04) & (sp < 0.05)] = np.nan
        vals = np.arange(n, dtype=np.uint32)
        assert_parity(keys, None)
        assert_parity(keys, vals)
        assert_parity(keys, vals, 8, 32, in_place=True)


@pytest.mark.parametrize("items", [16, 28])
@pytest.mark.parametrize("dtype", [np.uint32, np.int32, np.float32])
def test_keys_forced_tile_sizes(items, dtype):
    """Keys-only sorts of 32-bit keys take 16384- or 28672-key tiles,
    chosen per size; each size is forced here at sizes around both tiles'
    boundaries, with ragged tails, over a bit range and in place."""
    prev = rs.prof_tile_items(items)
    try:
        for n in (65537, 5 * PAIR_TILE + 3, 7 * KEY_TILE + 11, 40 * KEY_TILE + 777):
            keys = rand_keys(dtype, n, seed=n + items)
            assert_parity(keys)
            assert_parity(keys, None, 8, 24)
            assert_parity(keys, None, in_place=True)
    finally:
        rs.prof_tile_items(prev)

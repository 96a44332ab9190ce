"""GPU test of the all-pass digit histogram itself ([WA] "Las tres fases de
una pasada": the histogram is the first phase of every pass).  Output parity
cannot see a wrong count when every pass is skipped (keys already in order),
so the counts the histogram kernel leaves in temp are compared with numpy
counts of the same digits, per pass and per segment, on inputs that take
each of its paths: random keys, sorted keys (bins shared by a row of 64·V
consecutive keys), constant high bytes (bins shared by a wave's whole unit of
64·ITEMS keys), keys sorted except for one inversion, a bit range, and 64-bit
and 16-bit keys, all with a partial last unit."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
rs = pytest.importorskip("lsd_radix_sort_pass_amd")

pytestmark = pytest.mark.gpu

TILE = 28672          # forced keys-only tile of 32-bit keys (28 keys per thread)
SEGMENTS = 8


def note(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def ordered(keys):
    k = keys
    if k.dtype == np.int32:
        return k.view(np.uint32) ^ np.uint32(0x80000000)
    if k.dtype == np.int64:
        return k.view(np.uint64) ^ np.uint64(1 << 63)
    return k.view({2: np.uint16, 4: np.uint32, 8: np.uint64}[k.dtype.itemsize])


def expected_hist(keys, b, e, tile, seg_mode=0, bounds=None):
    """[passes][8][256] counts: pass 0 by position segment (whole tiles),
    pass p >= 1 by the top 3 bits of the pass-(p-1) digit, or, for a pass
    whose bit is set in seg_mode, by the number of its sampled boundaries at
    or below the 32-bit X = L * 2^(32 - w) + (index >> s), with L the w
    ordered-key bits from b up to the pass's digit and s the smallest shift
    that fits index n - 1 into 32 - w bits, but at least 3."""
    n = keys.size
    k = ordered(keys).astype(np.uint64)
    passes = (e - b + 7) // 8
    tiles = (n + tile - 1) // tile
    first = [(s * tiles) // SEGMENTS * tile for s in range(SEGMENTS + 1)]
    seg0 = np.zeros(n, dtype=np.int64)
    for s in range(SEGMENTS):
        seg0[min(first[s], n):min(first[s + 1], n)] = s
    out = np.zeros((passes, SEGMENTS, 256), dtype=np.int64)
    prev = None
    for p in range(passes):
        shift = b + 8 * p
        w = min(8, e - shift)
        d = ((k >> np.uint64(shift)) & np.uint64((1 << w) - 1)).astype(np.int64)
        if p == 0:
            seg = seg0
        elif (seg_mode >> p) & 1:
            below = shift - b
            low = (k >> np.uint64(b)) & np.uint64((1 << below) - 1)
            room = 32 - below
            ishift = max(3, int(n - 1).bit_length() - room)
            x = (low << np.uint64(room)) | (np.arange(n, dtype=np.uint64) >> np.uint64(ishift))
            assert int(x.max()) < 2**32
            seg = np.searchsorted(np.asarray(bounds[p], dtype=np.uint64), x, side="right").astype(np.int64)
        else:
            seg = prev >> 5
        np.add.at(out[p], (seg, d), 1)
        prev = d
    return out


def device_hist(temp, passes):
    off = rs._lib.load().rs_prof_header_offset(3)
    h = temp[off:off + passes * SEGMENTS * 256 * 4].view(torch.int32).cpu().numpy().astype(np.int64)
    return h.reshape(passes, SEGMENTS, 256)


def device_segment_rule(temp, passes):
    """Bit p set for a pass p >= 1 whose segments are cut by position (only
    the words of passes 1..passes-1 are written), and the boundaries."""
    lib = rs._lib.load()
    mo, bo = lib.rs_prof_header_offset(4), lib.rs_prof_header_offset(5)
    words = temp[mo:mo + 32].view(torch.int32).cpu().numpy()
    mode = sum(1 << p for p in range(1, passes) if words[p] != 0)
    bounds = temp[bo:bo + 8 * 7 * 4].view(torch.int32).cpu().numpy().view(np.uint32).reshape(8, 7)
    return mode, bounds


def check(keys, b=0, e=None, pairs=False, want_mode=None):
    e = 8 * keys.dtype.itemsize if e is None else e
    note(f"histogram dtype={keys.dtype} n={keys.size} bits=[{b},{e}) pairs={pairs}")
    dk = torch.from_numpy(keys).to("cuda")
    tdt = {np.dtype(np.uint32): torch.uint32, np.dtype(np.int32): torch.int32, np.dtype(np.uint64): torch.uint64,
           np.dtype(np.uint16): torch.uint16}[keys.dtype]
    temp = rs.alloc_temp(keys.size, pairs, b, e, device=dk.device, key_dtype=tdt)
    if pairs:
        rs.sort_pairs(dk, torch.arange(keys.size, dtype=torch.int32, device="cuda"), b, e, temp=temp, check=True)
    else:
        rs.sort_keys(dk, b, e, temp=temp, check=True)
    torch.cuda.synchronize()
    tile = {2: 28672, 4: 17408 if pairs else TILE, 8: 11264 if pairs else 14336}[keys.dtype.itemsize]
    passes = (e - b + 7) // 8
    mode, bounds = device_segment_rule(temp, passes) if keys.size >= (1 << 22) else (0, None)
    if want_mode is not None:
        assert mode == want_mode, f"segment mode {mode:#x}, expected {want_mode:#x}"
    want = expected_hist(keys, b, e, tile, mode, bounds)
    got = device_hist(temp, passes)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} wrong counts, first (pass, segment, digit) {bad[:4].tolist()}: " \
                          f"got {[got[tuple(x)] for x in bad[:4]]} want {[want[tuple(x)] for x in bad[:4]]}"


@pytest.fixture(autouse=True)
def long_tiles():
    prev = rs.prof_tile_items(28)
    try:
        yield
    finally:
        rs.prof_tile_items(prev)


N = 11 * TILE + 1777


def test_hist_random():
    rng = np.random.default_rng(1)
    check(rng.integers(0, 2**32, N, dtype=np.uint32))
    check(rng.integers(-(2**31), 2**31, N, dtype=np.int32), 4, 29)


@pytest.mark.parametrize("step", [1, 16, 300, 70_000])
def test_hist_sorted(step):
    rng = np.random.default_rng(step)
    keys = np.cumsum(rng.integers(0, step, N, dtype=np.uint64)).astype(np.uint32)
    keys.sort()
    check(keys)
    check(keys, 3, 27)


def test_hist_sorted_with_one_inversion():
    rng = np.random.default_rng(7)
    keys = np.sort(rng.integers(0, 2**32, N, dtype=np.uint32))
    # a lane's run, a unit's last key (its successor is the next unit's
    # first), a row's last key, the end
    for at in (N // 3, 5 * 1024 * 16 + 63, 7 * 1024 - 1, 9 * 1024 + 255, N - 2):
        k = keys.copy()
        k[at], k[at + 1] = k[at + 1], k[at]
        check(k)


@pytest.mark.parametrize("high", [0x12, 0x0000, 0xABCD])
def test_hist_constant_high_bytes(high):
    rng = np.random.default_rng(high)
    if high > 0xFF:
        keys = (np.uint32(high) << np.uint32(16)) | rng.integers(0, 2**16, N, dtype=np.uint32)
    else:
        keys = (np.uint32(high) << np.uint32(24)) | rng.integers(0, 2**24, N, dtype=np.uint32)
    check(keys)
    check(keys, pairs=True)
    # constant in a window of the steps only: the first third random
    k = keys.copy()
    k[: N // 3] = rng.integers(0, 2**32, N // 3, dtype=np.uint32)
    check(k)


def test_hist_all_equal_and_two_values():
    check(np.full(N, 0x7F00FF01, dtype=np.uint32))
    rng = np.random.default_rng(3)
    check(np.where(rng.random(N) < 0.5, 0x10203040, 0x10203041).astype(np.uint32))


def test_hist_64_and_16_bit_keys():
    rng = np.random.default_rng(11)
    n = 9 * 14336 + 555
    k64 = (np.uint64(0x0123456700000000) | rng.integers(0, 2**32, n, dtype=np.uint64))
    check(k64)
    check(np.sort(rng.integers(0, 2**64, n, dtype=np.uint64)))
    n16 = 7 * 28672 + 99
    check(np.sort(rng.integers(0, 2**16, n16, dtype=np.uint16)))
    check((rng.integers(0, 256, n16, dtype=np.uint16)))


BIG = (1 << 22) + 3 * TILE + 1001


def test_hist_position_segments_duplicate_heavy():
    """Keys whose bytes are AND-of-three draws: every pass >= 1 would put two
    thirds of the keys in one digit-group segment, so the sampling step
    flags all of them and the histogram counts by position."""
    rng = np.random.default_rng(21)
    k = (rng.integers(0, 2**32, BIG, dtype=np.uint32) & rng.integers(0, 2**32, BIG, dtype=np.uint32)
         & rng.integers(0, 2**32, BIG, dtype=np.uint32))
    check(k, want_mode=0b1110)
    check(k, pairs=True, want_mode=0b1110)
    check(k, 3, 27)


def test_hist_position_segments_constant_low_byte():
    """A constant low byte (pass 0 moves nothing) puts every key in one
    digit group for pass 1; only that pass is cut by position."""
    rng = np.random.default_rng(22)
    k = (rng.integers(0, 2**24, BIG, dtype=np.uint32) << np.uint32(8)) | np.uint32(0x5A)
    check(k, want_mode=0b0010)


def test_hist_no_position_segments_uniform():
    rng = np.random.default_rng(23)
    check(rng.integers(0, 2**32, BIG, dtype=np.uint32), want_mode=0)


@pytest.mark.parametrize("n", [65537, 3 * TILE - 1, 3 * TILE + 1025])
def test_hist_small_chunks_and_partial_units(n):
    """Sizes just above the one-launch limit: most workgroups' chunks hold
    no keys, and the last segment ends in a partial unit (1 to 1023 keys
    after its whole 1024-key units)."""
    rng = np.random.default_rng(n)
    check(rng.integers(0, 2**32, n, dtype=np.uint32))
    check(np.sort(rng.integers(0, 2**32, n, dtype=np.uint32)))

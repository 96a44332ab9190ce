"""GPU parity of the one-launch path for small inputs (up to 16 tiles of
4096 keys): every pass in a single launch, phases separated by waits for
all tiles of the phase before.  Sizes straddle its tiles and its upper limit (65536 keys; one
key more takes the multi-launch path), with 1 to 4 passes (8 for 64-bit
keys), in place, key-value, heavy duplicates, 64-bit keys; the device
guard word stays zero and the profiling hook shows which path ran."""
import sys

import numpy as np
import pytest

import oracle
from lsd_radix_sort_pass_amd import _lib

torch = pytest.importorskip("torch")
rs = pytest.importorskip("lsd_radix_sort_pass_amd")

pytestmark = pytest.mark.gpu

SMALL_TILE = 4096
SMALL_MAX = 16 * SMALL_TILE


def note(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def run(keys, values=None, b=0, e=None, in_place=False):
    kb = 8 * keys.dtype.itemsize
    e = kb if e is None else e
    note(f"small dtype={keys.dtype} n={keys.size} pairs={values is not None} bits=[{b},{e}) in_place={in_place}")
    dk = torch.from_numpy(np.ascontiguousarray(keys)).to("cuda")
    temp = rs.alloc_temp(keys.size, values is not None, b, e, device="cuda", key_dtype=dk.dtype)
    if values is None:
        ko = rs.sort_keys(dk, b, e, out=dk if in_place else None, temp=temp)
        vo = None
    else:
        dv = torch.from_numpy(values).to("cuda")
        ko, vo = rs.sort_pairs(dk, dv, b, e, keys_out=dk if in_place else None,
                               values_out=dv if in_place else None, temp=temp)
    torch.cuda.synchronize()
    assert rs.error_word(temp) == 0
    word = np.uint64 if kb == 64 else np.uint32
    if values is None:
        ek = oracle.lsd_sort(keys, None, b, e)
        assert np.array_equal(ko.cpu().numpy().view(word), ek.view(word))
    else:
        ek, ev = oracle.lsd_sort(keys, values, b, e)
        assert np.array_equal(ko.cpu().numpy().view(word), ek.view(word))
        assert np.array_equal(vo.cpu().numpy(), ev)


def keys_of(dtype, n, seed):
    rng = np.random.default_rng(seed)
    if dtype == np.uint32:
        return rng.integers(0, 2**32, n, dtype=np.uint32)
    if dtype == np.int32:
        return rng.integers(-(2**31), 2**31, n, dtype=np.int32)
    if dtype == np.float32:
        x = (rng.standard_normal(n) * 1000).astype(np.float32)
        x[rng.random(n) < 0.01] = np.nan
        x[rng.random(n) < 0.01] = -0.0
        return x
    if dtype == np.uint64:
        return rng.integers(0, 2**64, n, dtype=np.uint64)
    if dtype == np.int64:
        return rng.integers(-(2**63), 2**63, n, dtype=np.int64)
    x = rng.standard_normal(n) * np.exp2(rng.integers(-40, 40, n))
    x[rng.random(n) < 0.01] = -np.inf
    return x


SIZES = [2, 3, 63, 64, 65, 511, 4095, 4096, 4097, 8191, 8192, 8193, 12345, 32768, SMALL_MAX - 1, SMALL_MAX, SMALL_MAX + 1]


@pytest.mark.parametrize("dtype", [np.uint32, np.int32, np.float32])
@pytest.mark.parametrize("n", SIZES)
def test_small_sizes(dtype, n):
    keys = keys_of(dtype, n, seed=n + 17)
    run(keys)
    run(keys, np.arange(n, dtype=np.uint32))


@pytest.mark.parametrize("bits", [(0, 8), (0, 16), (3, 29), (24, 32), (0, 1), (5, 21), (0, 24)])
def test_small_bit_ranges_and_in_place(bits):
    b, e = bits
    n = 5 * SMALL_TILE + 77
    keys = keys_of(np.uint32, n, seed=b * 40 + e)
    vals = np.random.default_rng(e).integers(0, 2**32, n, dtype=np.uint32)
    run(keys, None, b, e)
    run(keys, vals, b, e)
    run(keys, None, b, e, in_place=True)
    run(keys, vals, b, e, in_place=True)


@pytest.mark.parametrize("pattern", ["two_values", "all_equal", "runs", "one_hot"])
def test_small_stability(pattern):
    n = 60000
    rng = np.random.default_rng(31 + len(pattern))
    keys = {
        "two_values": rng.integers(0, 2, n, dtype=np.uint32) * np.uint32(0x01010101),
        "all_equal": np.full(n, 0xCAFEF00D, dtype=np.uint32),
        "runs": np.repeat(rng.integers(0, 2**32, n // 50 + 1, dtype=np.uint32), 50)[:n],
        "one_hot": (np.uint32(1) << rng.integers(0, 32, n, dtype=np.uint32)).astype(np.uint32),
    }[pattern]
    run(keys, np.arange(n, dtype=np.uint32))
    run(keys, np.arange(n, dtype=np.uint32), 4, 28)


@pytest.mark.parametrize("dtype", [np.uint64, np.int64, np.float64])
@pytest.mark.parametrize("n", [2, 100, 4097, SMALL_MAX])
def test_small_64bit(dtype, n):
    keys = keys_of(dtype, n, seed=n + 3)
    run(keys)
    run(keys, np.arange(n, dtype=np.uint32))
    run(keys, None, 8, 40, in_place=True)
    run(keys, np.arange(n, dtype=np.uint32), 0, 24, in_place=True)      # 3 passes in place


@pytest.mark.parametrize("n", [2, 4097, 3 * SMALL_TILE + 5, SMALL_MAX])
def test_single_workgroup_claims_every_tile(n):
    """With one workgroup the launch still completes: it claims every tile of
    every phase itself (no phase waits for a workgroup that is not running)."""
    prev = rs.prof_small_path(2)
    try:
        for dtype in (np.uint32, np.float32, np.uint64):
            keys = keys_of(dtype, n, seed=n + 11)
            run(keys)
            run(keys, np.arange(n, dtype=np.uint32))
            run(keys, np.arange(n, dtype=np.uint32), 0, 8, in_place=True)
            run(keys, None, 0, 24, in_place=True)
    finally:
        rs.prof_small_path(prev)


def test_small_path_is_one_launch():
    """Timing hook: a sort of SMALL_MAX keys records one launch of the
    one-launch kernel (plus its zero fill) and no pass kernel; one key more
    takes the multi-launch path."""
    for n, small in [(SMALL_MAX, True), (SMALL_MAX + 1, False)]:
        dk = torch.from_numpy(keys_of(np.uint32, n, seed=5)).to("cuda")
        torch.cuda.synchronize()
        rs.prof_reset()
        rs.prof_enable(True)
        rs.sort_keys(dk)
        torch.cuda.synchronize()
        rs.prof_enable(False)
        small_launches, _ = rs.prof_summary(_lib.RS_KERNEL_SMALL)
        pass_launches, _ = rs.prof_summary(_lib.RS_KERNEL_PASS)
        rs.prof_reset()
        assert (small_launches, pass_launches) == ((1, 0) if small else (0, 4))


@pytest.mark.parametrize("dtype", [np.uint32, np.float32, np.int64])
def test_multi_launch_path_at_small_sizes(dtype):
    """With the one-launch path forbidden, small inputs take the multi-launch
    path (the fallback when a cooperative launch is unavailable)."""
    prev = rs.prof_small_path(0)
    try:
        for n in [2, 3, 100, 4097, 28673, SMALL_MAX]:
            keys = keys_of(dtype, n, seed=n + 99)
            run(keys)
            run(keys, np.arange(n, dtype=np.uint32))
            run(keys, None, 0, 8, in_place=True)
    finally:
        rs.prof_small_path(prev)

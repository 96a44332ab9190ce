"""Structure of the seeded workloads (no GPU): sizes, dtypes, seeds, and the
properties each generator promises (value ranges, ordering, constant
digits), so that a workload measures what its name says."""
import numpy as np
import pytest

from lsd_radix_sort_pass_amd import workloads


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_shapes_and_seeds(name):
    w = workloads.WORKLOADS[name]
    keys, values, b, e = workloads.make(name, n=5000)
    assert keys.dtype == w.dtype and keys.size == 5000
    assert (b, e) == (w.begin_bit, w.end_bit) and 0 <= b < e <= 8 * keys.dtype.itemsize
    if w.pairs:
        assert values.dtype == w.value_dtype and np.array_equal(values, np.arange(5000))
    else:
        assert values is None
    again = workloads.make(name, n=5000)[0]
    assert np.array_equal(keys.view(np.uint8), again.view(np.uint8))       # seeded
    other = workloads.make(name, n=5000, seed=1)[0]
    assert not np.array_equal(keys.view(np.uint8), other.view(np.uint8))


def test_indices_unique():
    idx = [w.index for w in workloads.WORKLOADS.values()] + [workloads.POINTS_WORKLOAD_INDEX]
    assert len(idx) == len(set(idx))


def test_sorted_workload_is_sorted():
    keys = workloads.make("sorted_u32_2^28", n=1 << 20)[0]
    assert np.all(keys[1:] >= keys[:-1]) and keys[-1] < 2**32 - 1
    assert np.unique(keys).size > (1 << 20) // 2             # mostly distinct


def test_sorted_workload_cannot_wrap():
    # running sums of steps < 16 over 2^28 keys stay below 2^32
    assert 15 * (1 << 28) < 2**32


def test_low16_high_bytes_constant():
    keys = workloads.make("low16_u32_2^28", n=1 << 20)[0]
    assert np.all(keys >> np.uint32(16) == 0)
    assert np.unique(keys & np.uint32(0xFF)).size == 256 and np.unique(keys >> np.uint32(8)).size == 256


def test_wide_workloads_cover_their_range():
    k16 = workloads.make("uniform_u16_2^28", n=1 << 18)[0]
    assert np.unique(k16 >> np.uint16(8)).size == 256
    k64 = workloads.make("uniform_u64_2^27", n=1 << 16)[0]
    assert np.unique(k64 >> np.uint64(56)).size == 256

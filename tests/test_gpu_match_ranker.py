"""GPU parity of the ballot match ranker (rs_prof_ranker(1)): the same sorts
as the default LDS-atomic ranker, compared bit-exactly with the oracle.
The match ranker never depends on the order in which the LDS serves
same-address atomics, so these runs show that stability ([WA] "La idea y el
requisito de estabilidad": stability is each pass's condition of
correctness) also holds with a ranker whose order is fixed by ballots and
mbcnt alone."""
import numpy as np
import pytest

from lsd_radix_sort_pass_amd import workloads
from test_gpu_parity import KEY_TILE, PAIR_TILE, assert_parity, note, rand_keys

torch = pytest.importorskip("torch")
rs = pytest.importorskip("lsd_radix_sort_pass_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def match_ranker():
    prev = rs.prof_ranker(1)
    try:
        yield
    finally:
        rs.prof_ranker(prev)


SIZES = [2, 100, 4097, 40_000, 65536, 65537, PAIR_TILE + 1, KEY_TILE + 1, 3 * KEY_TILE + 1234,
         17 * PAIR_TILE + 4321]


@pytest.mark.parametrize("dtype", [np.uint32, np.int32, np.float32])
@pytest.mark.parametrize("n", SIZES)
def test_match_keys_and_pairs(dtype, n):
    keys = rand_keys(dtype, n, seed=n + 31)
    assert_parity(keys)
    assert_parity(keys, np.arange(n, dtype=np.uint32))


@pytest.mark.parametrize("items", [16, 28])
@pytest.mark.parametrize("dtype", [np.uint32, np.float32])
def test_match_forced_tiles(items, dtype):
    prev = rs.prof_tile_items(items)
    try:
        for n in (5 * PAIR_TILE + 3, 7 * KEY_TILE + 11):
            keys = rand_keys(dtype, n, seed=n + items)
            assert_parity(keys)
            assert_parity(keys, None, 8, 24, in_place=True)
    finally:
        rs.prof_tile_items(prev)


@pytest.mark.parametrize("pattern", ["two_values", "all_equal", "one_hot_digit", "runs", "specials_block"])
def test_match_stability(pattern):
    """Heavy duplication: whole waves and slots of one digit, where the
    match ranker's peer sets are largest."""
    n = 7 * 2 * KEY_TILE + 4097
    rng = np.random.default_rng(900 + len(pattern))
    if pattern == "two_values":
        keys = rng.integers(0, 2, n, dtype=np.uint32) * np.uint32(0x01010101)
    elif pattern == "all_equal":
        keys = np.full(n, 0x12345678, dtype=np.uint32)
    elif pattern == "one_hot_digit":
        keys = (np.uint32(1) << rng.integers(0, 32, n, dtype=np.uint32)).astype(np.uint32)
    elif pattern == "runs":
        keys = np.repeat(rng.integers(0, 2**32, n // 100 + 1, dtype=np.uint32), 100)[:n]
    else:
        keys = (rng.standard_normal(n) * 100).astype(np.float32)
        keys[rng.random(n) < 0.3] = np.nan
    values = np.arange(n, dtype=np.uint32)
    assert_parity(keys, values)
    assert_parity(keys, values, 8, 24)
    assert_parity(keys, None)


@pytest.mark.parametrize("name", ["gauss_f32_2^24", "dup_pairs_u32_2^26", "uniform_u32_2^16"])
def test_match_workloads_full_size(name):
    note(f"match ranker, full workload {name}")
    keys, values, b, e = workloads.make(name)
    assert_parity(keys, values, b, e)


def test_match_small_path_one_workgroup():
    prev = rs.prof_small_path(2)
    try:
        keys = rand_keys(np.uint32, 50_001, seed=3)
        assert_parity(keys, np.arange(keys.size, dtype=np.uint32))
        assert_parity(keys, None, 0, 24, in_place=True)
    finally:
        rs.prof_small_path(prev)

"""GPU parity of the fused Morton-code sort (rs_sort_morton30): the codes the
library computes from float32 points, sorted with their point indices, must
equal the oracle's codes (oracle.morton30) put through the oracle's stable
sort over bits [0, 30), bit for bit, on boxes that clamp, boxes with an
inexact scale, special coordinates, duplicate-heavy lattices and identical
points, at sizes around the key-value tile and at the workload's full size."""
import sys

import numpy as np
import pytest

import oracle
from lsd_radix_sort_pass_amd import workloads

torch = pytest.importorskip("torch")
rs = pytest.importorskip("lsd_radix_sort_pass_amd")

pytestmark = pytest.mark.gpu

PAIR_TILE = 17408  # keys per key-value pass tile


def note(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def assert_morton_parity(points, lo=(0, 0, 0), hi=(1, 1, 1)):
    pts = np.ascontiguousarray(points, dtype=np.float32)
    n = pts.shape[0]
    note(f"morton n={n} box={lo}..{hi}")
    dp = torch.from_numpy(pts).to("cuda")
    codes, index = rs.sort_morton30(dp, lo, hi)
    torch.cuda.synchronize()
    gc, gi = codes.cpu().numpy(), index.cpu().numpy()
    oc = oracle.morton30(pts, lo, hi)
    ek, ev = oracle.lsd_sort(oc, np.arange(n, dtype=np.uint32), 0, 30)
    if not np.array_equal(gc, ek):
        bad = np.flatnonzero(gc != ek)
        raise AssertionError(f"codes differ at {bad.size} positions, first {bad[:6].tolist()}: "
                             f"gpu {gc[bad[:6]].tolist()} oracle {ek[bad[:6]].tolist()}")
    if not np.array_equal(gi, ev):
        bad = np.flatnonzero(gi != ev)
        raise AssertionError(f"indices differ at {bad.size} positions, first {bad[:6].tolist()}")


def unit_points(n, seed):
    return np.random.default_rng(seed).random((n, 3), dtype=np.float32)


@pytest.mark.parametrize("n", [1, 2, 3, 100, 4097, PAIR_TILE - 1, PAIR_TILE, PAIR_TILE + 1,
                               5 * PAIR_TILE + 777, (1 << 20) + 11])
def test_unit_box_sizes(n):
    assert_morton_parity(unit_points(n, seed=n))


def test_boxes_that_clamp_and_inexact_scales():
    n = 3 * PAIR_TILE + 91
    rng = np.random.default_rng(5)
    pts = (rng.random((n, 3), dtype=np.float32) * 3 - 1.5).astype(np.float32)  # beyond [-1, 1]
    assert_morton_parity(pts, (-1, -1, -1), (1, 1, 1))
    pts = (rng.random((n, 3), dtype=np.float32) * 0.8).astype(np.float32)
    assert_morton_parity(pts, (0.1, 0.0, 0.05), (0.7, 0.3, 0.9))          # scales not powers of two
    # points placed on and next to quantisation steps of an inexact box
    lo, hi = np.float32(0.1), np.float32(0.7)
    s = np.float32(1024) / (hi - lo)
    k = rng.integers(0, 1024, n)
    x = (lo + k / np.float64(s)).astype(np.float32)
    x = np.where(rng.random(n) < 0.5, x, np.nextafter(x, np.float32(0)))
    pts = np.stack([x, np.roll(x, 1), np.roll(x, 2)], axis=1)
    assert_morton_parity(pts, (lo, lo, lo), (hi, hi, hi))
    big = (rng.standard_normal((n, 3)) * 1e4).astype(np.float32)
    assert_morton_parity(big, (-3e4, -1e4, -5e3), (3e4, 2e4, 5e3))


def test_special_coordinates():
    n = 2 * PAIR_TILE + 5
    rng = np.random.default_rng(6)
    pts = rng.random((n, 3), dtype=np.float32)
    specials = np.array([np.nan, np.inf, -np.inf, -0.0, 0.0, 1.0, -1e-30, 1e-30, 0.999999], dtype=np.float32)
    mask = rng.random((n, 3)) < 0.2
    pts[mask] = specials[rng.integers(0, specials.size, mask.sum())]
    assert_morton_parity(pts)


def test_duplicates_and_identical_points():
    """Coarse lattices give runs of equal codes (indices must stay in
    order); identical points make every pass after the first move nothing."""
    n = 4 * PAIR_TILE + 333
    rng = np.random.default_rng(7)
    lattice = (np.floor(rng.random((n, 3), dtype=np.float32) * 4) / 4).astype(np.float32)
    assert_morton_parity(lattice)
    assert_morton_parity(np.full((n, 3), 0.3, dtype=np.float32))
    line = np.zeros((n, 3), dtype=np.float32)
    line[:, 0] = rng.random(n, dtype=np.float32)                   # only x varies
    assert_morton_parity(line)
    sorted_pts = np.repeat(np.linspace(0, 1, n, endpoint=False, dtype=np.float32)[:, None], 3, axis=1)
    assert_morton_parity(sorted_pts)                                # codes already ascending


def test_full_workload_size():
    pts = workloads.make_points(workloads.POINTS_WORKLOAD_N)
    assert_morton_parity(pts)


def test_empty_and_errors():
    empty = torch.empty((0, 3), dtype=torch.float32, device="cuda")
    c, i = rs.sort_morton30(empty)
    assert c.numel() == 0 and i.numel() == 0
    pts = torch.rand((10, 3), device="cuda")
    with pytest.raises(rs.RadixSortError):
        rs.sort_morton30(pts, (0, 0, 0), (1, 0, 1))                 # empty box on y
    with pytest.raises(rs.RadixSortError):
        rs.sort_morton30(pts, (0, 0, 0), (1, float("inf"), 1))
    temp = torch.empty(rs.temp_bytes_morton30(10) - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(rs.RadixSortError):
        rs.sort_morton30(pts, temp=temp)

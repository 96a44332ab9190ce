"""Pins for the oracle's 30-bit Morton codes (no GPU).

The sort's pages use it inside an LBVH build ("高性能计算：GPU上的基数排序"
on onikatahoshio); the Morton code itself is not defined on them, so the
oracle follows stated readings (10 bits per axis over a box, x highest in
each bit triple, quantisation in single precision).  These tests tie it to
facts other than its own formula: closed-form codes of chosen points, the
Z-order of a lattice, an independent order comparator on the quantised
coordinates (most significant differing bit), the clamping rules, the
single-precision rounding of the quantisation, and the workload
generator's own float64 implementation of the unit-box codes."""
import math

import numpy as np
import pytest

import oracle
from lsd_radix_sort_pass_amd import workloads


def codes(points, lo=(0, 0, 0), hi=(1, 1, 1)):
    return oracle.morton30(np.asarray(points, dtype=np.float32), lo, hi)


def test_closed_form_codes():
    pts = [(0, 0, 0), (1, 1, 1), (0.5, 0, 0), (0, 0.5, 0), (0, 0, 0.5),
           (1 / 1024, 0, 0), (0, 1 / 1024, 0), (0, 0, 1 / 1024), (3 / 1024, 0, 0), (0.75, 0.25, 0.5)]
    # (3/1024, 0, 0): qx = 0b11 -> bits 2 and 5.  (0.75, 0.25, 0.5): qx = 768 = bits 9, 8;
    # qy = 256 = bit 8; qz = 512 = bit 9 -> x at 29, 26; y at 25; z at 27.
    want = [0, 2**30 - 1, 2**29, 2**28, 2**27, 4, 2, 1, 4 + 32, 2**29 + 2**26 + 2**25 + 2**27]
    assert codes(pts).tolist() == want


def test_lattice_is_z_order():
    """The 8 corners of the half-unit lattice get the octant number
    4x + 2y + z in the top bit triple."""
    pts = [(x / 2, y / 2, z / 2) for x in (0, 1) for y in (0, 1) for z in (0, 1)]
    got = codes(pts)
    assert got.tolist() == [(4 * x + 2 * y + z) << 27 for x in (0, 1) for y in (0, 1) for z in (0, 1)]


def _z_less(a, b):
    """Z-order comparison of two integer triples without interleaving: the
    axis whose coordinates differ in the highest bit decides (x before y
    before z at equal bit levels)."""
    best_axis, best_bit = None, -1
    for axis in range(3):
        x = int(a[axis]) ^ int(b[axis])
        if x and x.bit_length() - 1 > best_bit:
            best_axis, best_bit = axis, x.bit_length() - 1
    if best_axis is None:
        return False
    return a[best_axis] < b[best_axis]


def test_order_matches_msb_comparator():
    rng = np.random.default_rng(11)
    q = rng.integers(0, 1024, (400, 3))
    pts = (q / 1024.0).astype(np.float32)          # exactly on the lattice
    c = codes(pts)
    for i in range(0, 400, 2):
        a, b = q[i], q[i + 1]
        assert (c[i] < c[i + 1]) == _z_less(a, b)
        assert (c[i + 1] < c[i]) == _z_less(b, a)
    # equal triples give equal codes
    assert codes([(0.25, 0.5, 0.125), (0.25, 0.5, 0.125)]).tolist()[0] == codes([(0.25, 0.5, 0.125)])[0]


def test_clamping_and_specials():
    lo, hi = (0, 0, 0), (2, 2, 2)                   # scale 512
    below = np.nextafter(np.float32(2), np.float32(0))
    xs = [1.0, 2.0, 3.0, -1.0, float("nan"), float("inf"), float("-inf"), 0.0, float(below), 1 / 512]
    want_q = [512, 1023, 1023, 0, 0, 1023, 0, 0, 1023, 1]
    got = codes([(x, 0, 0) for x in xs], lo, hi)
    spread = lambda q: sum(((q >> i) & 1) << (3 * i) for i in range(10))
    assert got.tolist() == [spread(q) << 2 for q in want_q]


def test_quantisation_is_single_precision():
    """Points near a quantisation step in a box whose scale is inexact: the
    codes follow the single-precision evaluation (p - lo) * s, which differs
    from the real-number and double-precision results for some points."""
    lo, hi = np.float32(0.1), np.float32(0.7)
    s = np.float32(1024) / (hi - lo)
    assert oracle.morton_scale(float(lo), float(hi)) == float(s)
    rng = np.random.default_rng(12)
    k = rng.integers(1, 1023, 20000)
    x = (lo + (k / np.float64(s))).astype(np.float32)            # near step k
    x = np.concatenate([x, np.nextafter(x, np.float32(0)), np.nextafter(x, np.float32(1))])
    t32 = (x - lo) * s                                            # float32 arithmetic throughout
    q32 = np.where(~(t32 > 0), 0, np.where(t32 >= 1023, 1023, np.floor(t32))).astype(np.int64)
    t64 = (x.astype(np.float64) - np.float64(lo)) * (1024.0 / (np.float64(hi) - np.float64(lo)))
    q64 = np.clip(np.floor(t64), 0, 1023).astype(np.int64)
    assert np.any(q32 != q64)                                     # the precision matters here
    pts = np.stack([x, np.full_like(x, lo), np.full_like(x, lo)], axis=1)
    got = codes(pts, (lo, lo, lo), (hi, hi, hi))
    spread = np.vectorize(lambda q: sum(((int(q) >> i) & 1) << (3 * i) for i in range(10)))
    assert np.array_equal(got, (spread(q32) << 2).astype(np.uint32))


def test_matches_workload_generator_on_unit_box():
    """workloads.py builds the unit-box codes of float64 points in numpy; for
    float32 points both quantisations are exact (scale 1024) and must agree."""
    rng = np.random.default_rng(13)
    pts = rng.random((5000, 3), dtype=np.float32)
    q = np.minimum(np.floor(pts.astype(np.float64) * 1024.0), 1023.0).astype(np.uint32)
    ref = ((workloads._spread3(q[:, 0]) << np.uint32(2)) | (workloads._spread3(q[:, 1]) << np.uint32(1))
           | workloads._spread3(q[:, 2]))
    assert np.array_equal(codes(pts), ref)


def test_sorted_codes_with_indices():
    """Morton codes sorted with point indices: stable, equal codes keep index order."""
    rng = np.random.default_rng(14)
    pts = np.floor(rng.random((3000, 3), dtype=np.float32) * 8) / 8     # many equal codes
    c = codes(pts)
    ks, vs = oracle.lsd_sort(c, np.arange(c.size, dtype=np.uint32), 0, 30)
    order = np.argsort(c, kind="stable")
    assert np.array_equal(vs, order.astype(np.uint32)) and np.array_equal(ks, c[order])


@pytest.mark.parametrize("lo,hi", [((0, 0, 0), (0, 1, 1)), ((1, 0, 0), (0, 1, 1)),
                                   ((0, 0, 0), (math.inf, 1, 1)), ((math.nan, 0, 0), (1, 1, 1)),
                                   ((-3e38, 0, 0), (3e38, 1, 1))])
def test_invalid_boxes_rejected(lo, hi):
    with pytest.raises(ValueError):
        codes([(0.5, 0.5, 0.5)], lo, hi)

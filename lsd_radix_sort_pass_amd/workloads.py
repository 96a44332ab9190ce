"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws random numbers and packs them into arrays; it holds
none of the sort's arithmetic (no ordered-key transform, no digit, no scan).
Both the GPU tests/benchmark and the CPU oracle take their inputs from here,
which is the one thing the two sides share.

Five workloads (sizes are the full ones; every generator accepts a smaller n
for tests, keeping the same value distribution and structure):

  uniform_u32_2^16     2^16 uint32 keys uniform over [0, 2^32), keys only.
  gauss_f32_2^24       2^24 float32 keys from N(0, 1000^2) with 0.1% +-Inf,
                       0.1% quiet NaN and 1024 each of -0.0 / +0.0 at random
                       disjoint positions, keys only.
  dup_pairs_u32_2^26   2^26 uint32 keys made as the AND of three uniform draws
                       (bit density 1/8, many equal keys) with value = index.
  morton_pairs_2^24    2^24 points uniform in the unit cube, 10 bits per axis,
                       interleaved into 30-bit Morton codes, value = index,
                       sorted over bits [0, 30).
  uniform_i32_2^28     2^28 int32 keys uniform over the full signed range.
  uniform_u32_2^28     2^28 uint32 keys uniform over [0, 2^32), keys only.

Further workloads for the other key and value widths and for pass skipping:

  uniform_u16_2^28     2^28 uint16 keys uniform over [0, 2^16), keys only.
  uniform_u64_2^27     2^27 uint64 keys uniform over [0, 2^64), keys only.
  pairs_u32_v64_2^26   2^26 uniform uint32 keys with uint64 value = index.
  sorted_u32_2^28      2^28 uint32 keys already in ascending order (running
                       sums of uniform steps in [0, 16)), keys only.
  low16_u32_2^28       2^28 uint32 keys uniform over [0, 2^16): the digits of
                       the two high bytes are the same for every key.

Seeds: numpy PCG64 with seed 1000 + workload index unless given.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    index: int            # used for the default seed
    n: int                # full size
    dtype: np.dtype       # key dtype
    pairs: bool           # carries values = original index
    begin_bit: int
    end_bit: int
    make_keys: Callable[[np.random.Generator, int], np.ndarray]
    description: str
    value_dtype: np.dtype = np.dtype(np.uint32)


def _uniform_u32(rng: np.random.Generator, n: int) -> np.ndarray:
    return rng.integers(0, 2**32, size=n, dtype=np.uint32)


def _uniform_u16(rng: np.random.Generator, n: int) -> np.ndarray:
    return rng.integers(0, 2**16, size=n, dtype=np.uint16)


def _uniform_u64(rng: np.random.Generator, n: int) -> np.ndarray:
    return rng.integers(0, 2**64, size=n, dtype=np.uint64)


def _sorted_u32(rng: np.random.Generator, n: int) -> np.ndarray:
    steps = rng.integers(0, 16, size=n, dtype=np.uint32)
    return np.cumsum(steps, dtype=np.uint32)     # at most 15 * 2^28 < 2^32


def _low16_u32(rng: np.random.Generator, n: int) -> np.ndarray:
    return rng.integers(0, 2**16, size=n, dtype=np.uint32)


def _uniform_i32(rng: np.random.Generator, n: int) -> np.ndarray:
    return rng.integers(-(2**31), 2**31, size=n, dtype=np.int32)


def _gauss_f32_with_specials(rng: np.random.Generator, n: int) -> np.ndarray:
    keys = rng.normal(0.0, 1000.0, size=n).astype(np.float32)
    bits = keys.view(np.uint32)
    n_inf = int(round(n * 0.001))
    n_nan = int(round(n * 0.001))
    n_zero = max(1, (1024 * n) >> 24)          # 1024 each at n = 2^24
    total = n_inf + n_nan + 2 * n_zero
    if total > n:
        n_inf = n_nan = 0
        n_zero = n // 2
        total = 2 * n_zero
    pos = rng.choice(n, size=total, replace=False)
    p_inf = pos[:n_inf]
    p_nan = pos[n_inf:n_inf + n_nan]
    p_nzero = pos[n_inf + n_nan:n_inf + n_nan + n_zero]
    p_pzero = pos[n_inf + n_nan + n_zero:]
    # +-Inf, sign 50/50.
    inf_sign = rng.integers(0, 2, size=n_inf, dtype=np.uint32) << np.uint32(31)
    bits[p_inf] = np.uint32(0x7F800000) | inf_sign
    # Quiet NaNs: half the canonical 0x7FC00000, half a random sign and a
    # random 22-bit payload under the quiet bit.
    half = n_nan // 2
    canon = np.full(half, 0x7FC00000, dtype=np.uint32)
    nan_sign = rng.integers(0, 2, size=n_nan - half, dtype=np.uint32) << np.uint32(31)
    payload = rng.integers(0, 2**22, size=n_nan - half, dtype=np.uint32)
    noisy = nan_sign | np.uint32(0x7FC00000) | payload
    bits[p_nan] = np.concatenate([canon, noisy])
    bits[p_nzero] = np.uint32(0x80000000)
    bits[p_pzero] = np.uint32(0x00000000)
    return keys


def _and3_u32(rng: np.random.Generator, n: int) -> np.ndarray:
    a = rng.integers(0, 2**32, size=n, dtype=np.uint32)
    b = rng.integers(0, 2**32, size=n, dtype=np.uint32)
    c = rng.integers(0, 2**32, size=n, dtype=np.uint32)
    return a & b & c


def _spread3(q: np.ndarray) -> np.ndarray:
    """Move bit i of a 10-bit integer to bit 3i."""
    out = np.zeros(q.shape, dtype=np.uint32)
    for i in range(10):
        out |= ((q >> np.uint32(i)) & np.uint32(1)) << np.uint32(3 * i)
    return out


def _morton30(rng: np.random.Generator, n: int) -> np.ndarray:
    pts = rng.random((n, 3))
    q = np.minimum(np.floor(pts * 1024.0), 1023.0).astype(np.uint32)
    return ((_spread3(q[:, 0]) << np.uint32(2))
            | (_spread3(q[:, 1]) << np.uint32(1))
            | _spread3(q[:, 2]))


WORKLOADS = {
    w.name: w for w in [
        Workload("uniform_u32_2^16", 1, 1 << 16, np.dtype(np.uint32), False, 0, 32,
                 _uniform_u32, "2^16 uniform uint32 keys, keys only"),
        Workload("gauss_f32_2^24", 2, 1 << 24, np.dtype(np.float32), False, 0, 32,
                 _gauss_f32_with_specials,
                 "2^24 float32 N(0,1000^2) keys with 0.1% +-Inf, 0.1% NaN, +-0.0"),
        Workload("dup_pairs_u32_2^26", 3, 1 << 26, np.dtype(np.uint32), True, 0, 32,
                 _and3_u32, "2^26 duplicate-heavy uint32 keys (AND of 3 draws), value = index"),
        Workload("morton_pairs_2^24", 4, 1 << 24, np.dtype(np.uint32), True, 0, 30,
                 _morton30, "2^24 30-bit Morton codes of unit-cube points, value = index"),
        Workload("uniform_i32_2^28", 5, 1 << 28, np.dtype(np.int32), False, 0, 32,
                 _uniform_i32, "2^28 uniform int32 keys over the full signed range, keys only"),
        Workload("uniform_u32_2^28", 6, 1 << 28, np.dtype(np.uint32), False, 0, 32,
                 _uniform_u32, "2^28 uniform uint32 keys, keys only"),
        Workload("uniform_u16_2^28", 8, 1 << 28, np.dtype(np.uint16), False, 0, 16,
                 _uniform_u16, "2^28 uniform uint16 keys, keys only"),
        Workload("uniform_u64_2^27", 9, 1 << 27, np.dtype(np.uint64), False, 0, 64,
                 _uniform_u64, "2^27 uniform uint64 keys, keys only"),
        Workload("pairs_u32_v64_2^26", 10, 1 << 26, np.dtype(np.uint32), True, 0, 32,
                 _uniform_u32, "2^26 uniform uint32 keys with uint64 value = index",
                 np.dtype(np.uint64)),
        Workload("sorted_u32_2^28", 11, 1 << 28, np.dtype(np.uint32), False, 0, 32,
                 _sorted_u32, "2^28 uint32 keys already in ascending order, keys only"),
        Workload("low16_u32_2^28", 12, 1 << 28, np.dtype(np.uint32), False, 0, 32,
                 _low16_u32, "2^28 uint32 keys below 2^16 (two constant high bytes), keys only"),
    ]
}


# Points for the Morton-code sort: uniform in the unit cube, float32.
POINTS_WORKLOAD = "morton_points_2^24"
POINTS_WORKLOAD_N = 1 << 24
POINTS_WORKLOAD_INDEX = 7


def make_points(n: int, seed: Optional[int] = None) -> np.ndarray:
    """(n, 3) float32 points uniform in [0, 1)^3 (seed 1000 + 7 by default)."""
    rng = np.random.default_rng(1000 + POINTS_WORKLOAD_INDEX if seed is None else seed)
    return rng.random((int(n), 3), dtype=np.float32)


def make(name: str, n: Optional[int] = None, seed: Optional[int] = None):
    """Return (keys, values_or_None, begin_bit, end_bit) for a workload."""
    w = WORKLOADS[name]
    n = w.n if n is None else int(n)
    rng = np.random.default_rng(1000 + w.index if seed is None else seed)
    keys = w.make_keys(rng, n)
    assert keys.dtype == w.dtype and keys.size == n
    values = np.arange(n, dtype=w.value_dtype) if w.pairs else None
    return keys, values, w.begin_bit, w.end_bit

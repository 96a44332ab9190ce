"""Seeded random configurations against the CPU oracle: key width and kind
(16/32/64-bit unsigned, signed and float), keys only or with 32- or 64-bit
values, bit range, in place or not, and sizes from 1 key to a few hundred
thousand (one-launch and multi-launch paths, both pass-tile sizes of 32-bit
keys).  Every configuration is compared bit-exactly; the draw of each case is
printed before it runs."""
import sys

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
rs = pytest.importorskip("lsd_radix_sort_pass_amd")

pytestmark = pytest.mark.gpu

KEY_TYPES = [np.uint16, np.int16, np.float16, np.uint32, np.int32, np.float32, np.uint64, np.int64, np.float64]
WORD = {2: np.uint16, 4: np.uint32, 8: np.uint64}


def draw_keys(rng, dtype, n):
    dtype = np.dtype(dtype)
    style = rng.integers(0, 4)
    if dtype.kind == "f":
        x = (rng.standard_normal(n) * 10.0 ** rng.integers(0, 4)).astype(dtype)
        sp = rng.random(n)
        x[sp < 0.01] = np.inf
        x[(sp >= 0.01) & (sp < 0.02)] = -np.inf
        x[(sp >= 0.02) & (sp < 0.03)] = np.nan
        x[(sp >= 0.03) & (sp < 0.04)] = -0.0
    else:
        info = np.iinfo(dtype)
        x = rng.integers(info.min, int(info.max) + 1, n, dtype=dtype)
    if style == 1 and n > 0:                       # few distinct keys
        x = x[rng.integers(0, max(1, n // 1000 + 1), n)]
    elif style == 2:                               # already sorted (by value)
        x = np.sort(x)
    elif style == 3 and n > 0:                     # runs of equal keys
        x = np.repeat(x[: n // 50 + 1], 50)[:n]
    return np.ascontiguousarray(x)


def case(seed):
    rng = np.random.default_rng(9000 + seed)
    dtype = np.dtype(KEY_TYPES[rng.integers(0, len(KEY_TYPES))])
    width = 8 * dtype.itemsize
    n = int(rng.choice([1, 2, 7, 300, 4097, 65536, 65537, 100000, 200003, 333333, 500001]))
    vb = int(rng.choice([0, 4, 8]))
    b = int(rng.integers(0, width))
    e = int(rng.integers(b, width + 1)) if rng.random() < 0.5 else width
    if rng.random() < 0.5:
        b = 0
    in_place = bool(rng.random() < 0.3)
    items = int(rng.choice([0, 0, 16, 28]))
    return dtype, n, vb, b, e, in_place, items, rng


@pytest.mark.parametrize("seed", range(60))
def test_random_config(seed):
    dtype, n, vb, b, e, in_place, items, rng = case(seed)
    keys = draw_keys(rng, dtype, n)
    vals = None
    if vb:
        vals = rng.integers(0, 2**32 if vb == 4 else 2**63, n, dtype=np.uint32 if vb == 4 else np.uint64)
    print(f"\n[case] seed={seed} dtype={dtype} n={n} value_bytes={vb} bits=[{b},{e}) in_place={in_place} tile_items={items}",
          flush=True)
    sys.stdout.flush()
    prev = rs.prof_tile_items(items)
    try:
        dk = torch.from_numpy(keys.copy()).to("cuda")
        if vals is None:
            out = rs.sort_keys(dk, b, e, out=dk if in_place else None)
            torch.cuda.synchronize()
            ek = oracle.lsd_sort(keys, None, b, e)
        else:
            dv = torch.from_numpy(vals.copy()).to("cuda")
            out, vo = rs.sort_pairs(dk, dv, b, e, keys_out=dk if in_place else None,
                                    values_out=dv if in_place else None)
            torch.cuda.synchronize()
            ek, ev = oracle.lsd_sort(keys, vals, b, e)
            assert np.array_equal(vo.cpu().numpy(), ev), "values differ"
        w = WORD[dtype.itemsize]
        assert np.array_equal(out.cpu().numpy().view(w), ek.view(w)), "keys differ"
    finally:
        rs.prof_tile_items(prev)

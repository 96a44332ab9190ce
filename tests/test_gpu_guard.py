"""GPU tests of what the pass kernel's correctness rests on, beyond output
parity:

* the device-side guard: a look-back that gives up must surface as an error
  (check=True raises), and the next sort with the same temp must be correct;
* the LDS property the local rank relies on: same-address atomic adds of one
  wave64 instruction return lane-ascending prefix counts (stability, the
  condition of correctness of each pass per [WA] "La idea y el requisito de
  estabilidad", depends on it).
"""
import sys

import numpy as np
import pytest

import oracle
from lsd_radix_sort_pass_amd import workloads

torch = pytest.importorskip("torch")
rs = pytest.importorskip("lsd_radix_sort_pass_amd")

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("pairs", [False, True])
def test_forced_giveup_raises_then_recovers(pairs):
    """With the test hook on, pass 0 withholds tile 0's status words and the
    look-back bound is 64 polls: tile 1 gives up through the ordinary
    bounded wait, so every kernel ends normally and the error word is set.
    check=True must raise; with the hook off the same temp sorts correctly."""
    n = (1 << 20) + 333
    note(f"forced give-up n={n} pairs={pairs}")
    keys, _, b, e = workloads.make("uniform_u32_2^28", n=n)
    vals = np.arange(n, dtype=np.uint32)
    dk = torch.from_numpy(keys).to("cuda")
    dv = torch.from_numpy(vals).to("cuda")
    temp = rs.alloc_temp(n, pairs, device=dk.device)
    prev = rs.prof_force_giveup(True)
    try:
        with pytest.raises(rs.DeviceGuardError):
            if pairs:
                rs.sort_pairs(dk, dv, temp=temp, check=True)
            else:
                rs.sort_keys(dk, temp=temp, check=True)
        assert rs.error_word(temp) != 0
    finally:
        rs.prof_force_giveup(prev)
    if pairs:
        ko, vo = rs.sort_pairs(dk, dv, temp=temp, check=True)
        ek, ev = oracle.lsd_sort(keys, vals, b, e)
        assert np.array_equal(ko.cpu().numpy(), ek) and np.array_equal(vo.cpu().numpy(), ev)
    else:
        ko = rs.sort_keys(dk, temp=temp, check=True)
        assert np.array_equal(ko.cpu().numpy(), oracle.lsd_sort(keys, None, b, e))
    assert rs.error_word(temp) == 0


def test_check_passes_on_good_sorts():
    """check=True is silent on successful sorts of every path: one launch,
    multi-launch, Morton."""
    for n in (5000, 300_001):
        keys, _, b, e = workloads.make("gauss_f32_2^24", n=n)
        out = rs.sort_keys(torch.from_numpy(keys).to("cuda"), check=True)
        assert np.array_equal(out.cpu().numpy().view(np.uint32), oracle.lsd_sort(keys, None, b, e).view(np.uint32))
    pts = workloads.make_points(200_000)
    codes, index = rs.sort_morton30(torch.from_numpy(pts).to("cuda"), check=True)
    ec, ei = oracle.lsd_sort(oracle.morton30(pts), np.arange(200_000, dtype=np.uint32), 0, 30)
    assert np.array_equal(codes.cpu().numpy(), ec) and np.array_equal(index.cpu().numpy(), ei)


def _expected_ranks(digits: np.ndarray, slots: int, unit: int) -> np.ndarray:
    """unit x (number of the wave's earlier elements with the same digit),
    element order within a wave being (slot, lane); computed with a stable
    argsort per wave (independent of any LDS behaviour)."""
    d = (digits & 0xFF).astype(np.int64).reshape(-1, slots * 64)     # one row per wave, element order
    waves = d.shape[0]
    key = d + 256 * np.arange(waves, dtype=np.int64)[:, None]        # distinct digit ranges per wave
    flat = key.ravel()
    order = np.argsort(flat, kind="stable")
    sk = flat[order]
    starts = np.r_[0, np.flatnonzero(sk[1:] != sk[:-1]) + 1]
    run_start = np.repeat(starts, np.diff(np.r_[starts, sk.size]))
    rank = np.empty(flat.size, dtype=np.int64)
    rank[order] = np.arange(sk.size) - run_start
    return (rank * unit).astype(np.uint32)


def _patterns(rng, words, slots):
    lane = np.tile(np.arange(64, dtype=np.uint32), words // 64)
    return {
        "uniform": rng.integers(0, 256, words, dtype=np.uint32),
        "all_equal": np.full(words, 0xA7, dtype=np.uint32),
        "two_values": rng.integers(0, 2, words, dtype=np.uint32) * 0x55,
        "four_values": rng.integers(0, 4, words, dtype=np.uint32) * 64,
        "sixteen_values": rng.integers(0, 16, words, dtype=np.uint32),
        "skewed_and3": (rng.integers(0, 256, words, dtype=np.uint32) & rng.integers(0, 256, words, dtype=np.uint32)
                        & rng.integers(0, 256, words, dtype=np.uint32)),
        "lane_mod4": lane % 4,
        "lane_div16": lane // 16,
        "bank_stride32": (lane % 8) * 32,      # same LDS bank, different words
        "half_waves": (lane >= 32).astype(np.uint32) * 3,
        "reversed_lanes": 63 - lane,
    }


@pytest.mark.parametrize("slots,unit", [(28, 4), (16, 4), (16, 1), (8, 1), (28, 1)])
def test_lds_atomic_lane_order(slots, unit):
    """The property the pass kernel's rank (and the one-launch kernel's)
    relies on: each wave adds `unit` per element to its (wave, digit) LDS
    counter, all slots back to back, and every add must return unit x the
    number of the wave's earlier elements with that digit.  Counter layouts
    and units as in the kernels: 28 and 16 keys per thread with byte units
    (4-byte keys), 16 and 10-like element units, 8 slots for the one-launch
    path; 256 workgroups of 16 waves, so every compute unit runs them under
    contention."""
    rng = np.random.default_rng(4242 + slots * 10 + unit)
    blocks = 256
    words = blocks * 1024 * slots
    for name, digits in _patterns(rng, words, slots).items():
        note(f"lds lane order slots={slots} unit={unit} pattern={name}")
        dd = torch.from_numpy(np.ascontiguousarray(digits.astype(np.uint32))).to("cuda")
        got = rs.lds_rank_probe(dd, slots, unit).cpu().numpy()
        want = _expected_ranks(digits, slots, unit)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (f"{name}: {bad.size} adds returned out-of-order ranks, first at word {bad[0]}: "
                               f"got {got[bad[0]]}, expected {want[bad[0]]}")

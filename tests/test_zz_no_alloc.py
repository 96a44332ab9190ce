"""GPU test of the allocation-free entry point rs_sort_keys_u32_noalloc,
called through the C ABI: its output must equal, bit for bit, that of
rs_sort_keys_u32 with a caller temp buffer (and the CPU oracle's) on
consecutive calls of decreasing size, so a call never depends on what the
previous one left in the shared scratch."""
import ctypes
import sys

import numpy as np
import pytest

import oracle
from lsd_radix_sort_pass_amd import _lib

torch = pytest.importorskip("torch")
rs = pytest.importorskip("lsd_radix_sort_pass_amd")

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def _noalloc(lib, kin, kout, n, b, e):
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.rs_sort_keys_u32_noalloc(ctypes.c_void_p(kin.data_ptr()), ctypes.c_void_p(kout.data_ptr()),
                                        n, b, e, stream)


def _with_temp(lib, kin, kout, n, b, e):
    temp = torch.empty(max(lib.rs_temp_bytes(n, 0, b, e), 1), dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    code = lib.rs_sort_keys_u32(ctypes.c_void_p(kin.data_ptr()), ctypes.c_void_p(kout.data_ptr()), n, b, e,
                                ctypes.c_void_p(temp.data_ptr()), temp.numel(), stream)
    return code, temp


def test_noalloc_matches_temp_entry_point():
    lib = _lib.load()
    rng = np.random.default_rng(77)
    # Largest allowed size first, then smaller multi-launch sizes (ragged
    # tails, a narrower bit range), then the one-launch small path.
    cases = [(rs.NOALLOC_MAX_KEYS, 0, 32), (1_000_003, 0, 32), (300_001, 5, 27), (40_000, 0, 32), (777, 0, 32)]
    for n, b, e in cases:
        note(f"rs_sort_keys_u32_noalloc n={n} bits=[{b},{e})")
        keys = rng.integers(0, 2**32, n, dtype=np.uint32)
        if n == 300_001:
            keys &= np.uint32(0x0FFF00FF)      # a skipped middle pass
        dk = torch.from_numpy(keys).to("cuda")
        out_a = torch.full_like(dk, 0xAB)
        out_b = torch.full_like(dk, 0xCD)
        assert _noalloc(lib, dk, out_a, n, b, e) == _lib.RS_SUCCESS
        code, temp = _with_temp(lib, dk, out_b, n, b, e)
        assert code == _lib.RS_SUCCESS
        torch.cuda.synchronize()
        assert rs.error_word(temp) == 0
        a, bb = out_a.cpu().numpy(), out_b.cpu().numpy()
        assert np.array_equal(a, bb), f"noalloc differs from the temp entry point at n={n}"
        assert np.array_equal(a, oracle.lsd_sort(keys, None, b, e)), f"differs from the oracle at n={n}"
        assert np.array_equal(dk.cpu().numpy(), keys), "input modified"


def test_noalloc_in_place_and_limit():
    lib = _lib.load()
    rng = np.random.default_rng(78)
    for n in (200_000, 70_000):
        note(f"rs_sort_keys_u32_noalloc in place n={n}")
        keys = rng.integers(0, 2**32, n, dtype=np.uint32)
        dk = torch.from_numpy(keys).to("cuda")
        assert _noalloc(lib, dk, dk, n, 0, 24) == _lib.RS_SUCCESS       # 3 passes: odd, copy back
        torch.cuda.synchronize()
        assert np.array_equal(dk.cpu().numpy(), oracle.lsd_sort(keys, None, 0, 24))
    dk = torch.zeros(rs.NOALLOC_MAX_KEYS + 1, dtype=torch.uint32, device="cuda")
    assert _noalloc(lib, dk, dk, dk.numel(), 0, 32) == _lib.RS_ERROR_SCRATCH_LIMIT

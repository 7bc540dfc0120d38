"""The kernels' division-free quotient (small_div in veda_internal.hpp): for
0 <= a < 2^20 and b >= 1, trunc((f32(a) + 0.5) * r) == a // b whenever r is
within one ulp of 1/b, which is what the hardware reciprocal v_rcp_f32
guarantees.  Emulated here in numpy f32 (every operation rounded to nearest,
as the GPU's f32 add and multiply are) for the three candidate values of r,
over every a below 2^20 for the divisors the layouts use (tile extents up to
128, tile-grid sizes up to 256) and over random (a, b) pairs beyond them."""
import numpy as np


def _quotients(a, b):
    r0 = np.float32(1.0) / np.float32(b)
    out = []
    for r in (np.nextafter(r0, np.float32(0)), r0, np.nextafter(r0, np.float32(1e30))):
        x = a.astype(np.float32) + np.float32(0.5)   # exact: a < 2^23
        out.append(np.trunc(x * np.float32(r)).astype(np.int64))
    return out


def test_small_div_exhaustive_small_divisors():
    a = np.arange(1 << 20, dtype=np.int64)
    for b in range(1, 257):
        want = a // b
        for q in _quotients(a, b):
            assert np.array_equal(q, want), b


def test_small_div_random_pairs():
    rng = np.random.default_rng(0)
    for _ in range(200):
        b = int(rng.integers(257, 1 << 20))
        a = rng.integers(0, 1 << 20, size=1 << 14)
        a[:4] = [0, b - 1, b, (1 << 20) - 1]
        for q in _quotients(a, b):
            assert np.array_equal(q, a // b), b

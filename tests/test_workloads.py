"""Checks of the seeded input generator (no method arithmetic here)."""
import math

import numpy as np

import workloads
from workloads import bf16_round, bf16_to_f32, make


def test_bf16_round_to_nearest_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)                  # bf16 spacing at 1.0
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    got = bf16_to_f32(bf16_round(x))
    assert got.tolist() == [1.0, 1.0, float(one + 2 * ulp), -2.5, float(one + ulp)]


def test_deterministic_and_shaped():
    a, b = make("ragged-small", 3), make("ragged-small", 3)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.v, b.v) and np.array_equal(a.w, b.w)
    assert a.tile_shapes == b.tile_shapes
    c = make("ragged-small", 4)
    assert not np.array_equal(a.q, c.q)
    assert a.q.shape == (5 * 9 * 20, 4, 128) and a.q.dtype == np.uint16
    assert a.w.shape == (4, 128, 384) and a.w.dtype == np.float32


def test_length_sweep_keeps_tile_draw():
    short = make("long-720p-241f", 0, T=2)
    full_shapes = workloads.draw_tile_shapes(
        workloads.CONFIGS["long-720p-241f"], workloads._streams(0)["tiles"])
    assert short.tile_shapes == full_shapes
    assert all(s in workloads.TILE_CHOICES for s in full_shapes)


def test_positional_peak_is_alpha():
    rng = np.random.Generator(np.random.PCG64(9))
    sm = 1 / math.sqrt(128)
    pos = workloads.positional_term(3, 4, 5, 128, (4, 4, 8), sm, rng).astype(np.float64)
    self_logit = sm * np.einsum("nd,nd->n", pos, pos)
    np.testing.assert_allclose(self_logit, workloads.POS_ALPHA, rtol=1e-5)
    cross = sm * pos @ pos.T
    assert np.all(cross <= workloads.POS_ALPHA + 1e-4)


def test_subset_draw():
    wl = make("ragged-small", 0)
    sub = workloads.draw_subset(wl, [20, 7, 1])
    assert [s.size for s in sub] == [10, 4, 1]
    assert all(np.all(np.diff(s) > 0) for s in sub)
    again = workloads.draw_subset(wl, [20, 7, 1])
    assert all(np.array_equal(x, y) for x, y in zip(sub, again))


def test_bf16_round_matches_exact_integer_rounding():
    """The uint32 form gives the same bits as the rounding done in exact
    (Python integer) arithmetic, over random values, both signs of zero,
    infinities, NaN payloads near the top of the range, halfway cases, and a
    chunked (multi-threaded) size."""
    rng = np.random.default_rng(11)
    special = np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000,
                        0xFFFFFFFF, 0xFFFF8000, 0x7FFF8000, 0x3F808000, 0x3F818000,
                        0x7F7FFFFF, 0xFF7FFFFF, 0x00008000, 0x00018000], dtype=np.uint32)
    bits = np.concatenate([special, rng.integers(0, 2 ** 32, size=5000, dtype=np.uint32)])
    want = np.array([((int(v) + 0x7FFF + ((int(v) >> 16) & 1)) >> 16) & 0xFFFF for v in bits],
                    dtype=np.uint16)
    assert np.array_equal(bf16_round(bits.view(np.float32)), want)
    big = rng.standard_normal(3 * (1 << 22) + 17, dtype=np.float32)
    b64 = big.view(np.uint32).astype(np.uint64)
    ref = ((b64 + 0x7FFF + ((b64 >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(bf16_round(big), ref)

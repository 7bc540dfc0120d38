"""Pins for the oracle's tiling (gather / scatter / slot map).

Pinned against: a hand-worked example, an independent construction by
padding + reshape + axis transpose, the bijection onto the real tokens, and
the box each tile covers (integer division of token coordinates).
"""
import numpy as np
import pytest

import oracle
from oracle.tiling import HeadTiling


def test_hand_worked_slot_map():
    # Grid T,H,W = 2,3,4; tile (1,2,2): 2x2x2 tiles of 4 slots.
    # Token n = (t*3 + h)*4 + w.  Tile (it,ih,iw) holds t = it, h in {2ih, 2ih+1},
    # w in {2iw, 2iw+1}; h = 3 is outside the grid -> padding (-1).
    expected = [
        0, 1, 4, 5,        # tile 0 (0,0,0)
        2, 3, 6, 7,        # tile 1 (0,0,1)
        8, 9, -1, -1,      # tile 2 (0,1,0): h=2 real, h=3 padding
        10, 11, -1, -1,    # tile 3 (0,1,1)
        12, 13, 16, 17,    # tile 4 (1,0,0): t=1 starts at token 12
        14, 15, 18, 19,    # tile 5
        20, 21, -1, -1,    # tile 6
        22, 23, -1, -1,    # tile 7
    ]
    assert oracle.slot_tokens(2, 3, 4, (1, 2, 2)).tolist() == expected


@pytest.mark.parametrize("T,H,W,shape,n", [
    (21, 30, 52, (4, 4, 8), 336),
    (61, 45, 80, (4, 4, 8), 1920),
    (61, 45, 80, (1, 8, 16), 1830),
    (61, 45, 80, (2, 8, 8), 1860),
    (21, 45, 80, (1, 8, 16), 630),
    (31, 45, 80, (8, 4, 4), 960),
    (4, 8, 8, (4, 4, 4), 4),
])
def test_tile_counts(T, H, W, shape, n):
    g = oracle.tile_grid(T, H, W, shape)
    assert g[0] * g[1] * g[2] == n


def _reshape_construction(T, H, W, shape):
    """Independent slot map: pad the token-index grid, split every axis into
    (tile, offset) and move the three tile axes in front."""
    pt, ph, pw = shape
    nT, nH, nW = -(-T // pt), -(-H // ph), -(-W // pw)
    grid = np.full((nT * pt, nH * ph, nW * pw), -1, dtype=np.int64)
    grid[:T, :H, :W] = np.arange(T * H * W).reshape(T, H, W)
    return grid.reshape(nT, pt, nH, ph, nW, pw).transpose(0, 2, 4, 1, 3, 5).ravel()


@pytest.mark.parametrize("T,H,W,shape", [
    (2, 3, 4, (1, 2, 2)), (4, 8, 8, (4, 4, 4)), (5, 9, 20, (1, 8, 16)), (5, 9, 20, (2, 8, 8)),
    (5, 9, 20, (4, 4, 8)), (5, 9, 20, (8, 4, 4)), (21, 30, 52, (4, 4, 8)), (7, 3, 11, (2, 4, 8)),
])
def test_slot_map_matches_reshape_construction(T, H, W, shape):
    assert np.array_equal(oracle.slot_tokens(T, H, W, shape), _reshape_construction(T, H, W, shape))


@pytest.mark.parametrize("T,H,W,shape", [(5, 9, 20, (8, 4, 4)), (21, 30, 52, (4, 4, 8)), (3, 5, 7, (2, 2, 2))])
def test_bijection_and_boxes(T, H, W, shape):
    perm = oracle.slot_tokens(T, H, W, shape)
    real = perm[perm >= 0]
    assert np.array_equal(np.sort(real), np.arange(T * H * W))     # each token exactly once
    pt, ph, pw = shape
    S = pt * ph * pw
    nT, nH, nW = oracle.tile_grid(T, H, W, shape)
    for j in range(nT * nH * nW):
        it, ih, iw = j // (nH * nW), (j // nW) % nH, j % nW
        toks = perm[j * S:(j + 1) * S]
        toks = toks[toks >= 0]
        t, h, w = toks // (H * W), (toks // W) % H, toks % W
        assert np.all(t // pt == it) and np.all(h // ph == ih) and np.all(w // pw == iw)
        assert toks.size >= 1          # ceil padding never leaves an empty tile


def test_gather_scatter_roundtrip():
    rng = np.random.default_rng(1)
    T, H, W, shape = 5, 9, 20, (2, 8, 8)
    x = rng.standard_normal((T * H * W, 6))
    y = oracle.gather(x, T, H, W, shape)
    perm = oracle.slot_tokens(T, H, W, shape)
    assert np.all(y[perm < 0] == 0.0)
    assert np.array_equal(y[perm >= 0], x[perm[perm >= 0]])
    assert np.array_equal(oracle.scatter(y, T, H, W, shape), x)


def test_head_tiling_fields():
    ht = HeadTiling(5, 9, 20, (1, 8, 16))
    assert ht.S == 128 and ht.grid == (5, 2, 2) and ht.n == 20
    assert ht.valid.sum() == 5 * 9 * 20

"""Pins for the oracle's TripPool, projection and tile score.

Pinned against: a hand-worked tile with a padding slot, numpy masked-array
reductions (np.ma) over the tile-shaped view, shift / negation identities
(catch a mean/max/min mix-up), and closed forms computed straight from the
token-order data with tiles found by integer division of coordinates (no
slot map): with W = [I|0|0] the score is the mean-of-logits sum over the two
tiles' tokens, with W = [0|I|0] it is max_i . max_j, and with W = 0 it is the
bias product.
"""
import numpy as np
import pytest

import oracle
from workloads import bf16_to_f64, make


def test_hand_worked_tripool():
    # Grid 1x1x3, tile (1,1,2), d = 2: tile 0 = tokens 0,1; tile 1 = token 2 + padding.
    x = np.array([[1.0, -2.0], [3.0, 4.0], [5.0, 0.0]])
    xp = oracle.gather(x, 1, 1, 3, (1, 1, 2))
    valid = oracle.valid_slots(1, 1, 3, (1, 1, 2))
    d = oracle.tripool(xp, valid, 2)
    assert d.tolist() == [[2.0, 1.0, 3.0, 4.0, 1.0, -2.0],
                          [5.0, 0.0, 5.0, 0.0, 5.0, 0.0]]   # padding is not averaged in


def _ragged_head(seed=0, head=1):
    wl = make("ragged-small", seed)
    shape = wl.tile_shapes[head]
    q = bf16_to_f64(wl.q[:, head, :])
    k = bf16_to_f64(wl.k[:, head, :])
    return wl, shape, q, k


def test_tripool_matches_masked_array_reductions():
    wl, shape, q, _ = _ragged_head()
    T, H, W = wl.T, wl.config.H, wl.config.W
    xp = oracle.gather(q, T, H, W, shape)
    valid = oracle.valid_slots(T, H, W, shape)
    S = int(np.prod(shape))
    n = xp.shape[0] // S
    d = xp.shape[1]
    ma = np.ma.masked_array(xp.reshape(n, S, d),
                            mask=np.repeat(~valid.reshape(n, S)[:, :, None], d, axis=2))
    ref = np.concatenate([ma.mean(axis=1).data, ma.max(axis=1).data, ma.min(axis=1).data], axis=1)
    got = oracle.tripool(xp, valid, S)
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-14)


def test_tripool_shift_and_negation():
    wl, shape, q, _ = _ragged_head(head=2)
    T, H, W = wl.T, wl.config.H, wl.config.W
    xp = oracle.gather(q, T, H, W, shape)
    valid = oracle.valid_slots(T, H, W, shape)
    S = int(np.prod(shape))
    d = xp.shape[1]
    base = oracle.tripool(xp, valid, S)
    np.testing.assert_allclose(oracle.tripool(xp + 3.5, valid, S), base + 3.5, atol=1e-12)
    neg = oracle.tripool(-xp, valid, S)
    np.testing.assert_allclose(neg[:, :d], -base[:, :d], atol=1e-14)
    assert np.array_equal(neg[:, d:2 * d], -base[:, 2 * d:])       # max(-x) = -min(x)
    assert np.array_equal(neg[:, 2 * d:], -base[:, d:2 * d])
    assert np.all(base[:, d:2 * d] >= base[:, :d] - 1e-12)
    assert np.all(base[:, :d] >= base[:, 2 * d:] - 1e-12)


def test_constant_tile():
    x = np.full((16, 4), 2.25)
    xp = oracle.gather(x, 2, 2, 4, (1, 2, 4))
    valid = oracle.valid_slots(2, 2, 4, (1, 2, 4))
    d = oracle.tripool(xp, valid, 8)
    assert np.all(d == 2.25)


def _tile_of_token(T, H, W, shape):
    pt, ph, pw = shape
    nT, nH, nW = -(-T // pt), -(-H // ph), -(-W // pw)
    n = np.arange(T * H * W)
    t, h, w = n // (H * W), (n // W) % H, n % W
    return ((t // pt) * nH + h // ph) * nW + w // pw, nT * nH * nW


def test_mean_projection_score_closed_form():
    wl, shape, q, k = _ragged_head(head=0)
    T, H, W = wl.T, wl.config.H, wl.config.W
    dm = q.shape[1]
    S = int(np.prod(shape))
    valid = oracle.valid_slots(T, H, W, shape)
    wsel = np.concatenate([np.eye(dm), np.zeros((dm, 2 * dm))], axis=1)   # picks the mean
    phq = oracle.project(oracle.tripool(oracle.gather(q, T, H, W, shape), valid, S), wsel)
    phk = oracle.project(oracle.tripool(oracle.gather(k, T, H, W, shape), valid, S), wsel)
    got = oracle.tile_scores(phq, phk)
    tile, n = _tile_of_token(T, H, W, shape)
    qk = q @ k.T
    ref = np.zeros((n, n))
    for i in range(n):
        for j in range(n):
            blk = qk[np.ix_(tile == i, tile == j)]
            ref[i, j] = blk.sum() / blk.size
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-11)
    assert not np.allclose(ref, ref.T)         # the test can tell a transposed score


def test_max_projection_score_closed_form():
    wl, shape, q, k = _ragged_head(head=3)
    T, H, W = wl.T, wl.config.H, wl.config.W
    dm = q.shape[1]
    S = int(np.prod(shape))
    valid = oracle.valid_slots(T, H, W, shape)
    wsel = np.concatenate([np.zeros((dm, dm)), np.eye(dm), np.zeros((dm, dm))], axis=1)
    phq = oracle.project(oracle.tripool(oracle.gather(q, T, H, W, shape), valid, S), wsel)
    phk = oracle.project(oracle.tripool(oracle.gather(k, T, H, W, shape), valid, S), wsel)
    tile, n = _tile_of_token(T, H, W, shape)
    mq = np.stack([q[tile == i].max(axis=0) for i in range(n)])
    mk = np.stack([k[tile == i].max(axis=0) for i in range(n)])
    np.testing.assert_allclose(oracle.tile_scores(phq, phk), mq @ mk.T, rtol=1e-12, atol=1e-12)


def test_bias_only_projection():
    desc = np.random.default_rng(3).standard_normal((5, 12))
    bq, bk = np.arange(4.0), np.array([1.0, -1.0, 2.0, 0.5])
    s = oracle.tile_scores(oracle.project(desc, np.zeros((4, 12)), bq),
                           oracle.project(desc, np.zeros((4, 12)), bk))
    assert np.all(s == 0 * 1 + 1 * -1 + 2 * 2 + 3 * 0.5)


def test_hand_worked_projection_with_bias():
    desc = np.array([[1.0, 2.0, 3.0]])
    w = np.array([[1.0, 0.0, 0.0], [0.0, 0.0, 1.0]])
    assert oracle.project(desc, w, np.array([10.0, 20.0])).tolist() == [[11.0, 23.0]]
    assert oracle.project(desc, w).tolist() == [[1.0, 3.0]]
    phq = np.array([[1.0, 2.0], [0.0, 1.0]])
    phk = np.array([[3.0, 0.0], [1.0, -1.0], [2.0, 2.0]])
    # score[i][j] = <phi_q[i], phi_k[j]>: query tiles are rows, key tiles columns
    assert oracle.tile_scores(phq, phk).tolist() == [[3.0, -1.0, 6.0], [0.0, -1.0, 2.0]]

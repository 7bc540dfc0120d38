"""Pins for the oracle's two-pass max-pooled attention map.

Pinned against: a hand-worked map, brute force by definition (materialise
the whole attention matrix in token order, then block-max), the pass-1
normaliser summing every row's probabilities to one, the closed form Q = 0
(every entry is 1 / number of real tokens), bounds, and agreement of the
pass-1 log-sum-exp with dense attention's.
"""
import math

import numpy as np
import pytest

import oracle
from workloads import bf16_to_f64, make


def test_hand_worked_map():
    # 1x1x4 grid, tile (1,1,2), d = 1: rows 0,1 see weights 1:3:1:1, rows 2,3 see 1:1:1:1.
    q = np.array([[1.0], [1.0], [0.0], [0.0]])
    k = np.array([[0.0], [math.log(3.0)], [0.0], [0.0]])
    valid = oracle.valid_slots(1, 1, 4, (1, 1, 2))
    lse, M = oracle.maxpool_map(q, k, valid, 2, [0, 1], 1.0)
    np.testing.assert_allclose(M, [[0.5, 1 / 6], [0.25, 0.25]], rtol=1e-15)
    np.testing.assert_allclose(lse, [math.log(6)] * 2 + [math.log(4)] * 2, rtol=1e-15)


def _head(name, head, seed=0):
    wl = make(name, seed)
    T, H, W = wl.T, wl.config.H, wl.config.W
    shape = wl.tile_shapes[head]
    if wl.q32 is not None:
        q, k = wl.q32[:, head, :].astype(np.float64), wl.k32[:, head, :].astype(np.float64)
    else:
        q, k = bf16_to_f64(wl.q[:, head, :]), bf16_to_f64(wl.k[:, head, :])
    ht = oracle.HeadTiling(T, H, W, shape)
    return wl, ht, q, k, oracle.gather(q, T, H, W, shape), oracle.gather(k, T, H, W, shape)


@pytest.mark.parametrize("name,head", [("tiny", 0), ("ragged-small", 0), ("ragged-small", 3),
                                       ("ragged-d64", 0)])
def test_two_pass_equals_brute_force(name, head):
    wl, ht, q, k, qp, kp = _head(name, head)
    tiles = list(range(0, ht.n, 2)) if ht.n > 4 else list(range(ht.n))
    lse, M = oracle.maxpool_map(qp, kp, ht.valid, ht.S, tiles, wl.sm_scale)
    Mb = oracle.maxpool_map_bruteforce(q, k, ht.perm, ht.S, tiles, wl.sm_scale)
    np.testing.assert_allclose(M, Mb, rtol=1e-12, atol=1e-300)
    assert np.all(M > 0) and np.all(M <= 1.0)
    assert np.all(M.max(axis=1) >= 1.0 / q.shape[0])


def test_pass_one_normaliser_sums_rows_to_one():
    wl, ht, q, k, qp, kp = _head("ragged-small", 1)
    tiles = [0, ht.n // 2, ht.n - 1]
    lse, _ = oracle.maxpool_map(qp, kp, ht.valid, ht.S, tiles, wl.sm_scale)
    keys = kp[ht.valid]
    for a, i in enumerate(tiles):
        rows = np.arange(i * ht.S, (i + 1) * ht.S)
        vr = ht.valid[rows]
        p = np.exp(wl.sm_scale * qp[rows[vr]] @ keys.T - lse[a * ht.S:(a + 1) * ht.S][vr][:, None])
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-12)
    _, lsed = oracle.dense_attention(q, k, np.zeros((q.shape[0], 1)), wl.sm_scale)
    for a, i in enumerate(tiles):
        slots = np.arange(i * ht.S, (i + 1) * ht.S)
        vr = ht.valid[slots]
        np.testing.assert_allclose(lse[a * ht.S:(a + 1) * ht.S][vr], lsed[ht.perm[slots[vr]]], rtol=1e-12)


def test_q_zero_closed_form():
    wl, ht, q, k, qp, kp = _head("ragged-small", 2)
    lse, M = oracle.maxpool_map(np.zeros_like(qp), kp, ht.valid, ht.S, [0, 1, ht.n - 1], wl.sm_scale)
    np.testing.assert_allclose(M, 1.0 / q.shape[0], rtol=1e-13)
    np.testing.assert_allclose(lse[~np.isnan(lse)], math.log(q.shape[0]), rtol=1e-14)


def test_hand_worked_map_with_padding():
    # 1x1x3 grid, tile (1,1,2): tile 0 = tokens 0,1; tile 1 = token 2 + a padding slot.
    # q = 1 and k = (-1, -2, -3): every real row has probabilities e^-1, e^-2, e^-3 over Z.
    # A padding key (logit 0) or a padding query row (uniform 1/3) must not enter the max.
    q = np.ones((3, 1))
    k = np.array([[-1.0], [-2.0], [-3.0]])
    qp, kp = oracle.gather(q, 1, 1, 3, (1, 1, 2)), oracle.gather(k, 1, 1, 3, (1, 1, 2))
    valid = oracle.valid_slots(1, 1, 3, (1, 1, 2))
    Z = math.exp(-1) + math.exp(-2) + math.exp(-3)
    lse, M = oracle.maxpool_map(qp, kp, valid, 2, [0, 1], 1.0)
    np.testing.assert_allclose(M, [[math.exp(-1) / Z, math.exp(-3) / Z]] * 2, rtol=1e-14)
    np.testing.assert_allclose(lse[:3], math.log(Z), rtol=1e-14)
    assert np.isnan(lse[3])
    Mb = oracle.maxpool_map_bruteforce(q, k, oracle.slot_tokens(1, 1, 3, (1, 1, 2)), 2, [0, 1], 1.0)
    np.testing.assert_allclose(Mb, M, rtol=1e-14)

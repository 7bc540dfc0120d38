"""Pins for the oracle's block-sparse attention.

Pinned against: hand-worked logits with closed-form outputs (including a
padding key that must not count), dense attention in token order with no
tiling (every tile kept), torch's CPU float64 scaled_dot_product_attention
with a boolean mask built from the CSR, scipy softmax / logsumexp on a single
kept tile, and the closed forms Q = 0 (mean of the kept values) and V = 1.
"""
import math

import numpy as np
import pytest
import scipy.special

import oracle
from workloads import bf16_to_f64, make


def _csr(rows):
    rp = np.cumsum([0] + [len(r) for r in rows])
    return rp, np.concatenate([np.asarray(r, dtype=np.int64) for r in rows])


def test_hand_worked_sparse_and_dense():
    # 1x1x4 grid, tile (1,1,2), d = 1, sm_scale = 1; tile 0 = tokens 0,1, tile 1 = tokens 2,3.
    q = np.ones((4, 1))
    k = np.array([[0.0], [math.log(3.0)], [0.0], [0.0]])
    v = np.array([[1.0], [2.0], [3.0], [4.0]])
    o, lse = oracle.dense_attention(q, k, v, 1.0)
    np.testing.assert_allclose(o[:, 0], 14.0 / 6.0, rtol=1e-15)       # weights 1:3:1:1
    np.testing.assert_allclose(lse, math.log(6.0), rtol=1e-15)
    valid = oracle.valid_slots(1, 1, 4, (1, 1, 2))
    rp, ci = _csr([[0], [1]])                                         # tile 0 keeps 0, tile 1 keeps 1
    o, lse = oracle.sparse_attention(q, k, v, valid, 2, rp, ci, 1.0)
    np.testing.assert_allclose(o[:, 0], [7 / 4, 7 / 4, 7 / 2, 7 / 2], rtol=1e-15)
    np.testing.assert_allclose(lse, [math.log(4)] * 2 + [math.log(2)] * 2, rtol=1e-15)


def test_hand_worked_padding_key_is_masked():
    # 1x1x3 grid, tile (1,1,2): tile 1 = token 2 + a padding slot (k = 0, v = 0).
    q = np.ones((3, 1))
    k = np.array([[0.0], [math.log(3.0)], [math.log(2.0)]])
    v = np.array([[1.0], [2.0], [3.0]])
    valid = oracle.valid_slots(1, 1, 3, (1, 1, 2))
    qp, kp, vp = (oracle.gather(a, 1, 1, 3, (1, 1, 2)) for a in (q, k, v))
    rp, ci = _csr([[1], [1]])
    o, lse = oracle.sparse_attention(qp, kp, vp, valid, 2, rp, ci, 1.0)
    np.testing.assert_allclose(o[:3, 0], 3.0, rtol=1e-15)             # only token 2; padding excluded
    np.testing.assert_allclose(lse[:3], math.log(2.0), rtol=1e-15)
    assert np.isnan(o[3, 0]) and np.isnan(lse[3])                     # padding query row unspecified
    rp, ci = _csr([[0, 1], [0, 1]])
    o, lse = oracle.sparse_attention(qp, kp, vp, valid, 2, rp, ci, 1.0)
    np.testing.assert_allclose(o[:3, 0], 13.0 / 6.0, rtol=1e-15)      # weights 1:3:2


def _head(name, head, seed=0):
    wl = make(name, seed)
    T, H, W = wl.T, wl.config.H, wl.config.W
    shape = wl.tile_shapes[head]
    if wl.q32 is not None:
        q, k, v = (a[:, head, :].astype(np.float64) for a in (wl.q32, wl.k32, wl.v32))
    else:
        q, k, v = (bf16_to_f64(a[:, head, :]) for a in (wl.q, wl.k, wl.v))
    ht = oracle.HeadTiling(T, H, W, shape)
    g = lambda a: oracle.gather(a, T, H, W, shape)
    return wl, ht, q, k, v, g(q), g(k), g(v)


@pytest.mark.parametrize("name,head", [("tiny", 0), ("ragged-small", 0), ("ragged-small", 1),
                                       ("ragged-small", 2), ("ragged-small", 3), ("ragged-d64", 1)])
def test_zero_sparsity_equals_dense(name, head):
    wl, ht, q, k, v, qp, kp, vp = _head(name, head)
    n = ht.n
    rp = np.arange(n + 1) * n
    ci = np.tile(np.arange(n), n)
    o, lse = oracle.sparse_attention(qp, kp, vp, ht.valid, ht.S, rp, ci, wl.sm_scale)
    od, lsed = oracle.dense_attention(q, k, v, wl.sm_scale)
    np.testing.assert_allclose(oracle.scatter(np.nan_to_num(o), wl.T, wl.config.H, wl.config.W, ht.shape),
                               od, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[ht.valid], lsed[ht.perm[ht.valid]], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("name,head,s", [("ragged-small", 1, 75), ("ragged-small", 3, 60),
                                         ("ragged-d64", 2, 60), ("tiny", 0, 50)])
def test_matches_torch_sdpa_with_block_mask(name, head, s):
    torch = pytest.importorskip("torch")
    wl, ht, q, k, v, qp, kp, vp = _head(name, head)
    rng = np.random.default_rng(head + s)
    kk = oracle.keep_count(ht.n, s)
    rp, ci = oracle.select_topk(rng.standard_normal((ht.n, ht.n)), kk)
    o, lse = oracle.sparse_attention(qp, kp, vp, ht.valid, ht.S, rp, ci, wl.sm_scale)
    mask = oracle.csr_to_block_mask(rp, ci, ht.valid, ht.S)
    t = lambda a: torch.from_numpy(a)[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        t(qp), t(kp), t(vp), attn_mask=t(mask), scale=wl.sm_scale)[0, 0].numpy()
    np.testing.assert_allclose(o[ht.valid], ref[ht.valid], rtol=1e-11, atol=1e-12)


def test_single_kept_tile_is_plain_softmax():
    wl, ht, q, k, v, qp, kp, vp = _head("ragged-small", 2)
    S, n = ht.S, ht.n
    rng = np.random.default_rng(7)
    pick = rng.integers(0, n, size=n)
    rp, ci = np.arange(n + 1), pick.astype(np.int64)
    o, lse = oracle.sparse_attention(qp, kp, vp, ht.valid, S, rp, ci, wl.sm_scale)
    for i in range(n):
        qs = np.arange(i * S, (i + 1) * S)[ht.valid[i * S:(i + 1) * S]]
        ks = np.arange(pick[i] * S, (pick[i] + 1) * S)[ht.valid[pick[i] * S:(pick[i] + 1) * S]]
        lg = wl.sm_scale * qp[qs] @ kp[ks].T
        np.testing.assert_allclose(o[qs], scipy.special.softmax(lg, axis=1) @ vp[ks], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[qs], scipy.special.logsumexp(lg, axis=1), rtol=1e-13)


def test_closed_forms_q_zero_and_v_one():
    wl, ht, q, k, v, qp, kp, vp = _head("ragged-small", 0)
    S, n = ht.S, ht.n
    kk = oracle.keep_count(n, 75)
    rp, ci = oracle.select_topk(np.random.default_rng(2).standard_normal((n, n)), kk)
    o, lse = oracle.sparse_attention(np.zeros_like(qp), kp, vp, ht.valid, S, rp, ci, wl.sm_scale)
    for i in range(n):
        keys = np.concatenate([np.arange(j * S, (j + 1) * S) for j in ci[rp[i]:rp[i + 1]]])
        keys = keys[ht.valid[keys]]
        qs = np.arange(i * S, (i + 1) * S)[ht.valid[i * S:(i + 1) * S]]
        np.testing.assert_allclose(o[qs], np.broadcast_to(vp[keys].mean(axis=0), (qs.size, vp.shape[1])),
                                   rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[qs], math.log(keys.size), rtol=1e-14)
    o1, _ = oracle.sparse_attention(qp, kp, np.ones_like(vp), ht.valid, S, rp, ci, wl.sm_scale)
    np.testing.assert_allclose(o1[ht.valid], 1.0, rtol=1e-13)

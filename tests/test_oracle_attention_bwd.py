"""Pins for the oracle's attention backward (oracle/attention_bwd).

Pinned against:
  * central finite differences in fp64 of L = sum(o * do), o from the pinned
    forward oracle (oracle.sparse_attention), for every real entry of Q, K and
    V, on a grid with padding slots and a CSR that lists one tile twice;
  * torch CPU fp64 autograd of a masked dense formulation (the CSR expanded to
    a slot mask with oracle.csr_to_block_mask, -inf logits outside it), an
    independent library derivative;
  * 0 % sparsity: the gradients of dense attention in token order, by torch
    autograd, after the oracle's gather;
  * padding slots and empty rows get zero gradients.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.attention_bwd import sparse_attention_bwd

T, H, W, SHAPE = 2, 3, 4, (1, 2, 2)     # 2 x 2 x 2 tiles of 4 slots, padding in h


def _problem(seed, d=3):
    rng = np.random.default_rng(seed)
    N = T * H * W
    q, k, v, do = (rng.normal(size=(N, d)) for _ in range(4))
    g = lambda a: oracle.gather(a, T, H, W, SHAPE)
    ht = oracle.HeadTiling(T, H, W, SHAPE)
    return ht, g(q), g(k), g(v), g(do)


def _loss(qp, kp, vp, dop, ht, rp, ci, scale):
    o, _ = oracle.sparse_attention(qp, kp, vp, ht.valid, ht.S, rp, ci, scale)
    return float(np.nansum(o * dop))


def test_finite_differences_with_a_repeated_tile():
    ht, qp, kp, vp, dop = _problem(0)
    n = ht.n
    rows = [[0, 3, 3], [1], [2, 5, 6], [0, 7], [4], [1, 2, 3, 4], [6], [5, 7]]
    assert len(rows) == n
    rp = np.cumsum([0] + [len(r) for r in rows])
    ci = np.array(sum(rows, []))
    scale = 0.7
    dq, dk, dv = sparse_attention_bwd(qp, kp, vp, ht.valid, ht.S, rp, ci, scale, dop)
    h = 1e-6
    for x, g in ((qp, dq), (kp, dk), (vp, dv)):
        for s in np.flatnonzero(ht.valid):
            for c in range(x.shape[1]):
                orig = x[s, c]
                x[s, c] = orig + h
                up = _loss(qp, kp, vp, dop, ht, rp, ci, scale)
                x[s, c] = orig - h
                dn = _loss(qp, kp, vp, dop, ht, rp, ci, scale)
                x[s, c] = orig
                assert abs((up - dn) / (2 * h) - g[s, c]) < 1e-7, (s, c)
    pad = ~ht.valid
    for g in (dq, dk, dv):
        assert np.all(g[pad] == 0)


def test_matches_torch_autograd_of_the_masked_softmax():
    ht, qp, kp, vp, dop = _problem(1, d=5)
    rng = np.random.default_rng(2)
    s = rng.normal(size=(ht.n, ht.n))
    rp, ci = oracle.select_topk(s, 3)
    scale = 0.4
    dq, dk, dv = sparse_attention_bwd(qp, kp, vp, ht.valid, ht.S, rp, ci, scale, dop)
    mask = torch.from_numpy(oracle.csr_to_block_mask(rp, ci, ht.valid, ht.S))
    real = torch.from_numpy(ht.valid)
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (qp, kp, vp))
    logits = (scale * tq @ tk.T).masked_fill(~mask, float("-inf"))
    p = torch.softmax(logits[real], dim=1)
    o = p @ tv
    (o * torch.from_numpy(dop)[real]).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_zero_sparsity_is_dense_attention_gradient():
    rng = np.random.default_rng(3)
    N, d = T * H * W, 4
    q, k, v, do = (rng.normal(size=(N, d)) for _ in range(4))
    ht = oracle.HeadTiling(T, H, W, SHAPE)
    g = lambda a: oracle.gather(a, T, H, W, SHAPE)
    rp, ci = oracle.select_topk(np.zeros((ht.n, ht.n)), ht.n)
    dq, dk, dv = sparse_attention_bwd(g(q), g(k), g(v), ht.valid, ht.S, rp, ci, 0.9, g(do))
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    o = torch.softmax(0.9 * tq @ tk.T, dim=1) @ tv
    (o * torch.from_numpy(do)).sum().backward()
    for got, ref in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(oracle.scatter(got, T, H, W, SHAPE), ref.grad.numpy(),
                                   rtol=1e-10, atol=1e-12)


def test_empty_row_gets_zero_gradient():
    ht, qp, kp, vp, dop = _problem(4)
    rows = [[], [1], [2], [3], [4], [5], [6], [7]]
    rp = np.cumsum([0] + [len(r) for r in rows])
    ci = np.array(sum(rows, []), dtype=np.int64)
    dq, dk, dv = sparse_attention_bwd(qp, kp, vp, ht.valid, ht.S, rp, ci, 0.5, dop)
    assert np.all(dq[:ht.S] == 0)
    # tile 0's keys are kept by no row: their gradients are zero too
    assert np.all(dk[:ht.S] == 0) and np.all(dv[:ht.S] == 0)

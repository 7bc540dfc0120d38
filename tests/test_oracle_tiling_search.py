"""Pins for the oracle's head-aware tiling search (oracle/tiling_search).

Pinned against:
  * exactness: at 0 % sparsity every candidate reproduces full attention, so
    every error is 0 (R14), on a grid no candidate divides;
  * a case with a known answer: queries and keys are a large multiple of a
    one-hot code of their (1,2,4) box, so full attention stays inside the box;
    with k = 1 and a mean-feature projection, the (1,2,4) tiling keeps exactly
    each box (error ~ 0) and every other shape splits boxes (error > 0);
  * the sparse output recomputed independently: the CSR expanded to a
    token-order (query, key) mask through the slot map, then a masked softmax;
  * the tie rule: a candidate listed twice is chosen at its first position.
"""
import numpy as np

import oracle
from oracle import tiling_search as ts

CANDS8 = [(1, 2, 4), (2, 2, 2), (1, 1, 8), (2, 1, 4)]


def _box_problem(alpha=8.0):
    T, H, W = 2, 4, 8
    N = T * H * W
    box = np.array([((t // 1) * (H // 2) + h // 2) * (W // 4) + w // 4
                    for t in range(T) for h in range(H) for w in range(W)])
    nbox = box.max() + 1
    d = nbox
    q = np.zeros((N, d)); q[np.arange(N), box] = alpha
    k = q.copy()
    v = np.random.default_rng(0).normal(size=(N, d))
    w = np.zeros((d, 3 * d)); w[:, :d] = np.eye(d)          # phi = tile mean
    return T, H, W, q, k, v, w


def test_zero_sparsity_is_exact_for_every_shape():
    rng = np.random.default_rng(1)
    T, H, W, d = 3, 5, 7, 6
    q, k, v = (rng.normal(size=(T * H * W, d)) for _ in range(3))
    w = rng.normal(0, 0.1, size=(d, 3 * d))
    errs, ref, _ = ts.search_head(q, k, v, T, H, W, CANDS8, w, w, None, None, 0.4, 0)
    assert ref > 0
    assert np.all(errs <= 1e-20 * ref)


def test_box_local_attention_picks_the_box_shape():
    T, H, W, q, k, v, w = _box_problem()
    errs, ref, best = ts.search_head(q, k, v, T, H, W, CANDS8, w, w, None, None, 1.0, 90)
    assert best == 0
    assert errs[0] <= 1e-20 * ref                    # exp(-64) leakage only
    assert np.all(errs[1:] > 1e-2 * ref)


def test_sparse_output_matches_token_order_block_mask():
    rng = np.random.default_rng(2)
    T, H, W, d = 3, 5, 7, 6
    q, k, v = (rng.normal(size=(T * H * W, d)) for _ in range(3))
    w = rng.normal(0, 0.3, size=(d, 3 * d))
    b = rng.normal(0, 0.1, size=d)
    for shape in CANDS8:
        got = ts.sparse_head_output(q, k, v, T, H, W, shape, w, w, b, b, 0.5, 60)
        # independent route: selection -> slot mask -> token-order mask
        ht = oracle.HeadTiling(T, H, W, shape)
        qp, kp = (oracle.gather(a, T, H, W, shape) for a in (q, k))
        s = oracle.tile_scores(oracle.project(oracle.tripool(qp, ht.valid, ht.S), w, b),
                               oracle.project(oracle.tripool(kp, ht.valid, ht.S), w, b))
        rp, ci = oracle.select_topk(s, oracle.keep_count(ht.n, 60))
        slot_mask = oracle.csr_to_block_mask(rp, ci, ht.valid, ht.S)
        tok = oracle.slot_tokens(T, H, W, shape)
        N = T * H * W
        mask = np.zeros((N, N), bool)
        rs, cs = np.nonzero(slot_mask)
        real = tok[rs] >= 0                      # padding query slots have no token
        mask[tok[rs[real]], tok[cs[real]]] = True
        logits = np.where(mask, 0.5 * q @ k.T, -np.inf)
        p = np.exp(logits - logits.max(axis=1, keepdims=True))
        ref = (p / p.sum(axis=1, keepdims=True)) @ v
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_ties_prefer_the_first_candidate():
    T, H, W, q, k, v, w = _box_problem()
    cands = [(2, 2, 2), (1, 1, 8), (2, 2, 2)]
    errs, _, best = ts.search_head(q, k, v, T, H, W, cands, w, w, None, None, 1.0, 90)
    assert errs[0] == errs[2] and best in (0, 1) and best != 2

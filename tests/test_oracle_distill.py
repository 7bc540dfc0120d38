"""Pins for the oracle's distillation objective and gradients (oracle/distill).

Pinned against:
  * scipy.special.rel_entr (KL of two distributions, an independent library
    routine), on random rows, including zeros in the reference;
  * a hand-worked two-tile row (closed form 0.5 ln(4/3));
  * invariants: KL = 0 when the scores are log t + c; unchanged by adding a
    constant to a score row or scaling a map row; never negative;
  * central finite differences of the loss in fp64 for every entry of W_q,
    W_k, b_q, b_k (the loss as a function of the parameters, through the
    estimator forward), with repeated subset rows;
  * constant score rows (all key descriptors equal): every gradient is zero
    and the loss is the KL against the uniform distribution.
"""
import numpy as np
import pytest
from scipy.special import rel_entr

import oracle
from oracle import distill


def test_kl_matches_scipy_rel_entr():
    rng = np.random.default_rng(0)
    s = rng.normal(0, 2, size=(7, 11))
    m = rng.uniform(0, 1, size=(7, 11))
    m[2, [0, 5, 6]] = 0.0                      # zero reference entries
    got = distill.kl_rows(s, m)
    p = np.exp(s) / np.exp(s).sum(axis=1, keepdims=True)
    t = m / m.sum(axis=1, keepdims=True)
    ref = rel_entr(t, p).sum(axis=1)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_hand_worked_two_tiles():
    # p = [1/4, 3/4], t = [1/2, 1/2]: KL = 1/2 ln 2 + 1/2 ln(2/3) = 1/2 ln(4/3)
    got = distill.kl_rows(np.array([[0.0, np.log(3.0)]]), np.array([[0.3, 0.3]]))
    assert abs(got[0] - 0.5 * np.log(4.0 / 3.0)) < 1e-15


def test_invariants():
    rng = np.random.default_rng(1)
    m = rng.uniform(0.01, 1, size=(5, 9))
    t = m / m.sum(axis=1, keepdims=True)
    c = rng.normal(size=(5, 1))
    assert np.abs(distill.kl_rows(np.log(t) + c, m)).max() < 1e-13       # p = t
    s = rng.normal(size=(5, 9))
    base = distill.kl_rows(s, m)
    assert np.all(base > 0)
    np.testing.assert_allclose(distill.kl_rows(s + c, m), base, rtol=1e-12)
    np.testing.assert_allclose(distill.kl_rows(s, m * 37.5), base, rtol=1e-12)
    # a reference concentrated on one tile: KL = -log p of that tile
    one = np.zeros((1, 9)); one[0, 4] = 2.0
    z = s[:1] - s[:1].max()
    assert abs(distill.kl_rows(s[:1], one)[0] + (z[0, 4] - np.log(np.exp(z).sum()))) < 1e-12


def _problem(seed=2, n=6, d3=12, de=5):
    rng = np.random.default_rng(seed)
    desc_q = rng.normal(size=(n, d3))
    desc_k = rng.normal(size=(n, d3))
    w_q = rng.normal(0, 0.3, size=(de, d3))
    w_k = rng.normal(0, 0.3, size=(de, d3))
    b_q = rng.normal(0, 0.2, size=de)
    b_k = rng.normal(0, 0.2, size=de)
    rows = [0, 3, 3, 5]                          # a repeated subset row
    m = rng.uniform(0, 1, size=(len(rows), n))
    m[1, 2] = 0.0
    return desc_q, desc_k, w_q, w_k, b_q, b_k, rows, m


def _loss(desc_q, desc_k, w_q, w_k, b_q, b_k, rows, m, R):
    # the objective written out from its definition (R21-R23): estimator
    # forward, then the mean row KL against the normalised map rows
    s = oracle.tile_scores(oracle.project(desc_q, w_q, b_q), oracle.project(desc_k, w_k, b_k))
    return sum(rel_entr(mr / mr.sum(), np.exp(s[r]) / np.exp(s[r]).sum()).sum()
               for r, mr in zip(rows, m)) / R


@pytest.mark.parametrize("which", ["w_q", "w_k", "b_q", "b_k"])
def test_gradients_match_finite_differences(which):
    desc_q, desc_k, w_q, w_k, b_q, b_k, rows, m = _problem()
    R = 7                                        # rows of other heads count in R
    loss, dw_q, dw_k, db_q, db_k = distill.distill_head(desc_q, desc_k, w_q, w_k, b_q, b_k,
                                                        rows, m, R)
    params = dict(w_q=w_q, w_k=w_k, b_q=b_q, b_k=b_k)
    grads = dict(w_q=dw_q, w_k=dw_k, b_q=db_q, b_k=db_k)
    assert abs(loss - _loss(desc_q, desc_k, w_q, w_k, b_q, b_k, rows, m, R)) < 1e-13
    x = params[which]
    fd = np.zeros_like(x)
    h = 1e-6
    for idx in np.ndindex(x.shape):
        orig = x[idx]
        x[idx] = orig + h
        up = _loss(desc_q, desc_k, w_q, w_k, b_q, b_k, rows, m, R)
        x[idx] = orig - h
        dn = _loss(desc_q, desc_k, w_q, w_k, b_q, b_k, rows, m, R)
        x[idx] = orig
        fd[idx] = (up - dn) / (2 * h)
    np.testing.assert_allclose(grads[which], fd, rtol=1e-6, atol=1e-9)


def test_shared_weights_gradient_is_the_sum():
    # one weight set for both sides: d/dW of L(W, W) = dW_q + dW_k
    desc_q, desc_k, w_q, _, b_q, _, rows, m = _problem(seed=3)
    R = 4
    _, dw_q, dw_k, _, _ = distill.distill_head(desc_q, desc_k, w_q, w_q, b_q, b_q, rows, m, R)
    h = 1e-6
    for idx in [(0, 0), (2, 7), (4, 11)]:
        w = w_q.copy(); w[idx] += h
        up = _loss(desc_q, desc_k, w, w, b_q, b_q, rows, m, R)
        w[idx] -= 2 * h
        dn = _loss(desc_q, desc_k, w, w, b_q, b_q, rows, m, R)
        assert abs((up - dn) / (2 * h) - (dw_q + dw_k)[idx]) < 1e-8


def test_constant_score_rows_have_zero_gradient():
    # softmax ignores a constant added to a score row.  With every key tile's
    # descriptor equal, each score row is constant whatever W and b are, so
    # every gradient vanishes and the loss is the KL against the uniform
    # distribution.
    desc_q, desc_k, w_q, w_k, b_q, b_k, rows, m = _problem(seed=4)
    desc_k_const = np.ones_like(desc_k)
    loss, dw_q, dw_k, db_q, db_k = distill.distill_head(desc_q, desc_k_const, w_q, w_k, b_q,
                                                        b_k, rows, m, 4)
    for g in (dw_q, dw_k, db_q, db_k):
        assert np.abs(g).max() < 1e-15
    t = m / m.sum(axis=1, keepdims=True)
    ref = sum(rel_entr(tr, np.full(tr.size, 1.0 / tr.size)).sum() for tr in t) / 4
    assert abs(loss - ref) < 1e-13

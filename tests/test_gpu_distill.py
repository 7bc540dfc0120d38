"""GPU parity of the distillation step (veda_distill_grad) against the oracle.

The GPU computes the estimator forward (fused gather + TripPool, projection
and score), the max-pooled map of a subset of query tiles, then the row-wise
KL loss and the projection gradients.  The oracle (oracle.distill_head, fp64)
gets the GPU's own descriptors and map, so the step is checked on its own.

Bars, from f32 arithmetic: the loss within 1e-5 relative; each head's weight
and bias gradients within 1e-5 of the largest term magnitude that feeds them
(G = (p - t)/R sums to zero along a row, so gradients are differences of
terms of size |G| |phi| |desc|, and f32 rounding is relative to those terms).
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_common import Run, host, need_gpu, to_dev_f32

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _run(r, q_list, wq, wk, bq, bk):
    torch = need_gpu()
    ly = r.layer
    ly.permute_pool_inputs(r.q, r.k, r.v)
    dev = lambda a: None if a is None else to_dev_f32(a)
    ly.score_from_desc(dev(wq), dev(wk), dev(bq), dev(bk))
    qt = torch.tensor(np.asarray(q_list, np.int32), device="cuda")
    _, mp = ly.maxpool_map(qt, r.sm_scale)
    loss, grads = ly.distill_grad(qt, mp)
    torch.cuda.synchronize()
    return float(host(loss)[0]), [host(g) for g in grads], host(mp)


def _check(r, q_list, wq, wk, bq, bk):
    L = r.L
    loss, (gwq, gwk, gbq, gbk), mp = _run(r, q_list, wq, wk, bq, bk)
    tot, d, mt = L.total_tiles, r.d, L.max_tiles
    desc = host(r.layer.desc).reshape(2, tot, 3 * d).astype(np.float64)
    phi = host(r.layer.phi).reshape(2, tot, -1).astype(np.float64)
    mp = mp.reshape(len(q_list), mt).astype(np.float64)
    valid = [s for s, g in enumerate(q_list) if 0 <= g < tot]
    R = len(valid)
    ref_loss, worst = 0.0, 0.0
    for h in range(r.heads):
        a, b = int(L.tile_off[h]), int(L.tile_off[h + 1])
        n = b - a
        ents = [s for s in valid if a <= q_list[s] < b]
        rows = [q_list[s] - a for s in ents]
        f = lambda x: None if x is None else x[h].astype(np.float64)
        lh, dwq, dwk, dbq, dbk = oracle.distill_head(desc[0, a:b], desc[1, a:b], f(wq), f(wk),
                                                     f(bq), f(bk), rows, mp[ents, :n], R)
        ref_loss += lh
        # size of the terms each gradient sums: each G row has sum |G| <= 2/R,
        # so dW_q sums terms up to |G| |phi_k| |desc_q| and dW_k up to
        # |G| |phi_q| |desc_k| (the biases without the descriptor factor)
        g_abs = 2.0 * len(ents) / max(R, 1)
        sb_q = g_abs * np.abs(phi[1, a:b]).max()
        sb_k = g_abs * np.abs(phi[0, a:b]).max()
        sw_q = sb_q * np.abs(desc[0, a:b]).max()
        sw_k = sb_k * np.abs(desc[1, a:b]).max()
        for got, ref, sc in ((gwq[h], dwq, sw_q), (gwk[h], dwk, sw_k),
                             (gbq[h], dbq, sb_q), (gbk[h], dbk, sb_k)):
            err = np.abs(got - ref).max()
            worst = max(worst, err / max(sc, 1e-30))
            assert err <= 1e-5 * sc + 1e-12, (h, err, sc)
    assert abs(loss - ref_loss) <= 1e-5 * abs(ref_loss) + 1e-9, (loss, ref_loss)
    return loss, ref_loss, worst


def test_distill_ragged_separate_projections_with_bias():
    """Heterogeneous per-head tiles with padding; separate W_q, W_k with biases;
    the subset repeats an entry and holds two out-of-range entries."""
    _say("distill ragged-small")
    r = Run("ragged-small")
    L = r.L
    rng = np.random.default_rng(21)
    de = r.layer.d_e
    shape = (r.heads, de, 3 * r.d)
    wq = rng.normal(0, 0.02, size=shape).astype(np.float32)
    wk = rng.normal(0, 0.02, size=shape).astype(np.float32)
    bq = rng.normal(0, 0.1, size=(r.heads, de)).astype(np.float32)
    bk = rng.normal(0, 0.1, size=(r.heads, de)).astype(np.float32)
    q_list = []
    for h in range(r.heads):
        a, n = int(L.tile_off[h]), L.n(h)
        q_list += [a, a + n - 1, a + n // 2]
    q_list += [q_list[1], -1, L.total_tiles + 3]
    loss, ref, worst = _check(r, q_list, wq, wk, bq, bk)
    _say(f"  loss {loss:.6e} (oracle {ref:.6e}), worst gradient error / term size {worst:.2e}")


def test_distill_bench_config():
    """The Wan-1.3B-like layer with the workload's seeded 10 % subset and one
    weight set for both sides, as the benchmark runs it."""
    _say("distill wan1.3b")
    r = Run("wan1.3b-480p-81f", sparsity=90)
    L = r.L
    subset = workloads.draw_subset(r.wl, [L.n(h) for h in range(L.num_heads)])
    q_list = [int(L.tile_off[h]) + int(j) for h, s in enumerate(subset) for j in s]
    w = r.wl.w
    loss, ref, worst = _check(r, q_list, w, w, None, None)
    _say(f"  loss {loss:.6e} (oracle {ref:.6e}), worst gradient error / term size {worst:.2e}")


def test_distill_no_valid_entries():
    """Only out-of-range entries: loss and every gradient are 0."""
    _say("distill empty")
    r = Run("tiny")
    w = r.wl.w
    loss, grads, _ = _run(r, [-5, r.L.total_tiles], w, w, None, None)
    assert loss == 0.0
    for g in grads:
        assert np.all(g == 0)


def test_distill_deterministic():
    _say("distill determinism")
    r = Run("ragged-small")
    w = r.wl.w
    q_list = [0, 1, 2, 3, int(r.L.tile_off[1]), int(r.L.tile_off[1]) + 1]
    a = _run(r, q_list, w, w, None, None)
    b = _run(r, q_list, w, w, None, None)
    assert a[0] == b[0]
    for x, y in zip(a[1], b[1]):
        assert np.array_equal(x, y)

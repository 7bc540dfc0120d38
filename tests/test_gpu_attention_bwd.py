"""GPU parity of the attention backward (veda_sparse_attn_bwd) against the
oracle (oracle.sparse_attention_bwd, fp64) on the GPU's own CSR.

The GPU rounds P and dS to bf16 for the matrix products (as the forward
rounds P), uses the forward's bf16 O in D = dO . O, and writes bf16
gradients.  Bars, relative to the largest magnitude of each reference
gradient of a head, G = max |ref|:  max |gpu - ref| <= 2e-2 G and mean
|gpu - ref| <= 2e-3 G.  (bf16 rounding is 2^-9 = 2e-3 relative per operand;
sums of a few hundred such terms with random signs stay well inside 2e-2 of
the largest entry.)
"""
import numpy as np
import pytest

import oracle
from gpu_common import Run, bf16_bits, bf16_f64, need_gpu, to_dev_bf16
from workloads import bf16_round, bf16_to_f64

pytestmark = pytest.mark.gpu

REL_MAX, REL_MEAN = 2e-2, 2e-3


def _say(msg):
    print(msg, flush=True)


def _forward_backward(r, seed=7):
    torch = need_gpu()
    out = r.forward_fused()
    rng = np.random.default_rng(seed)
    do = bf16_round(rng.normal(size=(r.wl.q.shape[0], r.heads, r.d)).astype(np.float32))
    d_out = to_dev_bf16(do)
    grads = r.layer.backward(r.q, r.k, r.v, out, d_out, r.sm_scale)
    torch.cuda.synchronize()
    return out, do, grads


def _compare(name, got, ref, sel):
    g = np.abs(ref[sel]).max()
    err = np.abs(got[sel] - ref[sel])
    assert err.max() <= REL_MAX * g + 1e-6, (name, err.max(), g)
    assert err.mean() <= REL_MEAN * g + 1e-7, (name, err.mean(), g)
    return err.max() / max(g, 1e-30)


def _check_head(r, h, do, grads, rp, ci, q_sel=None, k_sel=None):
    """Oracle backward of head h on CSR (rp, ci); compare dQ on the real slots
    of query tiles q_sel and dK, dV on those of key tiles k_sel (all if None)."""
    ht = r.tilings[h]
    qp, kp, vp = r.head_perm(h)
    g = lambda a: oracle.gather(a, r.T, r.H, r.W, ht.shape)
    dop = g(bf16_to_f64(do[:, h, :]))
    dq, dk, dv = oracle.sparse_attention_bwd(qp, kp, vp, ht.valid, r.S, rp, ci, r.sm_scale, dop)
    gq, gk, gv = (g(bf16_f64(t)[:, h, :]) for t in grads)
    S = r.S

    def slots(tiles):
        if tiles is None:
            return ht.valid
        m = np.zeros_like(ht.valid)
        for j in tiles:
            m[j * S:(j + 1) * S] = True
        return m & ht.valid

    worst = 0.0
    worst = max(worst, _compare("dq", gq, dq, slots(q_sel)))
    worst = max(worst, _compare("dk", gk, dk, slots(k_sel)))
    worst = max(worst, _compare("dv", gv, dv, slots(k_sel)))
    return worst


@pytest.mark.parametrize("name,sparsity", [("tiny", 50), ("tiny", 0), ("ragged-small", 75),
                                           ("ragged-small", 0), ("ragged-d64", 60)])
def test_backward_small(name, sparsity):
    _say(f"backward {name} s={sparsity}")
    r = Run(name, sparsity=sparsity)
    _, do, grads = _forward_backward(r)
    worst = 0.0
    for h in range(r.heads):
        rp, ci = r.csr_head(h)
        worst = max(worst, _check_head(r, h, do, grads, rp, ci))
    _say(f"  worst max-abs / max|ref| {worst:.3e}")


def test_backward_edge_csr():
    """Hand CSR through both directions: an empty row, a repeated tile, an
    out-of-range entry."""
    _say("backward edge csr")
    torch = need_gpu()
    r = Run("tiny")
    L, ly = r.L, r.layer
    # the out-of-range entry goes last in its row, so the row stays ascending
    rows = [[], [0, 3, 3], [1, 2, 7], [3]]
    rp = np.cumsum([0] + [len(x) for x in rows]).astype(np.int32)
    ci = np.array(sum(rows, []), dtype=np.int32)
    ly.permute_pool_inputs(r.q, r.k, r.v)
    ly.row_ptr.copy_(torch.from_numpy(rp))
    ly.col_idx = torch.from_numpy(ci).cuda()
    ly.nnz = int(ci.size)
    out = torch.empty_like(r.q)
    ly.attend_tokens(r.sm_scale, out)
    rng = np.random.default_rng(8)
    do = bf16_round(rng.normal(size=(r.wl.q.shape[0], r.heads, r.d)).astype(np.float32))
    grads = ly.backward(r.q, r.k, r.v, out, to_dev_bf16(do), r.sm_scale)
    torch.cuda.synchronize()
    clean = [[j for j in row if 0 <= j < L.n(0)] for row in rows]
    crp = np.cumsum([0] + [len(x) for x in clean])
    cci = np.array(sum(clean, []), dtype=np.int64)
    worst = _check_head(r, 0, do, grads, crp, cci)
    # the empty row's queries get zero dQ
    ht = r.tilings[0]
    gq = oracle.gather(bf16_f64(grads[0])[:, 0, :], r.T, r.H, r.W, ht.shape)
    assert np.all(gq[:r.S] == 0)
    _say(f"  worst max-abs / max|ref| {worst:.3e}")


def test_backward_bench_config_sampled():
    """The Wan-1.3B-like layer at 90 %: per head, dQ on two query tiles and
    dK/dV on two key tiles (with every query tile keeping them), against the
    oracle run on the CSR rows those tiles depend on."""
    _say("backward wan1.3b 90% sampled")
    r = Run("wan1.3b-480p-81f", sparsity=90)
    _, do, grads = _forward_backward(r)
    rng = np.random.default_rng(11)
    worst = 0.0
    for h in range(r.heads):
        rp, ci = r.csr_head(h)
        n = r.L.n(h)
        q_sel = [int(rng.integers(0, n - 1)), n - 1]
        k_sel = [int(rng.integers(0, n - 1)), n - 1]
        keep = set(q_sel)
        for i in range(n):
            if any(j in k_sel for j in ci[rp[i]:rp[i + 1]]):
                keep.add(i)
        rows = [list(ci[rp[i]:rp[i + 1]]) if i in keep else [] for i in range(n)]
        srp = np.cumsum([0] + [len(x) for x in rows])
        sci = np.array(sum(rows, []), dtype=np.int64)
        worst = max(worst, _check_head(r, h, do, grads, srp, sci, q_sel, k_sel))
    _say(f"  worst max-abs / max|ref| {worst:.3e}")


def test_backward_deterministic():
    _say("backward determinism")
    r = Run("ragged-small")
    _, _, g1 = _forward_backward(r)
    a = [bf16_bits(t).copy() for t in g1]
    _, _, g2 = _forward_backward(r)
    for x, t in zip(a, g2):
        assert np.array_equal(x, bf16_bits(t))


def test_backward_bench_config_writes_every_row():
    """Every element of dQ, dK and dV is written at the Wan-1.3B-like 90 %
    layer (outputs start as NaN): the dK/dV workgroups, dispatched heaviest
    key tile first, cover every key tile once, including the tiles no query
    tile keeps (their dK = dV = 0)."""
    _say("backward wan1.3b 90% every row written")
    torch = need_gpu()
    r = Run("wan1.3b-480p-81f", sparsity=90)
    out = r.forward_fused()
    rng = np.random.default_rng(13)
    do = to_dev_bf16(bf16_round(rng.normal(size=(r.wl.q.shape[0], r.heads, r.d)).astype(np.float32)))
    grads = tuple(torch.full_like(r.q, float("nan")) for _ in range(3))
    r.layer.backward(r.q, r.k, r.v, out, do, r.sm_scale, grads=grads)
    torch.cuda.synchronize()
    for name, t in zip(("dq", "dk", "dv"), grads):
        assert bool(torch.isfinite(t).all()), name
    # key tiles no row keeps: zero dK and dV on their real slots
    for h in range(r.heads):
        rp, ci = r.csr_head(h)
        kept = np.zeros(r.L.n(h), bool)
        kept[ci[(ci >= 0) & (ci < r.L.n(h))]] = True
        if kept.all():
            continue
        ht = r.tilings[h]
        gk = oracle.gather(bf16_f64(grads[1])[:, h, :], r.T, r.H, r.W, ht.shape)
        gv = oracle.gather(bf16_f64(grads[2])[:, h, :], r.T, r.H, r.W, ht.shape)
        for j in np.flatnonzero(~kept)[:8]:
            sl = slice(j * r.S, (j + 1) * r.S)
            assert np.all(gk[sl][ht.valid[sl]] == 0) and np.all(gv[sl][ht.valid[sl]] == 0), (h, j)


def test_backward_large_heterogeneous_sampled():
    """The 720P 241-frame layer's 24-head heterogeneous draw cut to 9 frames,
    at 95 %: in three heads, dQ on a seeded query tile and the boundary tile,
    and dK/dV on the key tile kept by the most query tiles (the longest list,
    dispatched first), against the oracle on the CSR rows they depend on."""
    _say("backward long-720p T=9 95% sampled")
    r = Run("long-720p-241f", sparsity=95, T=9)
    assert len(set(r.wl.tile_shapes)) > 1
    _, do, grads = _forward_backward(r, seed=17)
    rng = np.random.default_rng(19)
    worst = 0.0
    for h in (0, 11, r.heads - 1):
        rp, ci = r.csr_head(h)
        n = r.L.n(h)
        cnt = np.bincount(ci[(ci >= 0) & (ci < n)], minlength=n)
        q_sel = [int(rng.integers(0, n - 1)), n - 1]
        k_sel = [int(np.argmax(cnt))]
        keep = set(q_sel)
        for i in range(n):
            if any(j in k_sel for j in ci[rp[i]:rp[i + 1]]):
                keep.add(i)
        rows = [list(ci[rp[i]:rp[i + 1]]) if i in keep else [] for i in range(n)]
        srp = np.cumsum([0] + [len(x) for x in rows])
        sci = np.array(sum(rows, []), dtype=np.int64)
        worst = max(worst, _check_head(r, h, do, grads, srp, sci, q_sel, k_sel))
    _say(f"  worst max-abs / max|ref| {worst:.3e}")


@pytest.mark.parametrize("name,sparsity", [("ragged-small", 75), ("wan1.3b-480p-81f", 90)])
def test_backward_tile_order_inputs_bit_identical(name, sparsity):
    """veda_sparse_attn_bwd_tiles on the forward's tile-order Q and K gives
    the same gradients, bit for bit, as veda_sparse_attn_bwd on the
    token-order tensors."""
    _say(f"backward tile-order inputs {name} {sparsity}%")
    torch = need_gpu()
    r = Run(name, sparsity=sparsity)
    out = r.forward_fused()
    rng = np.random.default_rng(23)
    do = to_dev_bf16(bf16_round(rng.normal(size=(r.wl.q.shape[0], r.heads, r.d)).astype(np.float32)))
    a = r.layer.backward(r.q, r.k, r.v, out, do, r.sm_scale, reuse_tiles=True)
    a = [bf16_bits(t).copy() for t in a]
    b = r.layer.backward(r.q, r.k, r.v, out, do, r.sm_scale, reuse_tiles=False)
    torch.cuda.synchronize()
    for x, t in zip(a, b):
        assert np.array_equal(x, bf16_bits(t))

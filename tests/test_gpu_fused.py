"""GPU parity of the fused calls (the layer's default ``forward``):

* veda_tile_permute_pool: tile-order gather plus TripPool descriptors in one
  pass, against the oracle's gather (bit-exact) and TripPool (max/min exact,
  mean within 1e-4), and bit-identical to veda_tile_permute +
  veda_tripool_score;
* veda_tile_score: projection and scores from those descriptors;
* veda_sparse_attn_fwd_tokens: O written straight to token order, against the
  oracle (same bars as the tile-order call) and bit-identical to
  veda_sparse_attn_fwd followed by the inverse permutation;
* veda_score_select: the CSR bit-identical to veda_tile_score followed by
  veda_select_tiles on the same phi, with and without exact ties.

The bit-identity checks compare the two GPU paths on the same inputs; the
oracle checks test the fused calls on their own.
"""
import numpy as np
import pytest

import oracle
from gpu_common import Run, bf16_bits, bf16_f64, host, need_gpu, to_dev_f32

pytestmark = pytest.mark.gpu

ATT_MAX, ATT_MEAN, LSE_TOL = 2e-2, 2e-3, 1e-4
SMALL = ["tiny", "ragged-small", "ragged-d64"]


def _say(msg):
    print(msg, flush=True)


def _unfused_then_fused(r):
    """Both layer paths on the same inputs; returns the unfused results and
    the fused ones (O in token order, desc, scores, CSR, lse)."""
    torch = need_gpu()
    ly = r.layer
    out_u = r.forward()
    ref = {"o": bf16_bits(out_u).copy(), "desc": host(ly.desc).copy(),
           "scores": host(ly.scores).copy(), "rp": host(ly.row_ptr).copy(),
           "ci": host(ly.col_idx).copy(), "lse": host(ly.lse).copy()}
    for t in (ly.desc, ly.scores, ly.lse):
        t.fill_(float("nan"))
    ly.row_ptr.fill_(-7)
    ly.col_idx.fill_(-7)
    out_f = torch.full_like(r.q, float("nan"))
    r.forward_fused(out_f)
    got = {"o": bf16_bits(out_f), "desc": host(ly.desc), "scores": host(ly.scores),
           "rp": host(ly.row_ptr), "ci": host(ly.col_idx), "lse": host(ly.lse), "out": out_f}
    return ref, got


@pytest.mark.parametrize("name,sparsity", [("tiny", 50), ("ragged-small", 75), ("ragged-d64", 60),
                                           ("ragged-small", 0), ("wan1.3b-480p-81f", 90),
                                           ("wan1.3b-480p-81f", 95)])
def test_fused_layer_bit_identical_to_unfused(name, sparsity):
    _say(f"fused vs unfused {name} s={sparsity}")
    r = Run(name, sparsity=sparsity)
    ref, got = _unfused_then_fused(r)
    n_rp = r.L.total_tiles + 1
    assert np.array_equal(got["desc"], ref["desc"]), "TripPool descriptors"
    assert np.array_equal(got["scores"], ref["scores"]), "tile scores"
    assert np.array_equal(got["rp"][:n_rp], ref["rp"][:n_rp]), "row_ptr"
    assert np.array_equal(got["ci"][:r.layer.nnz], ref["ci"][:r.layer.nnz]), "col_idx"
    # every token row written (no NaN left), and equal bit for bit
    assert np.array_equal(got["o"], ref["o"]), "O (token order)"
    for h in range(r.heads):
        rows = r.rows(h)
        v = r.tilings[h].valid
        assert np.array_equal(got["lse"][rows][v], ref["lse"][rows][v]), h


def _check_permute_pool(r, dtype):
    torch = need_gpu()
    V, L, d, S = r.V, r.L, r.d, r.S
    tot = L.total_tiles
    if dtype == "f32":
        xs = (to_dev_f32(r.wl.q32), to_dev_f32(r.wl.k32))
        ys = [torch.full((V.tiles_numel(L),), float("nan"), dtype=torch.float32, device="cuda")
              for _ in range(2)]
    else:
        xs = (r.q, r.k)
        ys = [torch.full((V.tiles_numel(L),), float("nan"), dtype=torch.bfloat16, device="cuda")
              for _ in range(2)]
    desc = torch.full((2 * tot * 3 * d,), float("nan"), dtype=torch.float32, device="cuda")
    n = tot * 3 * d
    for side in range(2):
        V.veda_tile_permute_pool(L, xs[side], ys[side], desc[side * n:(side + 1) * n])
    torch.cuda.synchronize()
    dg = host(desc).reshape(2, tot, 3 * d)
    for h in range(r.heads):
        ht = r.tilings[h]
        a, b = int(L.tile_off[h]), int(L.tile_off[h + 1])
        for side in range(2):
            if dtype == "f32":
                xt = (r.wl.q32 if side == 0 else r.wl.k32)[:, h, :].astype(np.float64)
                yg = host(ys[side]).reshape(-1, d)[r.rows(h)].astype(np.float64)
            else:
                xt = r.head_tokens(h)[side]
                yg = bf16_f64(ys[side]).reshape(-1, d)[r.rows(h)]
            gref = oracle.gather(xt, r.T, r.H, r.W, ht.shape)
            assert np.array_equal(yg, gref), (h, side, "gather")
            ref = oracle.tripool(gref, ht.valid, S)
            got = dg[side, a:b]
            assert np.array_equal(got[:, d:], ref[:, d:].astype(np.float32)), (h, side)
            assert np.abs(got[:, :d] - ref[:, :d]).max() <= 1e-4, (h, side)


@pytest.mark.parametrize("name", SMALL + ["wan1.3b-480p-81f"])
def test_permute_pool_vs_oracle(name):
    _say(f"permute_pool {name}")
    _check_permute_pool(Run(name), "bf16")


def test_permute_pool_f32_vs_oracle():
    _say("permute_pool f32")
    _check_permute_pool(Run("tiny"), "f32")


def test_tile_score_from_desc_vs_oracle():
    """veda_tile_score on the GPU's descriptors, with biases and two
    different projections, against the oracle's projection and score."""
    _say("tile_score")
    torch = need_gpu()
    r = Run("ragged-small")
    V, L, d = r.V, r.L, r.d
    rng = np.random.default_rng(11)
    wq = rng.normal(0, 0.02, size=r.wl.w.shape).astype(np.float32)
    wk = rng.normal(0, 0.02, size=r.wl.w.shape).astype(np.float32)
    bq = rng.normal(0, 0.1, size=(r.heads, wq.shape[1])).astype(np.float32)
    bk = rng.normal(0, 0.1, size=(r.heads, wq.shape[1])).astype(np.float32)
    r.layer.permute_pool_inputs(r.q, r.k, r.v)
    V.veda_tile_score(L, r.layer.desc, to_dev_f32(wq), to_dev_f32(wk), r.layer.phi,
                      r.layer.scores, to_dev_f32(bq), to_dev_f32(bk))
    torch.cuda.synchronize()
    tot = L.total_tiles
    desc = host(r.layer.desc).reshape(2, tot, 3 * d).astype(np.float64)
    phi = host(r.layer.phi).reshape(2, tot, -1)
    for h in range(r.heads):
        a, b = int(L.tile_off[h]), int(L.tile_off[h + 1])
        pq = oracle.project(desc[0, a:b], wq[h].astype(np.float64), bq[h].astype(np.float64))
        pk = oracle.project(desc[1, a:b], wk[h].astype(np.float64), bk[h].astype(np.float64))
        tol = 1e-4 * max(1.0, np.abs(pq).max(), np.abs(pk).max())
        assert np.abs(phi[0, a:b] - pq).max() <= tol, h
        assert np.abs(phi[1, a:b] - pk).max() <= tol, h
        sref = oracle.tile_scores(phi[0, a:b].astype(np.float64), phi[1, a:b].astype(np.float64))
        assert np.abs(r.scores_head(h) - sref).max() <= 1e-4 * max(1.0, np.abs(sref).max()), h


def test_attention_claimed_tiles_bit_identical():
    """Heads of 512 tiles take the lockstep XCD order; with a workspace the
    last tenth of each XCD's share of query tiles is handed out through its
    counters.  O (token order, starting as NaN so that every element must be
    written) and lse must be bit-identical to the call without a workspace,
    on two calls in a row (the counters are reset by each call)."""
    _say("attention with claimed tiles")
    torch = need_gpu()
    import tile_sparse_attention_head_amd as V
    L = V.veda_layout_init(32, 32, 64, 128, 128, [(4, 4, 8), (2, 8, 8)])
    assert min(L.n(h) for h in range(L.num_heads)) >= 512
    g = torch.Generator(device="cuda").manual_seed(7)
    n_tok, H, d = 32 * 32 * 64, L.num_heads, L.head_dim
    q, k, v = (torch.randn(n_tok, H, d, generator=g, device="cuda").to(torch.bfloat16)
               for _ in range(3))
    nt = V.tiles_numel(L)
    qp, kp, vtp = (torch.empty(nt, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    V.veda_tile_permute(L, q, qp, V.VEDA_FWD)
    V.veda_tile_permute(L, k, kp, V.VEDA_FWD)
    V.veda_tile_permute(L, v, vtp, V.VEDA_FWD_T)
    rng = np.random.default_rng(3)
    kk = 26
    cols = [np.sort(rng.choice(L.n(h), size=kk, replace=False)) for h in range(H)
            for _ in range(L.n(h))]
    ci = torch.from_numpy(np.concatenate(cols).astype(np.int32)).cuda()
    rp = torch.from_numpy(np.arange(0, L.total_tiles * kk + 1, kk, dtype=np.int32)).cuda()
    ws = torch.empty(V.veda_sparse_attn_fwd_workspace(L), dtype=torch.uint8, device="cuda")
    sm = 1.0 / np.sqrt(d)

    def run(workspace):
        o = torch.full((n_tok, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((L.total_tiles * L.tile_size,), float("nan"), device="cuda")
        V.veda_sparse_attn_fwd_tokens(L, qp, kp, vtp, rp, ci, sm, o, lse, workspace=workspace)
        torch.cuda.synchronize()
        return o.view(torch.int16), lse
    o0, l0 = run(None)
    assert not torch.isnan(o0.view(torch.bfloat16)).any()
    for _ in range(2):
        o1, l1 = run(ws)
        assert torch.equal(o1, o0)
        assert torch.equal(l1.view(torch.int32), l0.view(torch.int32))


def test_tile_score_odd_width_and_unaligned_operands():
    """veda_tile_score with d_e = 50 (the score product's K is not a multiple
    of 4, nor of the 32-wide K step) on descriptors, weights, biases and phi
    shifted by 4 bytes from 16-byte alignment: the kernels' element-wise,
    zero-padded loads, against the oracle."""
    _say("tile_score d_e = 50, unaligned")
    torch = need_gpu()
    r = Run("ragged-small")
    V, L, d = r.V, r.L, r.d
    de = 50
    rng = np.random.default_rng(13)
    wq = rng.normal(0, 0.02, size=(r.heads, de, 3 * d)).astype(np.float32)
    wk = rng.normal(0, 0.02, size=(r.heads, de, 3 * d)).astype(np.float32)
    bq = rng.normal(0, 0.1, size=(r.heads, de)).astype(np.float32)
    bk = rng.normal(0, 0.1, size=(r.heads, de)).astype(np.float32)
    r.layer.permute_pool_inputs(r.q, r.k, r.v)
    tot = L.total_tiles

    def shifted(a):
        t = a if isinstance(a, torch.Tensor) else to_dev_f32(np.ascontiguousarray(a).ravel())
        buf = torch.empty(t.numel() + 1, dtype=torch.float32, device="cuda")
        buf[1:].copy_(t.reshape(-1))
        return buf[1:].view(a.shape)
    phi_u = shifted(torch.zeros(2 * tot * de, dtype=torch.float32, device="cuda"))
    scores = torch.empty(L.total_scores, dtype=torch.float32, device="cuda")
    V.veda_tile_score(L, shifted(r.layer.desc), shifted(wq), shifted(wk), phi_u, scores,
                      shifted(bq), shifted(bk))
    torch.cuda.synchronize()
    desc = host(r.layer.desc).reshape(2, tot, 3 * d).astype(np.float64)
    phi = host(phi_u).reshape(2, tot, de)
    sc = host(scores)
    for h in range(r.heads):
        a, b = int(L.tile_off[h]), int(L.tile_off[h + 1])
        pq = oracle.project(desc[0, a:b], wq[h].astype(np.float64), bq[h].astype(np.float64))
        pk = oracle.project(desc[1, a:b], wk[h].astype(np.float64), bk[h].astype(np.float64))
        tol = 1e-4 * max(1.0, np.abs(pq).max(), np.abs(pk).max())
        assert np.abs(phi[0, a:b] - pq).max() <= tol, h
        assert np.abs(phi[1, a:b] - pk).max() <= tol, h
        n = b - a
        off = int(L.score_off[h])
        sref = oracle.tile_scores(phi[0, a:b].astype(np.float64), phi[1, a:b].astype(np.float64))
        sg = sc[off:off + n * n].reshape(n, n)
        assert np.abs(sg - sref).max() <= 1e-4 * max(1.0, np.abs(sref).max()), h


def _check_tokens(r, out, q_tiles_per_head=None):
    """Token-order O of the fused layer against the oracle's sparse attention
    on the GPU's own CSR, scattered to token order."""
    o = bf16_f64(out)
    lse = host(r.layer.lse)
    worst = 0.0
    for h in range(r.heads):
        ht = r.tilings[h]
        qp, kp, vp = r.head_perm(h)
        rp, ci = r.csr_head(h)
        tiles = None if q_tiles_per_head is None else q_tiles_per_head[h]
        ro, rl = oracle.sparse_attention(qp, kp, vp, ht.valid, r.S, rp, ci, r.sm_scale,
                                         q_tiles=tiles)
        sel = ~np.isnan(rl)                      # real rows of the computed tiles
        # token-order O of head h, gathered back into tile order
        og = oracle.gather(o[:, h, :], r.T, r.H, r.W, ht.shape)
        err = np.abs(og[sel] - ro[sel])
        worst = max(worst, err.max())
        assert err.max() <= ATT_MAX and err.mean() <= ATT_MEAN, (h, err.max(), err.mean())
        assert np.abs(lse[r.rows(h)][sel] - rl[sel]).max() <= LSE_TOL, h
    return worst


@pytest.mark.parametrize("name,sparsity", [("tiny", 50), ("tiny", 0), ("ragged-small", 75),
                                           ("ragged-d64", 60), ("ragged-d64", 0)])
def test_attention_tokens_vs_oracle(name, sparsity):
    _say(f"attention tokens {name} s={sparsity}")
    torch = need_gpu()
    r = Run(name, sparsity=sparsity)
    out = torch.full_like(r.q, float("nan"))
    r.forward_fused(out)
    assert not np.isnan(bf16_f64(out)).any(), "a token row was not written"
    _say(f"  max-abs {_check_tokens(r, out):.3e}")


def test_attention_tokens_bench_config_sampled():
    """The Wan-1.3B-like layer (12 heads, 21x30x52, 90 %) as the benchmark
    runs it: every head, a seeded sample of query tiles with its last
    (boundary) tile."""
    _say("attention tokens wan1.3b 90% sampled")
    torch = need_gpu()
    r = Run("wan1.3b-480p-81f", sparsity=90)
    out = torch.full_like(r.q, float("nan"))
    r.forward_fused(out)
    assert not np.isnan(bf16_f64(out)).any()
    rng = np.random.default_rng(7)
    sample = [np.sort(np.append(rng.choice(r.L.n(h) - 1, size=4, replace=False), r.L.n(h) - 1))
              for h in range(r.heads)]
    _say(f"  max-abs {_check_tokens(r, out, sample):.3e}")


def test_attention_tokens_heterogeneous_sampled():
    """Heterogeneous per-head tiles (Wan-14B-like 720P layer, 40 heads, 95 %):
    fused output against the oracle on sampled tiles, and bit-identical to the
    unfused path."""
    _say("attention tokens wan14b 95% sampled")
    r = Run("wan14b-720p-81f", sparsity=95)
    assert len(set(r.wl.tile_shapes)) > 1
    ref, got = _unfused_then_fused(r)
    assert np.array_equal(got["o"], ref["o"])
    out = got["out"]
    rng = np.random.default_rng(9)
    sample = [np.array([rng.integers(0, r.L.n(h) - 1), r.L.n(h) - 1]) for h in range(r.heads)]
    _say(f"  max-abs {_check_tokens(r, out, sample):.3e}")


def test_attention_tokens_edge_csr():
    """Hand-made CSR through the token-order call: an empty row gives O = 0
    and lse = -inf on its tokens; out-of-range entries are skipped."""
    _say("attention tokens edge csr")
    torch = need_gpu()
    r = Run("tiny")
    V, L = r.V, r.L
    r.layer.permute_inputs(r.q, r.k, r.v)
    rows = [[], [3, -1, 7, 0], [2, 2], [1]]
    rp = np.cumsum([0] + [len(x) for x in rows]).astype(np.int32)
    ci = np.array(sum(rows, []), dtype=np.int32)
    out = torch.full_like(r.q, float("nan"))
    V.veda_sparse_attn_fwd_tokens(L, r.layer.q_perm, r.layer.k_perm, r.layer.vt_perm,
                                  torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda(),
                                  r.sm_scale, out, r.layer.lse)
    torch.cuda.synchronize()
    ht = r.tilings[0]
    og = oracle.gather(bf16_f64(out)[:, 0, :], r.T, r.H, r.W, ht.shape)
    lse = host(r.layer.lse)
    S = r.S
    assert np.all(og[:S][ht.valid[:S]] == 0) and np.all(np.isneginf(lse[:S]))
    qp, kp, vp = r.head_perm(0)
    clean = [[3, 0], [2, 2], [1]]
    crp = np.cumsum([0, 0] + [len(x) for x in clean])
    cci = np.array(sum(clean, []))
    ro, rl = oracle.sparse_attention(qp, kp, vp, ht.valid, S, crp, cci, r.sm_scale,
                                     q_tiles=[1, 2, 3])
    sel = ~np.isnan(rl)
    assert np.abs(og[sel] - ro[sel]).max() <= ATT_MAX
    assert np.abs(lse[sel] - rl[sel]).max() <= LSE_TOL


@pytest.mark.timeout(420)
@pytest.mark.parametrize("name,sparsity,tie", [("tiny", 50, False), ("ragged-small", 75, False),
                                               ("ragged-d64", 60, False),
                                               ("wan1.3b-480p-81f", 90, False),
                                               ("wan1.3b-480p-81f", 95, True),
                                               ("waver12b-720p-121f", 95, False),
                                               ("long-720p-241f", 95, False),
                                               ("long-720p-241f", 95, True)])
def test_score_select_bit_identical_to_two_calls(name, sparsity, tie):
    """veda_score_select (scores never stored) against veda_tile_score +
    veda_select_tiles on the same phi: row_ptr and col_idx bit-identical, at
    4-1920 key tiles per row (all three register widths of the selection).
    With tie, phi_K rows are copied within runs of four tiles, so every row
    holds many exactly equal scores and the lowest index must win."""
    _say(f"score_select {name} s={sparsity} tie={tie}")
    torch = need_gpu()
    r = Run(name, sparsity=sparsity, cache=name.startswith("long"))
    V, L, ly = r.V, r.L, r.layer
    ly.permute_pool_inputs(r.q, r.k, r.v)
    V.veda_tile_score(L, ly.desc, r.w, r.w, ly.phi, None)
    if tie:
        de = ly.d_e
        tot = L.total_tiles
        pk = ly.phi[tot * de:].view(tot, de)
        for h in range(r.heads):
            a, b = int(L.tile_off[h]), int(L.tile_off[h + 1])
            src = torch.arange(a, b, device="cuda") // 4 * 4
            pk[a:b] = pk[src]
    # reference: the standalone score kernel, from the same phi, then select
    ref_scores = torch.full((L.total_scores,), float("nan"), dtype=torch.float32, device="cuda")
    _score_only(r, ly.phi, ref_scores)
    rp_ref = torch.full((L.total_tiles + 1,), -7, dtype=torch.int32, device="cuda")
    ci_ref = torch.full((max(1, ly.nnz),), -7, dtype=torch.int32, device="cuda")
    V.veda_select_tiles(L, ref_scores, ly.k_per_head, rp_ref, ci_ref)
    ly.row_ptr.fill_(-9)
    ly.col_idx.fill_(-9)
    V.veda_score_select(L, ly.phi, ly.d_e, ly.k_per_head, ly.row_ptr, ly.col_idx)
    torch.cuda.synchronize()
    assert np.array_equal(host(ly.row_ptr), host(rp_ref))
    assert np.array_equal(host(ly.col_idx)[:ly.nnz], host(ci_ref)[:ly.nnz])
    if tie:
        s = host(ref_scores)
        a, n = int(L.score_off[0]), L.n(0)
        row = s[a:a + n]
        assert len(np.unique(row)) <= (n + 3) // 4   # the copies tie exactly
    _say(f"  {L.total_tiles} rows, nnz {ly.nnz}, max {L.max_tiles} tiles per row: bit-identical")
    del r
    torch.cuda.empty_cache()


def _score_only(r, phi, scores):
    """The score product of veda_tile_score from a given phi: its projection
    is run with an identity weight on descriptors that hold phi itself."""
    torch = need_gpu()
    V, L, ly = r.V, r.L, r.layer
    d, de, tot = L.head_dim, ly.d_e, L.total_tiles
    # desc rows [phi | 0 | 0] and W = [I | 0 | 0] reproduce phi exactly (each
    # output is one product by 1 plus exact zeros)
    desc = torch.zeros(2, tot, 3 * d, dtype=torch.float32, device="cuda")
    desc[:, :, :de] = phi.view(2, tot, de)
    w = torch.zeros(L.num_heads, de, 3 * d, dtype=torch.float32, device="cuda")
    w[:, torch.arange(de), torch.arange(de)] = 1.0
    phi2 = torch.empty_like(phi)
    V.veda_tile_score(L, desc.view(-1), w, w, phi2, scores)
    torch.cuda.synchronize()
    assert torch.equal(phi2, phi)

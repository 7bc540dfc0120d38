"""GPU parity of the attention forward on CSR rows longer than 64 entries.

The forward keeps a window of 64 CSR entries in one register and reloads it
in the middle of a row once a row has more.  Rows that long occur at the
Waver-12B-like layer at 90 % (93-96 kept tiles), the 720P 241-frame layer at
95 % (92-96) and at 0 % sparsity (every tile: 336 on the Wan-1.3B-like
layer).  These tests compare exactly those cases with the oracle
(Veda §2.3 tile-skipping attention; dense attention at 0 %, Veda §1):

* hand CSRs with rows of 63-200 entries (repeated tiles, entries outside the
  head after entry 64, window reloads mid-row) on the small heterogeneous
  layers, every query slot;
* the Waver-12B-like and 720P 241-frame layers in the benchmark's launch
  configuration (fused calls, O written in token order), sampled query tiles
  of every head including its last (boundary) tile;
* the Wan-1.3B-like layer at 0 % against dense attention in token order;
* top-k selection bit-exact at 1830-1920 and 8192 key tiles per row;
* the max-pooled map of the 720P 241-frame layer's whole 10 % subset,
  sampled per tile shape against the oracle.

Bars as in the other parity tests: bf16 O max-abs <= 2e-2, mean-abs <= 2e-3,
lse <= 1e-4; selection bit-exact.
"""
import numpy as np
import pytest

import oracle
from gpu_common import Run, bf16_bits, bf16_f64, check_attention, host, need_gpu, to_dev_f32

pytestmark = pytest.mark.gpu

ATT_MAX, ATT_MEAN, LSE_TOL = 2e-2, 2e-3, 1e-4
LENGTHS = (64, 65, 66, 67, 63, 127, 128, 129, 130, 200, 1, 131)


def _say(msg):
    print(msg, flush=True)


def _hand_rows(r, seed):
    """Per query tile a row of LENGTHS[...] entries drawn with repetition from
    the head's tiles; every other row longer than 70 gets three entries
    outside [0, n) (-1, n, n + 1000) at positions >= 64, which the kernel
    skips.  Returns (global row_ptr, col_idx, per-head clean local CSRs)."""
    rng = np.random.default_rng(seed)
    rows, clean = [], []
    for h in range(r.heads):
        n = r.L.n(h)
        crow = []
        for i in range(n):
            ln = LENGTHS[(i + 3 * h) % len(LENGTHS)]
            row = rng.integers(0, n, size=ln).astype(np.int64)
            if ln > 70 and i % 2 == 0:
                pos = rng.choice(np.arange(64, ln), size=3, replace=False)
                row[pos] = [-1, n, n + 1000]
            rows.append(row)
            crow.append(row[(row >= 0) & (row < n)])
        lrp = np.cumsum([0] + [len(x) for x in crow]).astype(np.int64)
        clean.append((lrp, np.concatenate(crow)))
    rp = np.cumsum([0] + [len(x) for x in rows]).astype(np.int32)
    return rp, np.concatenate(rows).astype(np.int32), clean


@pytest.mark.parametrize("name", ["ragged-small", "ragged-d64"])
def test_attention_long_hand_csr(name):
    _say(f"long hand CSR {name}")
    torch = need_gpu()
    r = Run(name)
    V, L = r.V, r.L
    r.layer.permute_inputs(r.q, r.k, r.v)
    rp, ci, clean = _hand_rows(r, seed=17)
    assert (np.diff(rp) > 64).sum() > 0
    rp_d, ci_d = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
    V.veda_sparse_attn_fwd(L, r.layer.q_perm, r.layer.k_perm, r.layer.vt_perm, rp_d, ci_d,
                           r.sm_scale, r.layer.o_perm, r.layer.lse)
    out_tok = torch.empty_like(r.q)
    V.veda_sparse_attn_fwd_tokens(L, r.layer.q_perm, r.layer.k_perm, r.layer.vt_perm, rp_d, ci_d,
                                  r.sm_scale, out_tok, None)
    inv = torch.empty_like(r.q)
    V.veda_tile_permute(L, r.layer.o_perm, inv, V.VEDA_INV)
    torch.cuda.synchronize()
    o = bf16_f64(r.layer.o_perm).reshape(-1, r.d)
    lse = host(r.layer.lse)
    worst = 0.0
    for h in range(r.heads):
        ht = r.tilings[h]
        qp, kp, vp = r.head_perm(h)
        lrp, lci = clean[h]
        ro, rl = oracle.sparse_attention(qp, kp, vp, ht.valid, r.S, lrp, lci, r.sm_scale)
        sel = ~np.isnan(rl)
        err = np.abs(o[r.rows(h)][sel] - ro[sel])
        worst = max(worst, err.max())
        assert err.max() <= ATT_MAX and err.mean() <= ATT_MEAN, (h, err.max(), err.mean())
        assert np.abs(lse[r.rows(h)][sel] - rl[sel]).max() <= LSE_TOL, h
    # the token-order epilogue writes the same bits as tile order + inverse permutation
    assert np.array_equal(bf16_bits(out_tok), bf16_bits(inv))
    _say(f"  max-abs {worst:.3e}, longest row {int(np.diff(rp).max())}")


def _sample(r, seed, per_head=2):
    rng = np.random.default_rng(seed)
    return [np.sort(np.append(rng.choice(r.L.n(h) - 1, size=per_head, replace=False),
                              r.L.n(h) - 1)) for h in range(r.heads)]


def _check_estimator_sampled(r, sample):
    """The projection (128-row tiles at these sizes) and the score product of
    the full-size layer on the sampled query tiles of every head: phi against
    the oracle's projection of the GPU's descriptors, and those tiles' score
    rows against the oracle's score of the GPU's phi.  Then the same call on
    copies of the descriptors, weights and phi shifted by 4 bytes (so the
    kernels take their generic, element-wise loads) must give the same bits."""
    torch = need_gpu()
    V, L, d, ly = r.V, r.L, r.d, r.layer
    tot, de = L.total_tiles, ly.d_e
    desc = host(ly.desc).reshape(2, tot, 3 * d).astype(np.float64)
    phi = host(ly.phi).reshape(2, tot, de)
    worst = 0.0
    for h in range(r.heads):
        a, b = int(L.tile_off[h]), int(L.tile_off[h + 1])
        w = r.wl.w[h].astype(np.float64)
        rows = a + sample[h]
        for side in (0, 1):
            ref = oracle.project(desc[side, rows], w)
            err = np.abs(phi[side, rows] - ref).max()
            assert err <= 1e-4 * max(1.0, np.abs(ref).max()), (h, side, err)
        sref = oracle.tile_scores(phi[0, rows].astype(np.float64), phi[1, a:b].astype(np.float64))
        sg = r.scores_head(h)[sample[h]]
        err = np.abs(sg - sref).max()
        worst = max(worst, err / max(1.0, np.abs(sref).max()))
        assert err <= 1e-4 * max(1.0, np.abs(sref).max()), (h, err)
    # unaligned operands: the element-wise path of both products, same bits
    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        buf[1:].copy_(t.reshape(-1))
        return buf[1:].view(t.shape)
    desc_u, w_u = shifted(ly.desc), shifted(r.w)
    phi_u = shifted(torch.zeros_like(ly.phi))
    sc_u = torch.empty_like(ly.scores)
    V.veda_tile_score(L, desc_u, w_u, w_u, phi_u, sc_u)
    torch.cuda.synchronize()
    assert torch.equal(phi_u, ly.phi)
    assert torch.equal(sc_u, ly.scores)
    _say(f"  projection and scores on sampled tiles: worst {worst:.2e} of max|S|; "
         f"unaligned operands bit-identical")


@pytest.mark.timeout(420)
@pytest.mark.parametrize("name,sparsity,T", [("waver12b-720p-121f", 90, None),
                                             ("waver12b-720p-121f", 95, None),
                                             ("long-720p-241f", 95, None)])
def test_attention_full_size_layer_sampled(name, sparsity, T):
    """Every head of the full-size heterogeneous layer through the fused
    calls (the benchmark's launch configuration); O compared in token order
    on two seeded query tiles per head plus the head's last tile.  At the
    720P 241-frame layer the selection is also checked bit-exact on the GPU's
    own scores for every row of one head of each tile shape (1830-1920 key
    tiles per row).  The projection and score product are checked on the
    sampled tiles too, with aligned and unaligned operands."""
    _say(f"full-size {name} {sparsity}%")
    torch = need_gpu()
    r = Run(name, sparsity=sparsity, T=T, cache=True)
    assert len(set(r.wl.tile_shapes)) > 1
    out = r.forward_fused()
    sample = _sample(r, seed=23)
    worst, mean, longest = check_attention(r, sample, o_tok=out)
    _say(f"  max-abs {worst:.3e} mean-abs {mean:.3e}, longest kept row {longest}")
    if sparsity == 90 or name.startswith("long"):
        assert longest > 64
    _check_estimator_sampled(r, sample)
    if name.startswith("long"):
        first = {}
        for h in range(r.heads):
            first.setdefault(r.wl.tile_shapes[h], h)
        for h in first.values():
            k = r.layer.k_per_head[h]
            rp, ci = r.csr_head(h)
            ref_rp, ref_ci = oracle.select_topk(r.scores_head(h), k)
            assert np.array_equal(rp, ref_rp) and np.array_equal(ci, ref_ci), h
            _say(f"  select head {h}: n = {r.L.n(h)}, k = {k} bit-exact")
    del r, out
    torch.cuda.empty_cache()


@pytest.mark.timeout(420)
def test_maxpool_map_720p_sampled():
    """The max-pooled map at the 720P 241-frame layer in the benchmark's
    launch shape: the whole seeded 10 % subset (4527 subset tiles, one chunk
    per tile) over the tile-order Q and K that the fused layer left.  The last
    subset tile of the first head of each tile shape against
    oracle.maxpool_map over all of the head's 1830-1920 key tiles (map entries
    within 1e-3 relative, lse within 1e-4; zeros past the head)."""
    _say("map 720p 241f 10% sampled")
    torch = need_gpu()
    import workloads
    r = Run("long-720p-241f", sparsity=95, cache=True)
    r.forward_fused()
    L = r.L
    subset = workloads.draw_subset(r.wl, [L.n(h) for h in range(r.heads)])
    flat = np.concatenate([int(L.tile_off[h]) + s for h, s in enumerate(subset)]).astype(np.int32)
    assert flat.size > 4000
    lse, mp = r.layer.maxpool_map(torch.from_numpy(flat).cuda(), r.sm_scale)
    torch.cuda.synchronize()
    lse = host(lse).reshape(-1, r.S)
    mp = host(mp).reshape(-1, L.max_tiles)
    starts = np.concatenate([[0], np.cumsum([len(s) for s in subset])])
    first = {}
    for h in range(r.heads):
        first.setdefault(r.wl.tile_shapes[h], h)
    assert len(first) > 1
    for h in first.values():
        ht = r.tilings[h]
        i = len(subset[h]) - 1
        qp, kp, _ = r.head_perm(h)
        rl, rm = oracle.maxpool_map(qp, kp, ht.valid, r.S, subset[h][i:i + 1], r.sm_scale)
        row = starts[h] + i
        got = mp[row]
        assert np.all(got[ht.n:] == 0), h
        rel = np.abs(got[:ht.n] - rm[0]) / np.maximum(rm[0], 1e-30)
        assert np.all(np.abs(got[:ht.n] - rm[0]) <= np.maximum(1e-3 * rm[0], 1e-7)), (h, rel.max())
        sel = ~np.isnan(rl)
        dl = np.abs(lse[row][sel] - rl[sel]).max()
        assert dl <= LSE_TOL, (h, dl)
        _say(f"  head {h} {r.wl.tile_shapes[h]}: subset tile {int(subset[h][i])} of {ht.n}, "
             f"map rel err {rel.max():.2e}, lse err {dl:.2e}")
    del r
    torch.cuda.empty_cache()


@pytest.mark.timeout(300)
def test_dense_full_size_sampled_against_token_order_dense_attention():
    """Wan-1.3B-like layer at 0 % sparsity (every row keeps all 336 tiles,
    five window reloads per row): the fused layer's token-order O on sampled
    query tiles of every head against oracle.dense_attention computed from the
    token-order inputs with no tiling at all."""
    _say("dense wan1.3b 0% sampled")
    torch = need_gpu()
    r = Run("wan1.3b-480p-81f", sparsity=0)
    assert all(k == r.L.n(h) for h, k in enumerate(r.layer.k_per_head))
    out = bf16_f64(r.forward_fused())
    sample = _sample(r, seed=29)
    worst = 0.0
    for h in range(r.heads):
        ht = r.tilings[h]
        q, k, v = r.head_tokens(h)
        for i in sample[h]:
            toks = ht.perm[i * r.S:(i + 1) * r.S]
            toks = toks[toks >= 0]
            od, _ = oracle.dense_attention(q[toks], k, v, r.sm_scale)
            err = np.abs(out[toks, h, :] - od)
            worst = max(worst, err.max())
            assert err.max() <= ATT_MAX and err.mean() <= ATT_MEAN, (h, i, err.max())
    _say(f"  max-abs {worst:.3e}")


@pytest.mark.parametrize("n_shape,pct,ties", [(((61, 45, 80), (4, 4, 8)), 95, False),
                                              (((61, 45, 80), (1, 8, 16)), 90, True),
                                              (((61, 45, 80), (4, 4, 8)), 90, "flat"),
                                              (((31, 45, 80), (1, 8, 16)), 95, "flat"),
                                              (((64, 64, 256), (1, 8, 16)), 95, False),
                                              (((64, 64, 256), (1, 8, 16)), 90, True)])
def test_select_bit_exact_large_rows(n_shape, pct, ties):
    """Random f32 score matrices of one head with 930 / 1830 / 1920 / 8192
    key tiles per row (8192 is the largest the selection call accepts), k at
    5 % and 10 %; with ties the values come from a six-value set with +-0, and
    NaN is planted on a lattice; "flat" rows are mostly one value with a few
    Gaussian entries, so that most keys tie at the k-th place (the wave
    kernel's open range never shrinks to 64 keys and its final pass takes the
    lowest-index ties).  Every row against oracle.select_topk."""
    grid, shape = n_shape
    _say(f"select large rows {grid} {shape} {pct}% ties={ties}")
    torch = need_gpu()
    import tile_sparse_attention_head_amd as V
    from workloads import random_scores
    L = V.veda_layout_init(*grid, 128, 128, [shape])
    n = L.n(0)
    k = V.veda_keep_count(n, pct)
    if ties == "flat":
        s = np.full((n, n), 0.5, dtype=np.float32)
        rng = np.random.default_rng(400 + n)
        mask = rng.random((n, n)) < 0.02
        s[mask] = rng.standard_normal(int(mask.sum())).astype(np.float32)
    else:
        s = random_scores(n, n, seed=300 + n + pct, ties=bool(ties))
    if ties is True:
        s[::7, ::11] = np.nan
    rp = torch.empty(n + 1, dtype=torch.int32, device="cuda")
    ci = torch.empty(n * k, dtype=torch.int32, device="cuda")
    V.veda_select_tiles(L, to_dev_f32(s.ravel()), [k], rp, ci)
    torch.cuda.synchronize()
    ref_rp, ref_ci = oracle.select_topk(s, k)
    assert np.array_equal(host(rp), ref_rp)
    assert np.array_equal(host(ci), ref_ci)
    _say(f"  n = {n}, k = {k} bit-exact")


def _row_kind(kind, n, rng):
    """One score row of a given kind (the shapes a threshold search can trip
    on: narrow ranges, infinities, NaN halves, all-equal rows, integer ties,
    heavy tails, a diagonal trend)."""
    if kind == 0:
        r = rng.normal(size=n)
    elif kind == 1:
        r = rng.integers(-3, 3, size=n).astype(np.float64)
    elif kind == 2:
        r = np.full(n, 1.5)
    elif kind == 3:
        r = rng.normal(size=n)
        r[rng.random(n) < 0.2] = np.nan
        r[rng.random(n) < 0.1] = -0.0
        r[rng.random(n) < 0.1] = 0.0
    elif kind == 4:
        r = 5.0 + 1e-3 * rng.normal(size=n)
    elif kind == 5:
        r = np.where(rng.random(n) < 0.5, np.inf, -np.inf)
    elif kind == 6:
        r = rng.normal(size=n)
        r[: n // 2] = np.nan
    elif kind == 7:
        r = rng.exponential(size=n)
    else:
        r = -np.abs(np.arange(n) - rng.integers(0, n)) * 0.002 + rng.normal(size=n)
    return r.astype(np.float32)


@pytest.mark.parametrize("grid,shape", [((21, 30, 52), (4, 4, 8)),      # 336 key tiles
                                        ((31, 45, 80), (4, 4, 8)),      # 960
                                        ((61, 45, 80), (4, 4, 8))])     # 1920
def test_select_row_kinds(grid, shape):
    """The wave-per-row selection (8, 16 and 32 keys per lane) on rows of nine
    kinds, one kind per row in turn, at k = 1, 2, 64, 65, 129, 256, 257, n and
    the 95 % / 90 % keep counts: the k that start the search from the largest,
    the second, the third-or-fourth largest key per lane or from zero, and the
    rows whose open range never narrows to 64 keys (ties).  Every row against
    oracle.select_topk (largest first, ties to the lowest index)."""
    _say(f"select row kinds {grid} {shape}")
    torch = need_gpu()
    import tile_sparse_attention_head_amd as V
    L = V.veda_layout_init(*grid, 128, 128, [shape])
    n = L.n(0)
    rng = np.random.default_rng(500 + n)
    s = np.stack([_row_kind(i % 9, n, rng) for i in range(n)])
    dev = to_dev_f32(s.ravel())
    ks = sorted({1, 2, 64, 65, 129, 256, 257, n, V.veda_keep_count(n, 95),
                 V.veda_keep_count(n, 90)} & set(range(1, n + 1)))
    for k in ks:
        rp = torch.empty(n + 1, dtype=torch.int32, device="cuda")
        ci = torch.empty(n * k, dtype=torch.int32, device="cuda")
        V.veda_select_tiles(L, dev, [k], rp, ci)
        torch.cuda.synchronize()
        ref_rp, ref_ci = oracle.select_topk(s, k)
        assert np.array_equal(host(rp), ref_rp), k
        assert np.array_equal(host(ci), ref_ci), k
    _say(f"  n = {n}, k in {ks} bit-exact")

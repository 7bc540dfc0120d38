"""GPU parity of the head-aware tiling search.

* veda_head_sq_error against the same sums taken on the host in f64 from the
  same bf16 tensors (bar 1e-12 relative: both sides sum exact squares of
  exact bf16 differences in f64, in different orders);
* the search on a case with a known answer (attention confined to (1,8,8)
  boxes): the GPU picks (1,8,8) for every head, and every candidate's error
  agrees with the oracle's search (oracle.search_head) within the bf16
  output rounding of the two attention runs;
* the search on the Wan-1.3B-like benchmark layer: every error is the host
  f64 sum over the GPU's outputs, and the chosen shapes are their argmins;
* veda_head_choose, the search's decision, against the first argmin on
  tied errors and against its documented scan with NaN errors.
"""
import numpy as np
import pytest

import oracle
from gpu_common import Run, bf16_f64, host, need_gpu, to_dev_bf16, to_dev_f32
from workloads import bf16_round, bf16_to_f64

pytestmark = pytest.mark.gpu

CANDS64 = [(1, 8, 8), (2, 4, 8), (2, 8, 4), (1, 4, 16)]


def _say(msg):
    print(msg, flush=True)


def test_head_sq_error_matches_host_sums():
    _say("head_sq_error")
    torch = need_gpu()
    import tile_sparse_attention_head_amd as V
    L = V.veda_layout_init(5, 9, 20, 128, 128, [(8, 4, 4), (1, 8, 16), (2, 8, 8)])
    rng = np.random.default_rng(3)
    N = L.tokens
    a = bf16_round(rng.normal(size=(N, 3, 128)).astype(np.float32))
    b = bf16_round((bf16_to_f64(a) + rng.normal(0, 0.01, size=(N, 3, 128))).astype(np.float32))
    ws = torch.empty(V.veda_head_sq_error_workspace(L), dtype=torch.uint8, device="cuda")
    err = torch.empty(3, dtype=torch.float64, device="cuda")
    ref = torch.empty(3, dtype=torch.float64, device="cuda")
    V.veda_head_sq_error(L, to_dev_bf16(a), to_dev_bf16(b), err, ws, ref=ref)
    torch.cuda.synchronize()
    fa, fb = bf16_to_f64(a), bf16_to_f64(b)
    e_ref = ((fa - fb) ** 2).sum(axis=(0, 2))
    r_ref = (fa ** 2).sum(axis=(0, 2))
    np.testing.assert_allclose(host(err), e_ref, rtol=1e-12)
    np.testing.assert_allclose(host(ref), r_ref, rtol=1e-12)


def _box_inputs(heads=2, alpha=8.0):
    """T, H, W = 2, 16, 16; queries and keys alpha * one-hot code of their
    (1,8,8) box, values random: full attention never leaves the box."""
    T, H, W, d = 2, 16, 16, 64
    box = np.array([(t * 2 + h // 8) * 2 + w // 8 for t in range(T) for h in range(H)
                    for w in range(W)])
    N = T * H * W
    qk = np.zeros((N, heads, d), np.float32)
    qk[np.arange(N), :, box] = alpha
    v = np.random.default_rng(4).normal(size=(N, heads, d)).astype(np.float32)
    w = np.zeros((heads, d, 3 * d), np.float32)
    w[:, :, :d] = np.eye(d, dtype=np.float32)             # phi = tile mean
    return T, H, W, d, bf16_round(qk), bf16_round(v), w


def test_search_box_case_picks_the_box_shape():
    _say("tiling search, box case")
    torch = need_gpu()
    import tile_sparse_attention_head_amd as V
    T, H, W, d, qk, v, w = _box_inputs()
    heads = qk.shape[1]
    q = to_dev_bf16(qk)
    chosen, errs, ref = V.search_tile_shapes(T, H, W, d, 64, q, q, to_dev_bf16(v), to_dev_f32(w),
                                             to_dev_f32(w), 1.0, 90, candidates=CANDS64)
    torch.cuda.synchronize()
    assert chosen == [CANDS64[0]] * heads
    e, r = host(errs), host(ref)
    for h in range(heads):
        assert e[0, h] <= 1e-6 * r[h]
        assert np.all(e[1:, h] > 1e-2 * r[h])
        f = bf16_to_f64(qk[:, h, :])
        oe, oref, best = oracle.search_head(f, f, bf16_to_f64(v[:, h, :]), T, H, W, CANDS64,
                                            w[h].astype(np.float64), w[h].astype(np.float64),
                                            None, None, 1.0, 90)
        assert best == 0
        assert abs(r[h] - oref) <= 1e-2 * oref
        # both outputs are rounded to bf16 (relative 2^-9 per element)
        for c in range(len(CANDS64)):
            assert abs(e[c, h] - oe[c]) <= 2e-2 * oe[c] + 1e-5 * oref, (c, h, e[c, h], oe[c])


def test_search_bench_layer_errors_are_host_sums():
    _say("tiling search, wan1.3b layer")
    torch = need_gpu()
    import tile_sparse_attention_head_amd as V
    r = Run("wan1.3b-480p-81f", sparsity=90)
    chosen, errs, ref = V.search_tile_shapes(r.T, r.H, r.W, r.d, r.S, r.q, r.k, r.v, r.w, r.w,
                                             r.sm_scale, 90)
    torch.cuda.synchronize()
    e = host(errs)
    assert e.shape == (4, r.heads) and np.all(e > 0)
    for h in range(r.heads):
        assert chosen[h] == V.tiling_search.SHAPES_128[int(np.argmin(e[:, h]))]
    # one candidate recomputed on the host from the GPU's outputs; the full
    # reference with the search's own tiling (the first candidate): dense
    # attention is exact whatever the tiling, but its bf16 rounding depends
    # on the order the key tiles are summed in
    full = V.TileSparseAttention(r.T, r.H, r.W, r.d, r.S, [V.tiling_search.SHAPES_128[0]] * r.heads,
                                 sparsity_pct=0)
    of = bf16_f64(full.forward(r.q, r.k, r.v, r.w, r.w, r.sm_scale))
    sp = V.TileSparseAttention(r.T, r.H, r.W, r.d, r.S, [(4, 4, 8)] * r.heads, sparsity_pct=90)
    os_ = bf16_f64(sp.forward(r.q, r.k, r.v, r.w, r.w, r.sm_scale))
    torch.cuda.synchronize()
    np.testing.assert_allclose(e[2], ((of - os_) ** 2).sum(axis=(0, 2)), rtol=1e-10)
    np.testing.assert_allclose(host(ref), (of ** 2).sum(axis=(0, 2)), rtol=1e-10)


@pytest.mark.parametrize("n_cand,heads", [(4, 24), (1, 3), (64, 64), (7, 40)])
def test_head_choose_matches_first_argmin(n_cand, heads):
    """veda_head_choose against the oracle search's rule (np.argmin: the first
    smallest error) on finite errors drawn from a few values, so that many
    heads tie; then with NaN planted, against the documented scan (a NaN never
    replaces an earlier candidate; a NaN candidate 0 stays)."""
    _say(f"head_choose {n_cand}x{heads}")
    torch = need_gpu()
    import tile_sparse_attention_head_amd as V
    rng = np.random.default_rng(100 * n_cand + heads)
    e = rng.choice(np.array([0.5, 0.25, 1.0, 0.25, 3.0, 1e-300, 0.0]), size=(n_cand, heads))
    choice = torch.empty(heads, dtype=torch.int32, device="cuda")
    V.veda_head_choose(torch.from_numpy(e).cuda(), choice)
    torch.cuda.synchronize()
    assert np.array_equal(host(choice), np.argmin(e, axis=0))
    e[rng.random(e.shape) < 0.2] = np.nan
    V.veda_head_choose(torch.from_numpy(e).cuda(), choice)
    torch.cuda.synchronize()
    want = []
    for h in range(heads):
        best = 0
        for c in range(1, n_cand):
            if e[c, h] < e[best, h]:
                best = c
        want.append(best)
    assert np.array_equal(host(choice), np.array(want))

"""VEDA_DEBUG_SYNC=1: every call synchronises, and the attention calls check
the CSR on the host before launching anything.  The mode is read once per
process, so the checks run in a child process; its results on a valid CSR
must be bit-identical to this process's, and every corrupted CSR must come
back as VEDA_ERR_BAD_CSR.  The corruptions keep row_ptr consistent with the
col_idx buffer (the forward call sizes its host copy from row_ptr)."""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
BAD_CSR = -4


def _step(name="ragged-small", sparsity=75):
    """The fused forward and the backward of one seeded workload; returns
    the layer, its inputs and the outputs as host arrays of bf16 bits."""
    from gpu_common import bf16_bits, need_gpu, to_dev_bf16, to_dev_f32
    import tile_sparse_attention_head_amd as V
    import workloads
    torch = need_gpu()
    wl = workloads.make(name, 0)
    cfg = wl.config
    ly = V.TileSparseAttention(wl.T, cfg.H, cfg.W, cfg.head_dim, cfg.tile_size, wl.tile_shapes,
                               sparsity_pct=sparsity)
    q, k, v = (to_dev_bf16(a) for a in (wl.q, wl.k, wl.v))
    w = to_dev_f32(wl.w)
    do = to_dev_bf16(workloads.bf16_round(
        np.random.default_rng(7).normal(size=wl.q.shape).astype(np.float32)))
    out = ly.forward(q, k, v, w, w, cfg.sm_scale)
    grads = ly.backward(q, k, v, out, do, cfg.sm_scale)
    torch.cuda.synchronize()
    res = {"out": bf16_bits(out)}
    res.update({n: bf16_bits(g) for n, g in zip(("dq", "dk", "dv"), grads)})
    return ly, (q, k, v, out, do, cfg.sm_scale), res


def _child(outdir: str) -> None:
    """Run in a process started with VEDA_DEBUG_SYNC=1."""
    import torch
    import tile_sparse_attention_head_amd as V
    from tile_sparse_attention_head_amd._lib import VedaError
    ly, (q, k, v, out, do, sc), res = _step()
    np.savez(os.path.join(outdir, "debug.npz"), **res)
    L = ly.L
    rp = ly.row_ptr.cpu().numpy()
    ci = ly.col_idx.cpu().numpy()
    h0_n = L.n(0)

    def expect_bad(fn, what):
        try:
            fn()
        except VedaError as e:
            assert e.status == BAD_CSR, f"{what}: status {e.status}"
            return
        raise AssertionError(f"{what}: accepted")

    def fwd(col):
        o = torch.empty_like(out)
        V.veda_sparse_attn_fwd_tokens(L, ly.q_perm, ly.k_perm, ly.vt_perm, ly.row_ptr, col, sc, o)
        torch.cuda.synchronize()

    def bwd(col, nnz):
        ws = torch.empty(max(16, V.veda_sparse_attn_bwd_workspace(L, nnz)), dtype=torch.uint8,
                         device="cuda")
        g = [torch.empty_like(q) for _ in range(3)]
        V.veda_sparse_attn_bwd(L, q, k, v, out, do, ly.lse, ly.row_ptr, col, nnz, sc, ws, *g)
        torch.cuda.synchronize()

    nnz = int(rp[-1])
    # an entry past its head's tile count
    bad = ci.copy()
    bad[rp[0]] = h0_n
    bad_t = torch.from_numpy(bad).cuda()
    expect_bad(lambda: fwd(bad_t), "forward, entry out of range")
    expect_bad(lambda: bwd(bad_t, nnz), "backward, entry out of range")
    # a negative entry
    neg = ci.copy()
    neg[rp[1]] = -1
    expect_bad(lambda: fwd(torch.from_numpy(neg).cuda()), "forward, negative entry")
    # a row whose entries are not ascending: the forward takes any order, the
    # backward needs ascending rows
    assert rp[1] - rp[0] >= 2
    swp = ci.copy()
    swp[rp[0]], swp[rp[0] + 1] = swp[rp[0] + 1], swp[rp[0]]
    swp_t = torch.from_numpy(swp).cuda()
    fwd(swp_t)
    expect_bad(lambda: bwd(swp_t, nnz), "backward, descending row")
    # an entry count that disagrees with row_ptr
    expect_bad(lambda: bwd(ly.col_idx, nnz - 1), "backward, nnz")
    print("debug-csr child ok", flush=True)


def test_debug_sync_checks_csr(tmp_path):
    env = dict(os.environ, VEDA_DEBUG_SYNC="1")
    code = (f"import sys; sys.path[:0] = [{ROOT!r}, {HERE!r}]; "
            f"import test_gpu_debug_csr as t; t._child({str(tmp_path)!r})")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "debug-csr child ok" in r.stdout
    _, _, res = _step()
    dbg = np.load(tmp_path / "debug.npz")
    for name, bits in res.items():
        assert np.array_equal(dbg[name], bits), f"{name} differs under VEDA_DEBUG_SYNC=1"

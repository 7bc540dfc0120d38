"""Shared helpers of the GPU parity tests: upload a seeded workload, run the
library's stages through the Python binding, bring results back, and build
the oracle's per-head inputs from the same host arrays."""
from __future__ import annotations

import numpy as np

import oracle
import workloads
from workloads import bf16_to_f64


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible MI355X (torch.cuda.is_available() is False)")
    return torch


def to_dev_bf16(bits: np.ndarray):
    torch = need_gpu()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_dev_f32(a: np.ndarray):
    torch = need_gpu()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def bf16_bits(t) -> np.ndarray:
    torch = need_gpu()
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_f64(t) -> np.ndarray:
    return bf16_to_f64(bf16_bits(t))


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


_WL_CACHE = {}


def cached_workload(name: str, seed: int = 0, T: int = None):
    """workloads.make with the last full-size draw kept, so that tests of one
    large layer at several sparsities draw its inputs once (one entry is kept,
    which bounds host memory)."""
    key = (name, seed, T)
    if key not in _WL_CACHE:
        _WL_CACHE.clear()
        _WL_CACHE[key] = workloads.make(name, seed, T=T)
    return _WL_CACHE[key]


def check_attention(r, q_tiles_per_head, o_tok=None, att_max=2e-2, att_mean=2e-3, lse_tol=1e-4,
                    say=None):
    """GPU attention against oracle.sparse_attention on the GPU's own CSR, for
    the query tiles ``q_tiles_per_head[h]`` of every head (None: all).  With
    ``o_tok`` (the token-order output of the fused call) each query slot is
    compared at its token's row; otherwise the tile-order o_perm is read.
    lse (tile-slot order) is read from the layer.  Returns (worst max-abs,
    mean of the per-head mean-abs, largest kept-row length seen)."""
    L = r.L
    o = None if o_tok is not None else bf16_f64(r.layer.o_perm).reshape(-1, r.d)
    ot = None if o_tok is None else bf16_f64(o_tok)
    lse = host(r.layer.lse)
    worst, means, longest = 0.0, [], 0
    for h in range(r.heads):
        ht = r.tilings[h]
        qp, kp, vp = r.head_perm(h)
        rp, ci = r.csr_head(h)
        tiles = None if q_tiles_per_head is None else q_tiles_per_head[h]
        for i in (range(ht.n) if tiles is None else tiles):
            longest = max(longest, int(rp[i + 1] - rp[i]))
        ro, rl = oracle.sparse_attention(qp, kp, vp, ht.valid, r.S, rp, ci, r.sm_scale,
                                         q_tiles=tiles)
        sel = ~np.isnan(rl)
        if ot is None:
            go = o[r.rows(h)][sel]
        else:
            go = ot[ht.perm[sel], h, :]            # slot -> its token's row of head h
        err = np.abs(go - ro[sel])
        worst = max(worst, float(err.max()))
        means.append(float(err.mean()))
        assert err.max() <= att_max, (h, err.max())
        assert err.mean() <= att_mean, (h, err.mean())
        assert np.abs(lse[r.rows(h)][sel] - rl[sel]).max() <= lse_tol, h
        if say is not None:
            say(f"  head {h} {ht.shape}: max-abs {err.max():.2e}")
    return worst, float(np.mean(means)), longest


class Run:
    """A workload on the GPU plus its oracle-side view."""

    def __init__(self, name: str, seed: int = 0, sparsity: int = None, T: int = None,
                 k_per_head=None, cache: bool = False):
        torch = need_gpu()
        import tile_sparse_attention_head_amd as V
        self.V = V
        self.wl = cached_workload(name, seed, T) if cache else workloads.make(name, seed, T=T)
        cfg = self.wl.config
        self.cfg = cfg
        self.T, self.H, self.W = self.wl.T, cfg.H, cfg.W
        self.sparsity = cfg.sparsities[0] if sparsity is None else sparsity
        self.layer = V.TileSparseAttention(self.T, self.H, self.W, cfg.head_dim, cfg.tile_size,
                                           self.wl.tile_shapes, sparsity_pct=self.sparsity,
                                           k_per_head=k_per_head)
        self.L = self.layer.L
        self.q = to_dev_bf16(self.wl.q)
        self.k = to_dev_bf16(self.wl.k)
        self.v = to_dev_bf16(self.wl.v)
        self.w = to_dev_f32(self.wl.w)
        self.sm_scale = cfg.sm_scale
        self.S = cfg.tile_size
        self.d = cfg.head_dim
        self.heads = cfg.heads
        self.tilings = [oracle.HeadTiling(self.T, self.H, self.W, s) for s in self.wl.tile_shapes]

    def forward(self):
        """The layer one method step per call: tile-order O stays in
        layer.o_perm, and the inverse permutation gives the returned O."""
        out = self.layer.forward_unfused(self.q, self.k, self.v, self.w, self.w, self.sm_scale)
        need_gpu().cuda.synchronize()
        return out

    def forward_fused(self, out=None):
        """The fused layer (gather + TripPool, score, select, attention writing
        token-order O); layer.o_perm is not written."""
        out = self.layer.forward(self.q, self.k, self.v, self.w, self.w, self.sm_scale, out=out)
        need_gpu().cuda.synchronize()
        return out

    # oracle-side per-head inputs (fp64, tile order)
    def head_tokens(self, h):
        return (bf16_to_f64(self.wl.q[:, h, :]), bf16_to_f64(self.wl.k[:, h, :]),
                bf16_to_f64(self.wl.v[:, h, :]))

    def head_perm(self, h):
        ht = self.tilings[h]
        q, k, v = self.head_tokens(h)
        g = lambda a: oracle.gather(a, self.T, self.H, self.W, ht.shape)
        return g(q), g(k), g(v)

    def rows(self, h):
        """Slice of tile-order rows of head h."""
        a = int(self.L.tile_off[h]) * self.S
        return slice(a, a + self.L.n(h) * self.S)

    def csr_head(self, h):
        rp = host(self.layer.row_ptr).astype(np.int64)
        ci = host(self.layer.col_idx).astype(np.int64)
        a, b = int(self.L.tile_off[h]), int(self.L.tile_off[h + 1])
        loc = rp[a:b + 1] - rp[a]
        return loc, ci[rp[a]:rp[b]]

    def scores_head(self, h):
        s = host(self.layer.scores)
        a, n = int(self.L.score_off[h]), self.L.n(h)
        return s[a:a + n * n].reshape(n, n)

"""The library's calls are stream-ordered, allocate nothing and never
synchronise, so they can run on several streams at once and be captured in a
HIP graph.  These tests check both against eager runs on one stream:
results must be bit-identical (every kernel is deterministic)."""
from __future__ import annotations

import numpy as np
import pytest

import tile_sparse_attention_head_amd as V
import workloads
from gpu_common import need_gpu, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu


def _same(a, b) -> bool:
    torch = need_gpu()
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


class _Case:
    def __init__(self, name: str, seed: int, sparsity: int, map_pct: int = 25):
        torch = need_gpu()
        wl = workloads.make(name, seed)
        cfg = wl.config
        self.sm_scale = cfg.sm_scale
        self.layer = V.TileSparseAttention(wl.T, cfg.H, cfg.W, cfg.head_dim, cfg.tile_size,
                                           wl.tile_shapes, sparsity_pct=sparsity)
        self.q, self.k, self.v = (to_dev_bf16(a) for a in (wl.q, wl.k, wl.v))
        self.w = to_dev_f32(wl.w)
        self.do = to_dev_bf16(workloads.bf16_round(
            np.random.default_rng(seed + 11).normal(size=wl.q.shape).astype(np.float32)))
        rng = np.random.default_rng(seed + 3)
        L = self.layer.L
        sub = []
        for h in range(L.num_heads):
            n = L.n(h)
            m = max(1, -(-n * map_pct // 100))
            sub += [int(L.tile_off[h]) + int(j) for j in np.sort(rng.choice(n, m, replace=False))]
        self.qt = torch.tensor(sub, dtype=torch.int32, device="cuda")
        self.out = torch.empty_like(self.q)
        self.grads = tuple(torch.empty_like(self.q) for _ in range(3))

    def step(self, q=None):
        """forward (fused), map and backward; returns the output tensors"""
        ly = self.layer
        q = self.q if q is None else q
        ly.forward(q, self.k, self.v, self.w, self.w, self.sm_scale, out=self.out)
        lse, mp = ly.maxpool_map(self.qt, self.sm_scale)
        ly.backward(q, self.k, self.v, self.out, self.do, self.sm_scale, grads=self.grads)
        return (self.out, lse, mp) + self.grads

    def snapshot(self, outs):
        return [t.clone() for t in outs]


@pytest.mark.parametrize("name,sparsity", [("ragged-small", 75), ("ragged-d64", 60)])
def test_step_replays_in_hip_graph(name, sparsity):
    """Forward, map and backward captured in one graph: every replay, with
    eager work on other inputs between replays, equals the eager step."""
    torch = need_gpu()
    c = _Case(name, 0, sparsity)
    ref = c.snapshot(c.step())
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        c.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = c.step()
    torch.cuda.synchronize()

    q_other = (c.q.float() * 0.5).to(torch.bfloat16)
    for rep in range(3):
        other = c.snapshot(c.step(q_other))   # eager work that rewrites every buffer
        torch.cuda.synchronize()
        assert not _same(other[0], ref[0])
        for t in captured:
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(captured, ref)):
            assert _same(a, b), f"replay {rep}: output {i} differs from the eager step"


def test_two_streams_at_once():
    """Two layers with different inputs stepping on two streams at once give
    what each gives alone."""
    torch = need_gpu()
    a = _Case("ragged-small", 0, 75)
    b = _Case("ragged-small", 1, 50)
    ref_a = a.snapshot(a.step())
    ref_b = b.snapshot(b.step())
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        with torch.cuda.stream(s1):
            out_a = a.step()
        with torch.cuda.stream(s2):
            out_b = b.step()
    torch.cuda.synchronize()
    for i, (x, r) in enumerate(zip(out_a, ref_a)):
        assert _same(x, r), f"stream 1 output {i}"
    for i, (x, r) in enumerate(zip(out_b, ref_b)):
        assert _same(x, r), f"stream 2 output {i}"

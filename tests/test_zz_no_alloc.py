"""veda_distill_grad_noalloc (the library's static per-GPU scratch instead of
a caller workspace) against veda_distill_grad on the same inputs: two calls
in a row, the second on a smaller problem, each bit-identical in loss and
every gradient to the entry point that takes a workspace."""
import numpy as np
import pytest

import workloads
from gpu_common import Run, host, need_gpu

pytestmark = pytest.mark.gpu


def _case(name):
    torch = need_gpu()
    r = Run(name)
    r.forward_fused()
    L = r.L
    sub = workloads.draw_subset(r.wl, [L.n(h) for h in range(r.heads)])
    flat = np.concatenate([int(L.tile_off[h]) + s for h, s in enumerate(sub)]).astype(np.int32)
    q_tiles = torch.from_numpy(flat).cuda()
    _, mp = r.layer.maxpool_map(q_tiles, r.sm_scale)
    loss_a, grads_a = r.layer.distill_grad(q_tiles, mp)
    torch.cuda.synchronize()
    want = [host(loss_a).copy()] + [host(g).copy() for g in grads_a]
    de = r.layer.d_e
    H, d3 = L.num_heads, 3 * L.head_dim
    out = [torch.full((1,), float("nan"), device="cuda"),
           torch.full((H, de, d3), float("nan"), device="cuda"),
           torch.full((H, de, d3), float("nan"), device="cuda"),
           torch.full((H, de), float("nan"), device="cuda"),
           torch.full((H, de), float("nan"), device="cuda")]
    r.V.veda_distill_grad_noalloc(L, r.layer.scores, mp, q_tiles, r.layer.desc, r.layer.phi, de,
                                  *out)
    torch.cuda.synchronize()
    for w, g in zip(want, out):
        assert np.array_equal(w.view(np.uint32), host(g).view(np.uint32))
    return int(flat.size), float(want[0][0])


def test_noalloc_distill_matches_workspace_entry_point_twice():
    n1, l1 = _case("wan1.3b-480p-81f")
    print(f"first call: {n1} subset rows, loss {l1:.6f}", flush=True)
    n2, l2 = _case("ragged-small")
    print(f"second call: {n2} subset rows, loss {l2:.6f}", flush=True)
    assert n2 < n1

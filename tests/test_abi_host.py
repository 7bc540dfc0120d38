"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

The library must load, export every function include/veda.h declares, derive
the same tile geometry and keep counts as the oracle, and reject bad
arguments before anything is enqueued.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import tile_sparse_attention_head_amd as V
from tile_sparse_attention_head_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "veda.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(V.LIB_PATH):
        pytest.fail("libveda.so is not built (python -m tile_sparse_attention_head_amd.build)")
    return V.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(veda_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 9
    for name in names:
        assert hasattr(lib, name), name


def test_layout_struct_size_matches(lib):
    assert lib.veda_layout_sizeof() == ctypes.sizeof(_lib.veda_layout)


@pytest.mark.parametrize("T,H,W,shapes", [
    (21, 30, 52, [(4, 4, 8)] * 12),
    (61, 45, 80, [(1, 8, 16), (2, 8, 8), (4, 4, 8), (8, 4, 4)]),
    (5, 9, 20, [(8, 4, 4), (1, 8, 16), (2, 8, 8)]),
    (4, 8, 8, [(4, 4, 4)]),
])
def test_layout_matches_oracle(lib, T, H, W, shapes):
    S = int(np.prod(shapes[0]))
    L = V.veda_layout_init(T, H, W, 128, S, shapes)
    off = 0
    soff = 0
    for h, s in enumerate(shapes):
        g = oracle.tile_grid(T, H, W, s)
        n = g[0] * g[1] * g[2]
        assert tuple(L.tile_grid[h]) == g and L.n(h) == n
        assert L.tile_off[h] == off and L.score_off[h] == soff
        off += n
        soff += n * n
    assert L.total_tiles == off and L.total_scores == soff
    assert L.max_tiles == max(L.n(h) for h in range(len(shapes)))


@pytest.mark.parametrize("n", [1, 4, 7, 336, 630, 720, 1830, 1920, 8191])
@pytest.mark.parametrize("s", [0, 1, 50, 90, 95, 99, 100])
def test_keep_count_matches_oracle(lib, n, s):
    assert V.veda_keep_count(n, s) == oracle.keep_count(n, s)


def _status(fn, *args):
    return fn(*args)


def test_layout_rejections(lib):
    bad = [
        dict(T=0), dict(H=-1), dict(head_dim=0), dict(tile_size=0),
    ]
    for b in bad:
        L = _lib.veda_layout()
        L.T, L.H, L.W, L.num_heads, L.head_dim, L.tile_size = 4, 8, 8, 1, 64, 64
        L.tile_shape[0][0], L.tile_shape[0][1], L.tile_shape[0][2] = 4, 4, 4
        for k, v in b.items():
            setattr(L, k, v)
        assert lib.veda_layout_init(ctypes.byref(L)) == -1
    L = _lib.veda_layout()
    L.T, L.H, L.W, L.num_heads, L.head_dim, L.tile_size = 4, 8, 8, 1, 64, 64
    L.tile_shape[0][0], L.tile_shape[0][1], L.tile_shape[0][2] = 4, 4, 8     # 128 != 64
    assert lib.veda_layout_init(ctypes.byref(L)) == -1
    L.num_heads = 65
    assert lib.veda_layout_init(ctypes.byref(L)) == -1
    assert lib.veda_layout_init(None) == -1
    with pytest.raises(V.VedaError):
        V.veda_layout_init(4, 8, 8, 64, 64, [(4, 4, 0)])


def test_keep_count_rejections(lib):
    k = ctypes.c_int32(0)
    assert lib.veda_keep_count(0, 50, ctypes.byref(k)) == -1
    assert lib.veda_keep_count(4, 101, ctypes.byref(k)) == -1
    assert lib.veda_keep_count(4, -1, ctypes.byref(k)) == -1
    assert lib.veda_keep_count(4, 50, None) == -1


def _layout():
    return V.veda_layout_init(5, 9, 20, 128, 128, [(8, 4, 4), (1, 8, 16)])


def test_device_calls_reject_before_launch(lib):
    L = _layout()
    Lp = ctypes.byref(L)
    fake = 1 << 20          # aligned, never dereferenced: calls must fail validation first
    # tampered layout
    L2 = _layout()
    L2.tile_off[1] += 1
    assert lib.veda_tile_permute(ctypes.byref(L2), 0, 0, fake, fake * 4, None) == -1
    # permute: nulls, bad enums, misalignment, overlap
    assert lib.veda_tile_permute(Lp, 0, 0, None, fake, None) == -1
    assert lib.veda_tile_permute(Lp, 7, 0, fake, fake * 4, None) == -1
    assert lib.veda_tile_permute(Lp, 0, 9, fake, fake * 4, None) == -1
    assert lib.veda_tile_permute(Lp, 0, 0, fake + 2, fake * 4, None) == -2
    assert lib.veda_tile_permute(Lp, 0, 0, fake, fake + 4096, None) == -1      # overlap
    # tiles above 256 slots, and an f32 FWD_T whose LDS image would not fit
    L4 = V.veda_layout_init(8, 8, 8, 64, 512, [(8, 8, 8)])
    assert lib.veda_tile_permute(ctypes.byref(L4), 0, 0, fake, fake * 64, None) == -2
    L5 = V.veda_layout_init(8, 8, 8, 128, 128, [(2, 8, 8)])
    assert lib.veda_tile_permute(ctypes.byref(L5), 1, 2, fake, fake * 64, None) == -2
    # tripool: null weights, bad d_e
    assert lib.veda_tripool_score(Lp, 0, fake, fake, None, fake, None, None, 128, fake, fake, fake, None) == -1
    assert lib.veda_tripool_score(Lp, 0, fake, fake, fake, fake, None, None, 0, fake, fake, fake, None) == -1
    assert lib.veda_tripool_score(Lp, 0, fake, fake, fake, fake, None, None, 999, fake, fake, fake, None) == -2
    # select: k out of range
    kh = (ctypes.c_int32 * 2)(0, 3)
    assert lib.veda_select_tiles(Lp, fake, kh, fake, fake, None) == -1
    kh = (ctypes.c_int32 * 2)(3, L.n(1) + 1)
    assert lib.veda_select_tiles(Lp, fake, kh, fake, fake, None) == -1
    # attention: nulls, NaN / zero / negative scale (the kernels scale the row
    # maximum of the raw logits, which is the maximum of the scaled logits only
    # for a positive scale), unsupported shape
    assert lib.veda_sparse_attn_fwd(Lp, fake, fake, None, fake, fake, 0.1, fake, None, None, 0, None) == -1
    for bad in (float("nan"), 0.0, -0.1, float("inf")):
        assert lib.veda_sparse_attn_fwd(Lp, fake, fake, fake, fake, fake, bad, fake, None, None, 0,
                                        None) == -1
    L3 = V.veda_layout_init(5, 9, 20, 96, 128, [(8, 4, 4)])
    assert lib.veda_sparse_attn_fwd(ctypes.byref(L3), fake, fake, fake, fake, fake, 0.1, fake, None, None,
                                    0, None) == -2
    # the optional workspace: its size query, too small, misaligned
    ws = ctypes.c_int64(-1)
    assert lib.veda_sparse_attn_fwd_workspace(Lp, ctypes.byref(ws)) == 0 and ws.value == 256
    assert lib.veda_sparse_attn_fwd_workspace(Lp, None) == -1
    assert lib.veda_sparse_attn_fwd_workspace(None, ctypes.byref(ws)) == -1
    assert lib.veda_sparse_attn_fwd(Lp, fake, fake * 16, fake * 32, fake, fake, 0.1, fake * 64,
                                    None, fake * 128, 255, None) == -1
    assert lib.veda_sparse_attn_fwd(Lp, fake, fake * 16, fake * 32, fake, fake, 0.1, fake * 64,
                                    None, fake * 128 + 4, 256, None) == -1
    assert lib.veda_sparse_attn_fwd_tokens(Lp, fake, fake * 16, fake * 32, fake, fake, 0.1,
                                           fake * 64, None, fake * 128, 8, None) == -1
    # token-order attention: same checks, plus an output overlapping an input
    A = lib.veda_sparse_attn_fwd_tokens
    assert A(Lp, fake, fake, None, fake, fake, 0.1, fake * 64, None, None, 0, None) == -1
    for bad in (float("nan"), 0.0, -0.1, float("inf")):
        assert A(Lp, fake, fake * 16, fake * 32, fake, fake, bad, fake * 64, None, None, 0,
                 None) == -1
    assert A(ctypes.byref(L3), fake, fake * 16, fake * 32, fake, fake, 0.1, fake * 64, None,
             None, 0, None) == -2
    assert A(Lp, fake, fake * 16, fake * 32, fake, fake, 0.1, fake * 64 + 8, None, None, 0,
             None) == -2
    assert A(Lp, fake, fake * 16, fake * 32, fake, fake, 0.1, fake + 4096, None, None, 0,
             None) == -1
    # fused gather + TripPool: nulls, bad dtype, head_dim outside {64, 128},
    # misalignment, overlaps
    P = lib.veda_tile_permute_pool
    assert P(Lp, 0, None, fake * 16, fake * 32, None) == -1
    assert P(Lp, 0, fake, fake * 16, None, None) == -1
    assert P(Lp, 5, fake, fake * 16, fake * 32, None) == -1
    assert P(ctypes.byref(L3), 0, fake, fake * 16, fake * 32, None) == -2
    assert P(Lp, 0, fake + 8, fake * 16, fake * 32, None) == -2
    assert P(Lp, 0, fake, fake + 4096, fake * 32, None) == -1
    assert P(Lp, 0, fake, fake * 16, fake * 16 + 64, None) == -1
    assert P(ctypes.byref(L4), 0, fake, fake * 64, fake * 128, None) == -2
    # projection + score from descriptors: null weights, bad d_e
    TS = lib.veda_tile_score
    assert TS(Lp, fake, None, fake, None, None, 128, fake, fake, None) == -1
    assert TS(Lp, None, fake, fake, None, None, 128, fake, fake, None) == -1
    assert TS(Lp, fake, fake, fake, None, None, 0, fake, fake, None) == -1
    assert TS(Lp, fake, fake, fake, None, None, 999, fake, fake, None) == -2
    assert TS(ctypes.byref(L3), fake, fake, fake, None, None, 96, fake, fake, None) == -2
    # map: negative count, nulls, bad scale, missing / short / misaligned workspace
    ws = ctypes.c_int64(0)
    assert lib.veda_oracle_maxpool_map_workspace(Lp, 3, ctypes.byref(ws)) == 0
    big = 1 << 40
    M = lib.veda_oracle_maxpool_map
    assert M(Lp, fake, fake, 0.1, fake, -1, fake, big, fake, fake, None) == -1
    assert M(Lp, None, fake, 0.1, fake, 3, fake, big, fake, fake, None) == -1
    for bad in (float("inf"), float("nan"), 0.0, -1.0):
        assert M(Lp, fake, fake, bad, fake, 3, fake, big, fake, fake, None) == -1
    assert M(Lp, fake, fake, 0.1, fake, 3, None, big, fake, fake, None) == -1
    assert M(Lp, fake, fake, 0.1, fake, 3, fake, ws.value - 1, fake, fake, None) == -1
    assert M(Lp, fake, fake, 0.1, fake, 3, fake + 8, big, fake, fake, None) == -2
    # more subset entries than VEDA_MAX_SUBSET (the launch grids' range)
    assert M(Lp, fake, fake, 0.1, fake, (1 << 20) + 1, fake, big, fake, fake, None) == -2
    assert lib.veda_oracle_maxpool_map_workspace(Lp, (1 << 20) + 1, ctypes.byref(ws)) == -2
    assert lib.veda_oracle_maxpool_map_workspace(Lp, 1 << 20, ctypes.byref(ws)) == 0


def test_distill_rejections_and_workspace(lib):
    L = _layout()
    Lp = ctypes.byref(L)
    fake = 1 << 20
    ws = ctypes.c_int64(0)
    assert lib.veda_distill_grad_workspace(Lp, 5, 128, ctypes.byref(ws)) == 0
    need = ws.value
    assert need >= 4 * 5 * L.max_tiles + 4 * L.total_tiles * 128
    assert lib.veda_distill_grad_workspace(Lp, -1, 128, ctypes.byref(ws)) == -1
    assert lib.veda_distill_grad_workspace(Lp, 5, 0, ctypes.byref(ws)) == -1
    assert lib.veda_distill_grad_workspace(Lp, 5, 128, None) == -1
    D = lib.veda_distill_grad
    ok = dict(sc=fake, mp=fake, qt=fake, n=5, desc=fake, phi=fake, de=128, ws=fake, wsb=need,
              loss=fake, gq=fake, gk=fake)
    def call(**kw):
        a = dict(ok, **kw)
        return D(Lp, a["sc"], a["mp"], a["qt"], a["n"], a["desc"], a["phi"], a["de"], a["ws"],
                 a["wsb"], a["loss"], a["gq"], a["gk"], None, None, None)
    assert call(n=-1) == -1
    assert call(de=0) == -1
    assert call(de=300) == -2
    assert call(desc=None) == -1
    assert call(loss=None) == -1
    assert call(gk=None) == -1
    assert call(mp=None) == -1
    assert call(ws=None) == -1
    assert call(wsb=need - 1) == -1
    assert call(ws=fake + 8) == -2
    assert call(n=(1 << 20) + 1, wsb=1 << 46) == -2
    assert lib.veda_distill_grad_workspace(Lp, (1 << 20) + 1, 128, ctypes.byref(ws)) == -2
    L3 = V.veda_layout_init(5, 9, 20, 96, 128, [(8, 4, 4)])
    ws3 = ctypes.c_int64(0)
    assert lib.veda_distill_grad_workspace(ctypes.byref(L3), 5, 128, ctypes.byref(ws3)) == 0
    assert D(ctypes.byref(L3), fake, fake, fake, 5, fake, fake, 128, fake, ws3.value, fake, fake,
             fake, None, None, None) == -2


def test_map_workspace_size(lib):
    # row maxima (n_sub x max_tiles x S f32), the per-chunk (m, l) pairs for up
    # to 16 chunks (n_sub x 16 x S x 2 f32), each rounded up to 256 bytes, then
    # 256 bytes for pass 1's eight work-claim counters
    L = _layout()
    out = ctypes.c_int64(-5)
    assert lib.veda_oracle_maxpool_map_workspace(ctypes.byref(L), 0, ctypes.byref(out)) == 0
    assert out.value == 0
    for n_sub in (1, 3, 400):
        assert lib.veda_oracle_maxpool_map_workspace(ctypes.byref(L), n_sub, ctypes.byref(out)) == 0
        rm = -(-n_sub * L.max_tiles * L.tile_size * 4 // 256) * 256
        ml = -(-n_sub * 16 * L.tile_size * 8 // 256) * 256
        assert out.value == rm + ml + 256
    assert lib.veda_oracle_maxpool_map_workspace(ctypes.byref(L), -1, ctypes.byref(out)) == -1
    assert lib.veda_oracle_maxpool_map_workspace(ctypes.byref(L), 3, None) == -1


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4):
        assert V.status_string(s).startswith("VEDA_")
    assert "unknown" in V.status_string(12345)


def test_product_path_does_not_touch_the_oracle(repo_root):
    pkg = os.path.join(repo_root, "tile_sparse_attention_head_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", src, re.M), f
                assert "oracle/" not in src, f
    for dirpath, _, files in os.walk(os.path.join(repo_root, "oracle")):
        for f in files:
            if f.endswith(".py"):
                src = open(os.path.join(dirpath, f)).read()
                assert "tile_sparse_attention_head_amd" not in src, f
                assert not re.search(r"^\s*(import|from)\s+workloads\b", src, re.M), f


@pytest.mark.parametrize("entry", ["veda_sparse_attn_bwd", "veda_sparse_attn_bwd_tiles"])
def test_backward_rejections_and_workspace(lib, entry):
    """Both backward entry points validate every argument before any launch
    (the fake addresses are never dereferenced)."""
    L = _layout()
    Lp = ctypes.byref(L)
    fake = 1 << 20
    ws = ctypes.c_int64(0)
    assert lib.veda_sparse_attn_bwd_workspace(Lp, 100, ctypes.byref(ws)) == 0
    need = ws.value
    tile_bytes = L.total_tiles * L.tile_size * L.head_dim * 2
    assert need >= 4 * tile_bytes      # gathered Q, K, V and dO at least
    assert lib.veda_sparse_attn_bwd_workspace(Lp, -1, ctypes.byref(ws)) == -1
    assert lib.veda_sparse_attn_bwd_workspace(Lp, 100, None) == -1
    B = getattr(lib, entry)
    span = 1 << 32                      # far apart: no two fake buffers overlap
    ok = dict(q=fake, k=fake + span, v=fake + 2 * span, o=fake + 3 * span, do=fake + 4 * span,
              lse=fake, rp=fake, ci=fake, nnz=100, sc=0.1, ws=fake, wsb=need,
              dq=fake + 5 * span, dk=fake + 6 * span, dv=fake + 7 * span)

    def call(layout=Lp, **kw):
        a = dict(ok, **kw)
        return B(layout, a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["rp"], a["ci"],
                 a["nnz"], a["sc"], a["ws"], a["wsb"], a["dq"], a["dk"], a["dv"], None)

    for name in ("q", "k", "v", "o", "do", "lse", "rp", "ci", "ws", "dq", "dk", "dv"):
        assert call(**{name: None}) == -1, name
    assert call(nnz=-1) == -1
    for bad in (float("nan"), 0.0, -0.1, float("inf")):
        assert call(sc=bad) == -1
    assert call(wsb=need - 1) == -1
    assert call(q=fake + 8) == -2
    assert call(dv=fake + 7 * span + 8) == -2
    assert call(dq=fake + 4096) == -1                 # output over an input
    assert call(dk=fake + 5 * span + 64) == -1        # outputs over each other
    L3 = V.veda_layout_init(5, 9, 20, 96, 128, [(8, 4, 4)])
    assert call(layout=ctypes.byref(L3)) == -2
    L2 = _layout()
    L2.tile_off[1] += 1
    assert call(layout=ctypes.byref(L2)) == -1


def test_head_sq_error_rejections_and_workspace(lib):
    L = _layout()
    Lp = ctypes.byref(L)
    fake = 1 << 20
    span = 1 << 32
    ws = ctypes.c_int64(0)
    assert lib.veda_head_sq_error_workspace(Lp, ctypes.byref(ws)) == 0
    need = ws.value
    assert need > 0
    assert lib.veda_head_sq_error_workspace(Lp, None) == -1
    E = lib.veda_head_sq_error
    assert E(Lp, None, fake + span, fake, None, fake, need, None) == -1
    assert E(Lp, fake, None, fake, None, fake, need, None) == -1
    assert E(Lp, fake, fake + span, None, None, fake, need, None) == -1
    assert E(Lp, fake, fake + span, fake, None, None, need, None) == -1
    assert E(Lp, fake, fake + span, fake, None, fake, need - 1, None) == -1
    assert E(Lp, fake + 8, fake + span, fake, None, fake, need, None) == -2
    assert E(Lp, fake, fake + span, fake, None, fake + 4, need, None) == -2
    L6 = V.veda_layout_init(4, 8, 8, 100, 64, [(4, 4, 4)])   # head_dim/8 does not divide 256
    ws6 = ctypes.c_int64(0)
    assert lib.veda_head_sq_error_workspace(ctypes.byref(L6), ctypes.byref(ws6)) == 0
    assert E(ctypes.byref(L6), fake, fake + span, fake, None, fake, ws6.value, None) == -2


def test_score_select_rejections(lib):
    """veda_score_select refuses bad arguments before any device work (no
    GPU call is made here): k out of range, d_e outside {64, 128}, a
    misaligned phi, rows longer than 2048 tiles."""
    L = _layout()
    Lp = ctypes.byref(L)
    S = lib.veda_score_select
    fake = 1 << 20
    H = L.num_heads
    good = (ctypes.c_int32 * H)(*[1] * H)
    bad = (ctypes.c_int32 * H)(*([0] + [1] * (H - 1)))
    assert S(Lp, None, 128, good, fake, fake, None) == -1
    assert S(Lp, fake, 128, None, fake, fake, None) == -1
    assert S(Lp, fake, 128, good, None, fake, None) == -1
    assert S(Lp, fake, 128, good, fake, None, None) == -1
    assert S(Lp, fake, 0, good, fake, fake, None) == -1
    assert S(Lp, fake, 128, bad, fake, fake, None) == -1
    assert S(Lp, fake, 96, good, fake, fake, None) == -2
    assert S(Lp, fake + 4, 128, good, fake, fake, None) == -2
    Lw = V.veda_layout_init(64, 64, 256, 128, 128, [(1, 8, 16)])   # 8192 tiles per head
    assert S(ctypes.byref(Lw), fake, 128, (ctypes.c_int32 * 1)(410), fake, fake, None) == -2


def test_head_choose_rejections(lib):
    """veda_head_choose refuses bad counts, null or misaligned pointers before
    any device work (no GPU call is made here)."""
    C = lib.veda_head_choose
    fake = 1 << 20
    assert C(None, 4, 24, fake, None) == -1
    assert C(fake, 4, 24, None, None) == -1
    assert C(fake, 0, 24, fake, None) == -1
    assert C(fake, 65, 24, fake, None) == -1
    assert C(fake, -1, 24, fake, None) == -1
    assert C(fake, 4, 0, fake, None) == -1
    assert C(fake, 4, 65, fake, None) == -1
    assert C(fake + 4, 4, 24, fake, None) == -1
    assert C(fake, 4, 24, fake + 2, None) == -1


def test_tiles_per_head_limit(lib):
    """The attention, backward and map calls read a head's K/V tiles through
    a 32-bit buffer range and the forward packs tile indices into 16 bits
    (VEDA_MAX_TILES_PER_HEAD = 65535).  veda_layout_init's own bound (sum of
    n_h^2 within int32) stops at 46340 tiles per head, so the largest layout
    it accepts passes the calls' check and the next one is refused by the
    layout itself; a layout whose max_tiles was raised by hand is refused as
    tampered."""
    text = open(HEADER).read()
    assert re.search(r"#define VEDA_MAX_TILES_PER_HEAD 65535\b", text)
    # one head of (1,1,128) tiles over a T x 1 x 128 grid: n = T tiles
    ok = V.veda_layout_init(46340, 1, 128, 128, 128, [(1, 1, 128)])
    assert ok.max_tiles == 46340
    with pytest.raises(Exception):
        V.veda_layout_init(46341, 1, 128, 128, 128, [(1, 1, 128)])
    ws = ctypes.c_int64(0)
    assert lib.veda_oracle_maxpool_map_workspace(ctypes.byref(ok), 4, ctypes.byref(ws)) == 0
    assert lib.veda_sparse_attn_bwd_workspace(ctypes.byref(ok), 100, ctypes.byref(ws)) == 0
    bad = V.veda_layout_init(46340, 1, 128, 128, 128, [(1, 1, 128)])
    bad.max_tiles = 70000
    fake = 1 << 20
    assert lib.veda_sparse_attn_fwd(ctypes.byref(bad), fake, fake, fake, fake, fake, 0.1, fake,
                                    None, None, 0, None) == -1
    assert lib.veda_oracle_maxpool_map_workspace(ctypes.byref(bad), 4, ctypes.byref(ws)) == -1


def test_distill_noalloc_rejections(lib):
    """The static-scratch distillation call validates like veda_distill_grad
    and refuses, before any device work, a problem whose workspace would not
    fit the library's scratch (VEDA_DISTILL_STATIC_SCRATCH_BYTES)."""
    text = open(HEADER).read()
    m = re.search(r"#define VEDA_DISTILL_STATIC_SCRATCH_BYTES \((\d+)ll << (\d+)\)", text)
    assert m
    cap = int(m.group(1)) << int(m.group(2))
    L = _layout()
    Lp = ctypes.byref(L)
    fake = 1 << 20
    N = lib.veda_distill_grad_noalloc
    ok = dict(sc=fake, mp=fake, qt=fake, n=5, desc=fake, phi=fake, de=128, loss=fake, gq=fake,
              gk=fake)

    def call(layout=Lp, **kw):
        a = dict(ok, **kw)
        return N(layout, a["sc"], a["mp"], a["qt"], a["n"], a["desc"], a["phi"], a["de"],
                 a["loss"], a["gq"], a["gk"], None, None, None)

    assert call(n=-1) == -1
    assert call(de=0) == -1
    assert call(de=300) == -2
    for name in ("desc", "phi", "loss", "gq", "gk", "mp", "sc", "qt"):
        assert call(**{name: None}) == -1, name
    assert call(n=(1 << 20) + 1) == -2
    L2 = _layout()
    L2.tile_off[1] += 1
    assert call(layout=ctypes.byref(L2)) == -1
    # the 720P 241-frame layer: 1920 tiles per head; enough subset rows to
    # overflow the scratch, and the workspace query agrees on the size
    big = V.veda_layout_init(61, 45, 80, 128, 128, [(4, 4, 8)] * 24)
    n_over = cap // (4 * big.max_tiles) + 1
    ws = ctypes.c_int64(0)
    assert lib.veda_distill_grad_workspace(ctypes.byref(big), n_over, 128, ctypes.byref(ws)) == 0
    assert ws.value > cap
    assert call(layout=ctypes.byref(big), n=n_over) == -2
    # the largest subset at this layer that the benchmark uses (10 % of every head) fits
    n_bench = 24 * 192
    assert lib.veda_distill_grad_workspace(ctypes.byref(big), n_bench, 128, ctypes.byref(ws)) == 0
    assert ws.value <= cap

"""ctypes binding of libveda.so.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Each function here has the name of the C entry point it calls
(declared in include/veda.h) and takes torch tensors for device buffers; the
tensors are checked for device, dtype, contiguity and size so that a call
can never hand the kernels a buffer smaller than the layout needs, then
their data pointers and the current HIP stream are passed on.  A non-zero
status raises VedaError.  The library must have been built
(``python -m tile_sparse_attention_head_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

MAX_HEADS = 64
VEDA_BF16, VEDA_F32 = 0, 1
VEDA_FWD, VEDA_INV, VEDA_FWD_T = 0, 1, 2

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libveda.so")

c_i32, c_i64, c_f32, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p


class VedaError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {status_string(status)} ({status})")


class veda_layout(ctypes.Structure):
    _fields_ = [
        ("T", c_i32), ("H", c_i32), ("W", c_i32),
        ("num_heads", c_i32), ("head_dim", c_i32), ("tile_size", c_i32),
        ("tile_shape", (c_i32 * 3) * MAX_HEADS),
        ("tile_grid", (c_i32 * 3) * MAX_HEADS),
        ("n_tiles", c_i32 * MAX_HEADS),
        ("max_tiles", c_i32), ("reserved0", c_i32),
        ("tile_off", c_i64 * (MAX_HEADS + 1)),
        ("score_off", c_i64 * (MAX_HEADS + 1)),
    ]

    # convenience views
    @property
    def heads(self) -> int:
        return self.num_heads

    @property
    def total_tiles(self) -> int:
        return int(self.tile_off[self.num_heads])

    @property
    def total_scores(self) -> int:
        return int(self.score_off[self.num_heads])

    @property
    def tokens(self) -> int:
        return self.T * self.H * self.W

    def n(self, h: int) -> int:
        return int(self.n_tiles[h])

    def shapes(self):
        return [tuple(self.tile_shape[h]) for h in range(self.num_heads)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libveda.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m tile_sparse_attention_head_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(veda_layout)
    sig = {
        "veda_layout_init": (c_i32, [P]),
        "veda_keep_count": (c_i32, [c_i32, c_i32, ctypes.POINTER(c_i32)]),
        "veda_tile_permute": (c_i32, [P, c_i32, c_i32, c_vp, c_vp, c_vp]),
        "veda_tripool_score": (c_i32, [P, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32,
                                       c_vp, c_vp, c_vp, c_vp]),
        "veda_tile_permute_pool": (c_i32, [P, c_i32, c_vp, c_vp, c_vp, c_vp]),
        "veda_tile_score": (c_i32, [P, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp]),
        "veda_select_tiles": (c_i32, [P, c_vp, ctypes.POINTER(c_i32), c_vp, c_vp, c_vp]),
        "veda_score_select": (c_i32, [P, c_vp, c_i32, ctypes.POINTER(c_i32), c_vp, c_vp, c_vp]),
        "veda_sparse_attn_fwd": (c_i32, [P, c_vp, c_vp, c_vp, c_vp, c_vp, c_f32, c_vp, c_vp,
                                         c_vp, c_i64, c_vp]),
        "veda_sparse_attn_fwd_tokens": (c_i32, [P, c_vp, c_vp, c_vp, c_vp, c_vp, c_f32, c_vp,
                                                c_vp, c_vp, c_i64, c_vp]),
        "veda_sparse_attn_fwd_workspace": (c_i32, [P, ctypes.POINTER(c_i64)]),
        "veda_oracle_maxpool_map": (c_i32, [P, c_vp, c_vp, c_f32, c_vp, c_i32, c_vp, c_i64,
                                            c_vp, c_vp, c_vp]),
        "veda_oracle_maxpool_map_workspace": (c_i32, [P, c_i32, ctypes.POINTER(c_i64)]),
        "veda_distill_grad": (c_i32, [P, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_i32, c_vp, c_i64,
                                      c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
        "veda_distill_grad_workspace": (c_i32, [P, c_i32, c_i32, ctypes.POINTER(c_i64)]),
        "veda_distill_grad_noalloc": (c_i32, [P, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_i32,
                                              c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
        "veda_head_sq_error": (c_i32, [P, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_vp]),
        "veda_head_sq_error_workspace": (c_i32, [P, ctypes.POINTER(c_i64)]),
        "veda_head_choose": (c_i32, [c_vp, c_i32, c_i32, c_vp, c_vp]),
        "veda_sparse_attn_bwd": (c_i32, [P, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64,
                                         c_f32, c_vp, c_i64, c_vp, c_vp, c_vp, c_vp]),
        "veda_sparse_attn_bwd_tiles": (c_i32, [P, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                               c_i64, c_f32, c_vp, c_i64, c_vp, c_vp, c_vp, c_vp]),
        "veda_sparse_attn_bwd_workspace": (c_i32, [P, c_i64, ctypes.POINTER(c_i64)]),
        "veda_status_string": (ctypes.c_char_p, [c_i32]),
        "veda_layout_sizeof": (c_i64, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype, fn.argtypes = res, args
    if L.veda_layout_sizeof() != ctypes.sizeof(veda_layout):
        raise ImportError("veda_layout size mismatch between libveda.so and the binding")
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().veda_status_string(int(status)).decode()


def _check(status: int, call: str) -> None:
    if status != 0:
        raise VedaError(status, call)


# ---------------------------------------------------------------- host calls
def veda_layout_init(T: int, H: int, W: int, head_dim: int, tile_size: int,
                     tile_shapes: Sequence[Tuple[int, int, int]]) -> veda_layout:
    L = veda_layout()
    L.T, L.H, L.W = int(T), int(H), int(W)
    L.num_heads = len(tile_shapes)
    L.head_dim, L.tile_size = int(head_dim), int(tile_size)
    if not 1 <= L.num_heads <= MAX_HEADS:
        raise VedaError(-1, "veda_layout_init")
    for h, s in enumerate(tile_shapes):
        for a in range(3):
            L.tile_shape[h][a] = int(s[a])
    _check(lib().veda_layout_init(ctypes.byref(L)), "veda_layout_init")
    return L


def veda_keep_count(n_tiles: int, sparsity_pct: int) -> int:
    k = c_i32(0)
    _check(lib().veda_keep_count(int(n_tiles), int(sparsity_pct), ctypes.byref(k)),
           "veda_keep_count")
    return int(k.value)


# ------------------------------------------------------------- device calls
def _torch():
    import torch
    return torch


def _stream(stream) -> int:
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return int(getattr(stream, "cuda_stream", stream))


def _dev(t, name: str, dtype, numel: int, allow_none: bool = False) -> Optional[int]:
    torch = _torch()
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return t.data_ptr()


def _code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return VEDA_BF16
    if t.dtype == torch.float32:
        return VEDA_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def tokens_numel(L: veda_layout) -> int:
    return L.tokens * L.num_heads * L.head_dim


def tiles_numel(L: veda_layout) -> int:
    return L.total_tiles * L.tile_size * L.head_dim


def veda_tile_permute(L: veda_layout, x, y, direction: int = VEDA_FWD, stream=None) -> None:
    torch = _torch()
    dt = _code(x)
    src_n = tiles_numel(L) if direction == VEDA_INV else tokens_numel(L)
    dst_n = tokens_numel(L) if direction == VEDA_INV else tiles_numel(L)
    px = _dev(x, "x", (torch.bfloat16, torch.float32), src_n)
    py = _dev(y, "y", x.dtype, dst_n)
    _check(lib().veda_tile_permute(ctypes.byref(L), dt, int(direction), px, py, _stream(stream)),
           "veda_tile_permute")


def veda_tripool_score(L: veda_layout, q_perm, k_perm, w_q, w_k, desc, phi, scores,
                       b_q=None, b_k=None, stream=None) -> None:
    torch = _torch()
    f32 = torch.float32
    H, d = L.num_heads, L.head_dim
    d_e = int(w_q.shape[1])
    if tuple(w_q.shape) != (H, d_e, 3 * d) or tuple(w_k.shape) != (H, d_e, 3 * d):
        raise ValueError("w_q/w_k must be [heads][d_e][3*head_dim]")
    dt = _code(q_perm)
    args = [
        _dev(q_perm, "q_perm", (torch.bfloat16, f32), tiles_numel(L)),
        _dev(k_perm, "k_perm", q_perm.dtype, tiles_numel(L)),
        _dev(w_q, "w_q", f32, H * d_e * 3 * d), _dev(w_k, "w_k", f32, H * d_e * 3 * d),
        _dev(b_q, "b_q", f32, H * d_e, True), _dev(b_k, "b_k", f32, H * d_e, True),
    ]
    outs = [_dev(desc, "desc", f32, 2 * L.total_tiles * 3 * d),
            _dev(phi, "phi", f32, 2 * L.total_tiles * d_e),
            _dev(scores, "scores", f32, L.total_scores)]
    _check(lib().veda_tripool_score(ctypes.byref(L), dt, args[0], args[1], args[2], args[3],
                                    args[4], args[5], d_e, *outs, _stream(stream)),
           "veda_tripool_score")


def veda_tile_permute_pool(L: veda_layout, x, y, desc, stream=None) -> None:
    """Gather x (token order) into y (tile order) and write the tiles'
    TripPool descriptors to desc ([tiles][3*head_dim] f32)."""
    torch = _torch()
    dt = _code(x)
    px = _dev(x, "x", (torch.bfloat16, torch.float32), tokens_numel(L))
    py = _dev(y, "y", x.dtype, tiles_numel(L))
    pd = _dev(desc, "desc", torch.float32, L.total_tiles * 3 * L.head_dim)
    _check(lib().veda_tile_permute_pool(ctypes.byref(L), dt, px, py, pd, _stream(stream)),
           "veda_tile_permute_pool")


def veda_tile_score(L: veda_layout, desc, w_q, w_k, phi, scores, b_q=None, b_k=None,
                    stream=None) -> None:
    """Projection and tile scores from descriptors desc [2][tiles][3*head_dim];
    scores None: the projection only (veda_score_select takes phi from there)."""
    torch = _torch()
    f32 = torch.float32
    H, d = L.num_heads, L.head_dim
    d_e = int(w_q.shape[1])
    if tuple(w_q.shape) != (H, d_e, 3 * d) or tuple(w_k.shape) != (H, d_e, 3 * d):
        raise ValueError("w_q/w_k must be [heads][d_e][3*head_dim]")
    args = [_dev(desc, "desc", f32, 2 * L.total_tiles * 3 * d),
            _dev(w_q, "w_q", f32, H * d_e * 3 * d), _dev(w_k, "w_k", f32, H * d_e * 3 * d),
            _dev(b_q, "b_q", f32, H * d_e, True), _dev(b_k, "b_k", f32, H * d_e, True)]
    outs = [_dev(phi, "phi", f32, 2 * L.total_tiles * d_e),
            _dev(scores, "scores", f32, L.total_scores, True)]
    _check(lib().veda_tile_score(ctypes.byref(L), *args, d_e, *outs, _stream(stream)),
           "veda_tile_score")


def csr_nnz(L: veda_layout, k_per_head: Sequence[int]) -> int:
    return sum(L.n(h) * int(k_per_head[h]) for h in range(L.num_heads))


def veda_select_tiles(L: veda_layout, scores, k_per_head: Sequence[int], row_ptr, col_idx,
                      stream=None) -> None:
    torch = _torch()
    if len(k_per_head) != L.num_heads:
        raise ValueError("k_per_head needs one entry per head")
    kh = (c_i32 * L.num_heads)(*[int(v) for v in k_per_head])
    ps = _dev(scores, "scores", torch.float32, L.total_scores)
    prp = _dev(row_ptr, "row_ptr", torch.int32, L.total_tiles + 1)
    pci = _dev(col_idx, "col_idx", torch.int32, csr_nnz(L, k_per_head))
    _check(lib().veda_select_tiles(ctypes.byref(L), ps, kh, prp, pci, _stream(stream)),
           "veda_select_tiles")


def veda_score_select(L: veda_layout, phi, d_e: int, k_per_head: Sequence[int], row_ptr,
                      col_idx, stream=None) -> None:
    """The tile scores of phi [2][tiles][d_e] and their row-wise top-k as CSR,
    with the score matrix never stored (same CSR as veda_tile_score followed
    by veda_select_tiles)."""
    torch = _torch()
    if len(k_per_head) != L.num_heads:
        raise ValueError("k_per_head needs one entry per head")
    kh = (c_i32 * L.num_heads)(*[int(v) for v in k_per_head])
    pp = _dev(phi, "phi", torch.float32, 2 * L.total_tiles * int(d_e))
    prp = _dev(row_ptr, "row_ptr", torch.int32, L.total_tiles + 1)
    pci = _dev(col_idx, "col_idx", torch.int32, csr_nnz(L, k_per_head))
    _check(lib().veda_score_select(ctypes.byref(L), pp, int(d_e), kh, prp, pci, _stream(stream)),
           "veda_score_select")


def veda_sparse_attn_fwd_workspace(L: veda_layout) -> int:
    """Bytes of device workspace the attention forward calls use."""
    out = c_i64(0)
    _check(lib().veda_sparse_attn_fwd_workspace(ctypes.byref(L), ctypes.byref(out)),
           "veda_sparse_attn_fwd_workspace")
    return int(out.value)


def _attn_workspace(L: veda_layout, workspace):
    """(pointer, bytes) of an optional attention workspace tensor."""
    if workspace is None:
        return None, 0
    need = veda_sparse_attn_fwd_workspace(L)
    pw = _dev(workspace, "workspace", None, 0)
    have = workspace.numel() * workspace.element_size()
    if have < need:
        raise ValueError(f"workspace holds {have} bytes, needs {need}")
    return pw, have


def veda_sparse_attn_fwd(L: veda_layout, q_perm, k_perm, vt_perm, row_ptr, col_idx,
                         sm_scale: float, o_perm, lse=None, workspace=None, stream=None) -> None:
    """workspace: None, or a contiguous GPU tensor of at least
    veda_sparse_attn_fwd_workspace(L) bytes (the end of each XCD's share of
    query tiles is then balanced across XCDs; the results are the same)."""
    torch = _torch()
    bf = torch.bfloat16
    n = tiles_numel(L)
    args = [_dev(q_perm, "q_perm", bf, n), _dev(k_perm, "k_perm", bf, n),
            _dev(vt_perm, "vt_perm", bf, n),
            _dev(row_ptr, "row_ptr", torch.int32, L.total_tiles + 1),
            _dev(col_idx, "col_idx", torch.int32, 0)]
    po = _dev(o_perm, "o_perm", bf, n)
    pl = _dev(lse, "lse", torch.float32, L.total_tiles * L.tile_size, True)
    pw, have = _attn_workspace(L, workspace)
    _check(lib().veda_sparse_attn_fwd(ctypes.byref(L), *args, float(sm_scale), po, pl, pw, have,
                                      _stream(stream)),
           "veda_sparse_attn_fwd")


def veda_sparse_attn_fwd_tokens(L: veda_layout, q_perm, k_perm, vt_perm, row_ptr, col_idx,
                                sm_scale: float, o, lse=None, workspace=None,
                                stream=None) -> None:
    """As veda_sparse_attn_fwd, with O written in token order [N][heads][d]."""
    torch = _torch()
    bf = torch.bfloat16
    n = tiles_numel(L)
    args = [_dev(q_perm, "q_perm", bf, n), _dev(k_perm, "k_perm", bf, n),
            _dev(vt_perm, "vt_perm", bf, n),
            _dev(row_ptr, "row_ptr", torch.int32, L.total_tiles + 1),
            _dev(col_idx, "col_idx", torch.int32, 0)]
    po = _dev(o, "o", bf, tokens_numel(L))
    pl = _dev(lse, "lse", torch.float32, L.total_tiles * L.tile_size, True)
    pw, have = _attn_workspace(L, workspace)
    _check(lib().veda_sparse_attn_fwd_tokens(ctypes.byref(L), *args, float(sm_scale), po, pl, pw,
                                             have, _stream(stream)),
           "veda_sparse_attn_fwd_tokens")


def veda_oracle_maxpool_map_workspace(L: veda_layout, n_sub: int) -> int:
    """Bytes of device workspace veda_oracle_maxpool_map needs for n_sub entries."""
    out = c_i64(0)
    _check(lib().veda_oracle_maxpool_map_workspace(ctypes.byref(L), int(n_sub), ctypes.byref(out)),
           "veda_oracle_maxpool_map_workspace")
    return int(out.value)


def veda_oracle_maxpool_map(L: veda_layout, q_perm, k_perm, sm_scale: float, q_tiles, workspace,
                            lse, out_map, stream=None) -> None:
    """workspace: a contiguous GPU tensor of at least
    veda_oracle_maxpool_map_workspace(L, n_sub) bytes (any dtype)."""
    torch = _torch()
    bf = torch.bfloat16
    n_sub = int(q_tiles.numel())
    n = tiles_numel(L)
    args = [_dev(q_perm, "q_perm", bf, n), _dev(k_perm, "k_perm", bf, n)]
    pq = _dev(q_tiles, "q_tiles", torch.int32, n_sub)
    need = veda_oracle_maxpool_map_workspace(L, n_sub)
    pw = _dev(workspace, "workspace", None, 0)
    have = workspace.numel() * workspace.element_size()
    if have < need:
        raise ValueError(f"workspace holds {have} bytes, needs {need}")
    pl = _dev(lse, "lse", torch.float32, n_sub * L.tile_size)
    pm = _dev(out_map, "map", torch.float32, n_sub * L.max_tiles)
    _check(lib().veda_oracle_maxpool_map(ctypes.byref(L), args[0], args[1], float(sm_scale), pq,
                                         n_sub, pw, have, pl, pm, _stream(stream)),
           "veda_oracle_maxpool_map")


def veda_distill_grad_workspace(L: veda_layout, n_sub: int, d_e: int) -> int:
    """Bytes of device workspace veda_distill_grad needs."""
    out = c_i64(0)
    _check(lib().veda_distill_grad_workspace(ctypes.byref(L), int(n_sub), int(d_e),
                                             ctypes.byref(out)),
           "veda_distill_grad_workspace")
    return int(out.value)


def veda_distill_grad(L: veda_layout, scores, out_map, q_tiles, desc, phi, d_e: int, workspace,
                      loss, grad_w_q, grad_w_k, grad_b_q=None, grad_b_k=None,
                      stream=None) -> None:
    """Row-wise KL distillation loss and its projection gradients; workspace
    of at least veda_distill_grad_workspace(L, n_sub, d_e) bytes."""
    torch = _torch()
    f32 = torch.float32
    n_sub = int(q_tiles.numel())
    d = L.head_dim
    H = L.num_heads
    ps = _dev(scores, "scores", f32, L.total_scores)
    pm = _dev(out_map, "map", f32, n_sub * L.max_tiles)
    pq = _dev(q_tiles, "q_tiles", torch.int32, n_sub)
    pd = _dev(desc, "desc", f32, 2 * L.total_tiles * 3 * d)
    pp = _dev(phi, "phi", f32, 2 * L.total_tiles * int(d_e))
    need = veda_distill_grad_workspace(L, n_sub, d_e)
    pw = _dev(workspace, "workspace", None, 0)
    have = workspace.numel() * workspace.element_size()
    if have < need:
        raise ValueError(f"workspace holds {have} bytes, needs {need}")
    pl = _dev(loss, "loss", f32, 1)
    gq = _dev(grad_w_q, "grad_w_q", f32, H * int(d_e) * 3 * d)
    gk = _dev(grad_w_k, "grad_w_k", f32, H * int(d_e) * 3 * d)
    bq = _dev(grad_b_q, "grad_b_q", f32, H * int(d_e), True)
    bk = _dev(grad_b_k, "grad_b_k", f32, H * int(d_e), True)
    _check(lib().veda_distill_grad(ctypes.byref(L), ps, pm, pq, n_sub, pd, pp, int(d_e), pw, have,
                                   pl, gq, gk, bq, bk, _stream(stream)),
           "veda_distill_grad")


def veda_distill_grad_noalloc(L: veda_layout, scores, out_map, q_tiles, desc, phi, d_e: int,
                              loss, grad_w_q, grad_w_k, grad_b_q=None, grad_b_k=None,
                              stream=None) -> None:
    """veda_distill_grad in the library's static per-GPU scratch: no
    workspace argument, nothing allocated; calls overlapping on one GPU race."""
    torch = _torch()
    f32 = torch.float32
    n_sub = int(q_tiles.numel())
    d = L.head_dim
    H = L.num_heads
    ps = _dev(scores, "scores", f32, L.total_scores)
    pm = _dev(out_map, "map", f32, n_sub * L.max_tiles)
    pq = _dev(q_tiles, "q_tiles", torch.int32, n_sub)
    pd = _dev(desc, "desc", f32, 2 * L.total_tiles * 3 * d)
    pp = _dev(phi, "phi", f32, 2 * L.total_tiles * int(d_e))
    pl = _dev(loss, "loss", f32, 1)
    gq = _dev(grad_w_q, "grad_w_q", f32, H * int(d_e) * 3 * d)
    gk = _dev(grad_w_k, "grad_w_k", f32, H * int(d_e) * 3 * d)
    bq = _dev(grad_b_q, "grad_b_q", f32, H * int(d_e), True)
    bk = _dev(grad_b_k, "grad_b_k", f32, H * int(d_e), True)
    _check(lib().veda_distill_grad_noalloc(ctypes.byref(L), ps, pm, pq, n_sub, pd, pp, int(d_e),
                                           pl, gq, gk, bq, bk, _stream(stream)),
           "veda_distill_grad_noalloc")


def veda_head_sq_error_workspace(L: veda_layout) -> int:
    out = c_i64(0)
    _check(lib().veda_head_sq_error_workspace(ctypes.byref(L), ctypes.byref(out)),
           "veda_head_sq_error_workspace")
    return int(out.value)


def veda_head_sq_error(L: veda_layout, a, b, err, workspace, ref=None, stream=None) -> None:
    """err[h] = sum (a - b)^2 over head h of two bf16 token-order outputs
    (and ref[h] = sum a^2); err/ref f64 [num_heads]."""
    torch = _torch()
    n = tokens_numel(L)
    pa = _dev(a, "a", torch.bfloat16, n)
    pb = _dev(b, "b", torch.bfloat16, n)
    pe = _dev(err, "err", torch.float64, L.num_heads)
    pr = _dev(ref, "ref", torch.float64, L.num_heads, True)
    pw = _dev(workspace, "workspace", None, 0)
    have = workspace.numel() * workspace.element_size()
    _check(lib().veda_head_sq_error(ctypes.byref(L), pa, pb, pe, pr, pw, have, _stream(stream)),
           "veda_head_sq_error")


def veda_head_choose(err, choice, stream=None) -> None:
    """choice[h] = the candidate c with the smallest err[c][h] (the first of
    equal ones); err f64 [n_cand][heads], choice int32 [heads], on the GPU."""
    torch = _torch()
    if err is None or err.dim() != 2:
        raise ValueError("err must be a 2-D [n_cand][heads] tensor")
    n_cand, heads = int(err.shape[0]), int(err.shape[1])
    pe = _dev(err, "err", torch.float64, n_cand * heads)
    pc = _dev(choice, "choice", torch.int32, heads)
    _check(lib().veda_head_choose(pe, n_cand, heads, pc, _stream(stream)), "veda_head_choose")


def veda_sparse_attn_bwd_workspace(L: veda_layout, nnz: int) -> int:
    out = c_i64(0)
    _check(lib().veda_sparse_attn_bwd_workspace(ctypes.byref(L), int(nnz), ctypes.byref(out)),
           "veda_sparse_attn_bwd_workspace")
    return int(out.value)


def veda_sparse_attn_bwd(L: veda_layout, q, k, v, o, d_o, lse, row_ptr, col_idx, nnz: int,
                         sm_scale: float, workspace, dq, dk, dv, stream=None) -> None:
    """dQ, dK, dV (bf16 token order) of the tile-skipping attention; workspace
    of at least veda_sparse_attn_bwd_workspace(L, nnz) bytes."""
    torch = _torch()
    bf = torch.bfloat16
    n = tokens_numel(L)
    ins = [_dev(t, name, bf, n) for t, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o"),
                                                (d_o, "d_o"))]
    pl = _dev(lse, "lse", torch.float32, L.total_tiles * L.tile_size)
    prp = _dev(row_ptr, "row_ptr", torch.int32, L.total_tiles + 1)
    pci = _dev(col_idx, "col_idx", torch.int32, int(nnz))
    pw = _dev(workspace, "workspace", None, 0)
    have = workspace.numel() * workspace.element_size()
    outs = [_dev(t, name, bf, n) for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv"))]
    _check(lib().veda_sparse_attn_bwd(ctypes.byref(L), *ins, pl, prp, pci, int(nnz),
                                      float(sm_scale), pw, have, *outs, _stream(stream)),
           "veda_sparse_attn_bwd")


def veda_sparse_attn_bwd_tiles(L: veda_layout, q_perm, k_perm, v, o, d_o, lse, row_ptr, col_idx,
                               nnz: int, sm_scale: float, workspace, dq, dk, dv,
                               stream=None) -> None:
    """veda_sparse_attn_bwd with Q and K already in tile order (the forward's
    gathers); the same results."""
    torch = _torch()
    bf = torch.bfloat16
    n, nt = tokens_numel(L), tiles_numel(L)
    ins = [_dev(q_perm, "q_perm", bf, nt), _dev(k_perm, "k_perm", bf, nt)]
    ins += [_dev(t, name, bf, n) for t, name in ((v, "v"), (o, "o"), (d_o, "d_o"))]
    pl = _dev(lse, "lse", torch.float32, L.total_tiles * L.tile_size)
    prp = _dev(row_ptr, "row_ptr", torch.int32, L.total_tiles + 1)
    pci = _dev(col_idx, "col_idx", torch.int32, int(nnz))
    pw = _dev(workspace, "workspace", None, 0)
    have = workspace.numel() * workspace.element_size()
    outs = [_dev(t, name, bf, n) for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv"))]
    _check(lib().veda_sparse_attn_bwd_tiles(ctypes.byref(L), *ins, pl, prp, pci, int(nnz),
                                            float(sm_scale), pw, have, *outs, _stream(stream)),
           "veda_sparse_attn_bwd_tiles")

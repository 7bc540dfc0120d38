"""Seeded synthetic video-token workloads for the tile-sparse attention path.

This module only draws inputs. It holds none of the method's arithmetic (no
tiling, pooling, scoring, selection or attention): both the HIP path and the
CPU oracle consume the arrays it returns, and neither is imported here.

Stand-in for real DiT activations
---------------------------------
The method is evaluated on self-attention layers of Wan2.1-T2V (1.3B/14B) and
Waver-T2V (1B/12B) at 480P/720P with 81/121/241 frames ("Veda" summary §4 and
the per-layer latency table of the aikraft.ru news item on Veda).  Those
weights and activations are not available, so seeded Gaussian tensors with the
same shapes stand in for them:

* Q, K, V are laid out ``[N][heads][d]`` with token ``n = (t*H + h)*W + w``
  (row-major over the T x H x W latent grid), as a fused QKV projection emits.
* Q and K of the large workloads carry a rank-8 spatio-temporal positional
  component so that nearby tokens (hence nearby tiles) have larger logits; V is
  plain Gaussian.  For head ``h`` with tile shape ``(pt, ph, pw)`` the length
  scale is ``l_h = 2*(pt, ph, pw)``; four frequencies ``w_i ~ N(0, diag(l_h^-2))``
  give features ``f(x) = [cos(w_i.x), sin(w_i.x)]`` at the integer coordinate
  ``x = (t, h, w)``; ``U_h`` (d x 8) has orthonormal columns and
  ``Q_pos = K_pos = beta * f(x) U_h^T`` with ``beta^2 = alpha / (4 sm_scale)``, so
  that ``sm_scale * Q_pos(x).K_pos(y) = (alpha/4) * sum_i cos(w_i.(x-y))``, which
  peaks at ``alpha = 6`` logits for co-located tokens.
* Values are drawn in fp32, summed in fp32 and rounded once to bf16
  (round-to-nearest-even); both sides consume the same rounded bits.
* Estimator weights are ``N(0, 0.02)`` of shape ``[heads][d_e][3d]`` (one
  projection per head, used for the query side and the key side alike).

Random streams: ``SeedSequence(seed).spawn(7)`` in the role order
``tiles, q, k, v, pos, mlp, subset``; each role has its own PCG64 generator, so
changing the token count (length sweep) keeps the per-head tile draw.
"""
from __future__ import annotations

import math
import os
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

ROLES = ("tiles", "q", "k", "v", "pos", "mlp", "subset")

# Tile shapes a head may draw: every one factorises a 128-token hardware tile
# ("Veda" summary §2.2: per-layer, per-head (pt, ph, pw) factorising the tile).
TILE_CHOICES: Tuple[Tuple[int, int, int], ...] = ((1, 8, 16), (2, 8, 8), (4, 4, 8), (8, 4, 4))

POS_ALPHA = 6.0
POS_RANK_FREQS = 4          # 4 frequencies -> 8 features (cos, sin)
MLP_STD = 0.02


@dataclass(frozen=True)
class Config:
    """One synthetic attention-layer workload."""

    name: str
    T: int
    H: int
    W: int
    heads: int
    head_dim: int
    tile_size: int
    fixed_tile: Optional[Tuple[int, int, int]]   # None -> per-head draw from TILE_CHOICES
    sparsities: Tuple[int, ...]                  # tile sparsity levels, percent
    positional: bool
    sm_scale: float
    q_prescale: float = 1.0
    dtype: str = "bf16"                          # "bf16" or "f32" (values before rounding)
    map_subset_pct: int = 0                      # query-tile subset for the max-pooled map
    description: str = ""

    @property
    def tokens(self) -> int:
        return self.T * self.H * self.W


CONFIGS: Dict[str, Config] = {
    "tiny": Config(
        "tiny", 4, 8, 8, heads=1, head_dim=64, tile_size=64, fixed_tile=(4, 4, 4),
        sparsities=(50, 0), positional=False, sm_scale=1.0, q_prescale=1.0 / 8.0,
        dtype="f32", map_subset_pct=100,
        description="1 head, 4x8x8 grid, d=64, tile (4,4,4), keep 2 of 4 KV tiles"),
    "wan1.3b-480p-81f": Config(
        "wan1.3b-480p-81f", 21, 30, 52, heads=12, head_dim=128, tile_size=128,
        fixed_tile=(4, 4, 8), sparsities=(90, 95, 0), positional=True,
        sm_scale=1.0 / math.sqrt(128.0), map_subset_pct=10,
        description="Wan2.1-1.3B-like 480P 81-frame layer, 12 heads, 21x30x52 latent"),
    "wan14b-720p-81f": Config(
        "wan14b-720p-81f", 21, 45, 80, heads=40, head_dim=128, tile_size=128,
        fixed_tile=None, sparsities=(95, 90, 0), positional=True,
        sm_scale=1.0 / math.sqrt(128.0), map_subset_pct=10,
        description="Wan2.1-14B-like 720P 81-frame layer, 40 heads, 21x45x80 latent"),
    "waver12b-720p-121f": Config(
        "waver12b-720p-121f", 31, 45, 80, heads=32, head_dim=128, tile_size=128,
        fixed_tile=None, sparsities=(0, 90, 95), positional=True,
        sm_scale=1.0 / math.sqrt(128.0), map_subset_pct=10,
        description="Waver-12B-like 720P 121-frame layer, 32 heads, 31x45x80 latent"),
    "long-720p-241f": Config(
        "long-720p-241f", 61, 45, 80, heads=24, head_dim=128, tile_size=128,
        fixed_tile=None, sparsities=(95, 0), positional=True,
        sm_scale=1.0 / math.sqrt(128.0), map_subset_pct=10,
        description="720P 241-frame layer, 24 heads, 61x45x80 latent (219,600 tokens)"),
    # Small heterogeneous case for full element-wise parity: several tiles per
    # head, partial tiles on every grid face, all four tile shapes.
    "ragged-small": Config(
        "ragged-small", 5, 9, 20, heads=4, head_dim=128, tile_size=128,
        fixed_tile=None, sparsities=(75, 0), positional=True,
        sm_scale=1.0 / math.sqrt(128.0), map_subset_pct=50,
        description="5x9x20 grid, 4 heads, d=128, mixed tile shapes, ragged edges"),
    # d=64 / S=64 heterogeneous case (tile shapes factorising 64).
    "ragged-d64": Config(
        "ragged-d64", 6, 10, 13, heads=3, head_dim=64, tile_size=64,
        fixed_tile=None, sparsities=(60, 0), positional=True,
        sm_scale=1.0 / math.sqrt(64.0), map_subset_pct=50,
        description="6x10x13 grid, 3 heads, d=64, S=64, mixed tile shapes"),
}

# Token-length sweep for the long workload (same per-head tile draw).
LENGTH_SWEEP_T = (9, 18, 36, 61)

TILE_CHOICES_64: Tuple[Tuple[int, int, int], ...] = ((1, 8, 8), (2, 4, 8), (4, 4, 4), (4, 2, 8))


@dataclass
class Workload:
    """Host arrays of one workload.  Q/K/V are bf16 bit patterns (uint16) for
    bf16 configs; for f32 configs ``q32/k32/v32`` hold the fp32 values and the
    bf16 fields hold their round-to-nearest-even images."""

    config: Config
    T: int
    seed: int
    tile_shapes: List[Tuple[int, int, int]]
    q: np.ndarray            # uint16 [N][heads][d]
    k: np.ndarray
    v: np.ndarray
    w: np.ndarray            # float32 [heads][d_e][3d]
    q32: Optional[np.ndarray] = None
    k32: Optional[np.ndarray] = None
    v32: Optional[np.ndarray] = None
    extras: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        return self.T * self.config.H * self.config.W

    @property
    def sm_scale(self) -> float:
        return self.config.sm_scale


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round to nearest, ties to even:
    bits 16..31 of ``b + 0x7FFF + bit16(b)`` for the fp32 bit pattern ``b``.
    The sum is formed in uint32; it wraps past 2^32 only for NaN patterns,
    and the wrap changes no bit below 32, so the kept half is the same as in
    exact arithmetic.  Large arrays are done in chunks on a few threads (numpy
    releases the GIL in these operations)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.reshape(-1).view(np.uint32)
    out = np.empty(b.size, dtype=np.uint16)

    def part(lo: int, hi: int) -> None:
        src = b[lo:hi]
        t = src >> 16
        t &= 1
        t += 0x7FFF
        t += src
        t >>= 16
        out[lo:hi] = t

    chunk = 1 << 22
    if b.size <= chunk:
        part(0, b.size)
    else:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            list(ex.map(lambda lo: part(lo, min(lo + chunk, b.size)), range(0, b.size, chunk)))
    return out.reshape(x.shape)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit pattern (uint16) -> exact fp32 values."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)


def _streams(seed: int) -> Dict[str, np.random.Generator]:
    children = np.random.SeedSequence(seed).spawn(len(ROLES))
    return {r: np.random.Generator(np.random.PCG64(c)) for r, c in zip(ROLES, children)}


def draw_tile_shapes(cfg: Config, rng: np.random.Generator) -> List[Tuple[int, int, int]]:
    if cfg.fixed_tile is not None:
        return [tuple(cfg.fixed_tile)] * cfg.heads
    choices = TILE_CHOICES if cfg.tile_size == 128 else TILE_CHOICES_64
    idx = rng.integers(0, len(choices), size=cfg.heads)
    return [tuple(choices[i]) for i in idx]


def _token_coords(T: int, H: int, W: int) -> np.ndarray:
    """Integer (t, h, w) of every token in row-major order, shape [N][3]."""
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    return np.stack([t.ravel(), h.ravel(), w.ravel()], axis=1).astype(np.float64)


def positional_term(T: int, H: int, W: int, d: int, tile_shape, sm_scale: float,
                    rng: np.random.Generator, alpha: float = POS_ALPHA) -> np.ndarray:
    """Rank-8 positional component of one head, fp32 [N][d] (see module doc)."""
    ell = 2.0 * np.asarray(tile_shape, dtype=np.float64)
    omega = rng.standard_normal((POS_RANK_FREQS, 3)) / ell[None, :]
    g = rng.standard_normal((d, 2 * POS_RANK_FREQS))
    u, _ = np.linalg.qr(g)                     # d x 8, orthonormal columns
    x = _token_coords(T, H, W)
    phase = x @ omega.T                        # [N][4]
    feats = np.concatenate([np.cos(phase), np.sin(phase)], axis=1)
    beta = math.sqrt(alpha / (4.0 * sm_scale))
    return (beta * (feats @ u.T)).astype(np.float32)


def make(name: str, seed: int = 0, T: Optional[int] = None) -> Workload:
    """Draw the workload ``name`` (a key of CONFIGS).  ``T`` overrides the
    frame count (length sweep) while keeping the per-head tile draw."""
    cfg = CONFIGS[name]
    T = cfg.T if T is None else int(T)
    H, W, nh, d = cfg.H, cfg.W, cfg.heads, cfg.head_dim
    N = T * H * W
    rs = _streams(seed)
    shapes = draw_tile_shapes(cfg, rs["tiles"])
    q = rs["q"].standard_normal((N, nh, d), dtype=np.float32)
    k = rs["k"].standard_normal((N, nh, d), dtype=np.float32)
    v = rs["v"].standard_normal((N, nh, d), dtype=np.float32)
    if cfg.positional:
        for h in range(nh):
            pos = positional_term(T, H, W, d, shapes[h], cfg.sm_scale, rs["pos"])
            q[:, h, :] += pos
            k[:, h, :] += pos
    if cfg.q_prescale != 1.0:
        q *= np.float32(cfg.q_prescale)
    w = (rs["mlp"].standard_normal((nh, d, 3 * d)) * MLP_STD).astype(np.float32)
    wl = Workload(cfg, T, seed, shapes, bf16_round(q), bf16_round(k), bf16_round(v), w)
    if cfg.dtype == "f32":
        wl.q32, wl.k32, wl.v32 = q, k, v
    wl.extras["subset_rng_state"] = rs["subset"].bit_generator.state
    return wl


def draw_subset(wl: Workload, n_tiles: Sequence[int], pct: Optional[int] = None) -> List[np.ndarray]:
    """Random query-tile subset per head for the max-pooled map: for head h,
    ceil(pct * n_tiles[h] / 100) distinct tile indices, sorted ascending.
    ``n_tiles`` is the per-head tile count (an input here)."""
    pct = wl.config.map_subset_pct if pct is None else pct
    rng = np.random.Generator(np.random.PCG64())
    rng.bit_generator.state = wl.extras["subset_rng_state"]
    out = []
    for n in n_tiles:
        m = max(1, -(-int(n) * int(pct) // 100))
        out.append(np.sort(rng.choice(int(n), size=m, replace=False)).astype(np.int64))
    return out


def random_scores(rows: int, cols: int, seed: int, ties: bool = False) -> np.ndarray:
    """fp32 score matrix for selection tests; with ``ties`` values are drawn
    from a small set so that equal scores (and +-0.0) are common."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if ties:
        vals = np.array([-1.0, -0.0, 0.0, 0.25, 0.5, 1.0], dtype=np.float32)
        return vals[rng.integers(0, len(vals), size=(rows, cols))]
    return rng.standard_normal((rows, cols), dtype=np.float32)

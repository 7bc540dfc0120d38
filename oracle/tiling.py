"""Head-aware tiling: which token sits in which slot of which tile.

Veda §2.2 (head-aware tiling): each head of each layer has its own tile shape
pi = (pt, ph, pw) whose volume is the hardware tile size S; the tokens of the
T x H x W latent grid are regrouped into such boxes.  Veda news (principles:
head-conditioned tile geometry) states the same.

Readings (the pages are silent on these):
  R1  token n of the input is (t, h, w) with n = (t*H + h)*W + w.
  R3  a grid dimension that the tile does not divide is padded up to whole
      tiles; slots that fall outside the grid are padding.
  R4  tiles are numbered row-major over (i_t, i_h, i_w) and the slots of a
      tile row-major over (dt, dh, dw).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Tuple

import numpy as np


def tile_grid(T: int, H: int, W: int, shape: Tuple[int, int, int]) -> Tuple[int, int, int]:
    """Number of tiles along t, h, w: ceil(T/pt), ceil(H/ph), ceil(W/pw)  (R3)."""
    pt, ph, pw = shape
    return (-(-T // pt), -(-H // ph), -(-W // pw))


def slot_tokens(T: int, H: int, W: int, shape: Tuple[int, int, int]) -> np.ndarray:
    """Token index held by every slot, or -1 for a padding slot.

    Slot u of tile j (global slot j*S + u) holds the token at
      t = i_t*pt + dt,  h = i_h*ph + dh,  w = i_w*pw + dw
    with j = (i_t*nH + i_h)*nW + i_w and u = (dt*ph + dh)*pw + dw  (R1, R3, R4).
    """
    pt, ph, pw = shape
    nT, nH, nW = tile_grid(T, H, W, shape)
    S = pt * ph * pw
    out = np.full(nT * nH * nW * S, -1, dtype=np.int64)
    for it in range(nT):
        for ih in range(nH):
            for iw in range(nW):
                j = (it * nH + ih) * nW + iw
                for dt in range(pt):
                    for dh in range(ph):
                        for dw in range(pw):
                            u = (dt * ph + dh) * pw + dw
                            t, h, w = it * pt + dt, ih * ph + dh, iw * pw + dw
                            if t < T and h < H and w < W:
                                out[j * S + u] = (t * H + h) * W + w
    return out


def valid_slots(T: int, H: int, W: int, shape: Tuple[int, int, int]) -> np.ndarray:
    """Boolean mask of the slots that hold a real token."""
    return slot_tokens(T, H, W, shape) >= 0


def gather(x: np.ndarray, T: int, H: int, W: int, shape) -> np.ndarray:
    """Tile order of one head's tokens: row j*S+u is x[token(j, u)], or a row
    of zeros for a padding slot.  ``x`` is [N][d] in token order."""
    perm = slot_tokens(T, H, W, shape)
    y = np.zeros((perm.size,) + x.shape[1:], dtype=np.float64)
    for s, n in enumerate(perm):
        if n >= 0:
            y[s] = x[n]
    return y


def scatter(y: np.ndarray, T: int, H: int, W: int, shape) -> np.ndarray:
    """Inverse of ``gather``: token order [N][d] from tile order, reading only
    the slots that hold a real token (padding rows are dropped)."""
    perm = slot_tokens(T, H, W, shape)
    x = np.zeros((T * H * W,) + y.shape[1:], dtype=np.float64)
    for s, n in enumerate(perm):
        if n >= 0:
            x[n] = y[s]
    return x


@dataclass
class HeadTiling:
    """Tiling of one head: grid, shape, tile count and slot map."""

    T: int
    H: int
    W: int
    shape: Tuple[int, int, int]

    def __post_init__(self):
        self.shape = tuple(int(s) for s in self.shape)
        self.S = self.shape[0] * self.shape[1] * self.shape[2]
        self.grid = tile_grid(self.T, self.H, self.W, self.shape)
        self.n = self.grid[0] * self.grid[1] * self.grid[2]
        self.perm = slot_tokens(self.T, self.H, self.W, self.shape)
        self.valid = self.perm >= 0

"""The max-pooled attention map that the tile-score estimator is distilled to.

Veda §2.1 (target construction): the reference map is the full attention
matrix max-pooled over query-tile x key-tile regions (max rather than mean,
so that isolated peaks survive).  Veda §2.3 (training efficiency): a
dedicated kernel builds this ground-truth heat map in two passes and only for
a random subset of query tiles.

Reading R16: the entries are probabilities of the full (unsparsified) softmax
over the real key tokens, maxed over the real (query, key) pairs of the
block; no renormalisation.  Pass 1 gives each query row's log-sum-exp over all
keys; pass 2 gives, per key tile, the largest exp(l_rc - lse_r).
"""
from __future__ import annotations

from typing import Iterable, Tuple

import numpy as np


def maxpool_map(qp: np.ndarray, kp: np.ndarray, valid: np.ndarray, S: int,
                q_tiles: Iterable[int], sm_scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Two-pass max-pooled map of one head for the query tiles ``q_tiles``.

    Returns (lse [len(q_tiles)*S] with NaN at padding query slots,
             M [len(q_tiles)][n]).
    """
    q = np.asarray(qp, np.float64)
    k = np.asarray(kp, np.float64)
    n = q.shape[0] // S
    q_tiles = list(q_tiles)
    lse_out = np.full(len(q_tiles) * S, np.nan)
    M = np.zeros((len(q_tiles), n))
    all_keys = np.flatnonzero(valid)
    for a, i in enumerate(q_tiles):
        rows = np.arange(i * S, (i + 1) * S)
        vrows = rows[valid[rows]]
        # pass 1: log-sum-exp of every valid query row over all valid keys
        logits = sm_scale * (q[vrows] @ k[all_keys].T)
        m = logits.max(axis=1)
        lse = m + np.log(np.exp(logits - m[:, None]).sum(axis=1))
        lse_out[a * S + (vrows - i * S)] = lse
        # pass 2: block maximum of the softmax probabilities, tile by tile
        for j in range(n):
            cols = np.arange(j * S, (j + 1) * S)
            cols = cols[valid[cols]]
            blk = sm_scale * (q[vrows] @ k[cols].T)
            M[a, j] = np.exp(blk - lse[:, None]).max()
    return lse_out, M


def maxpool_map_bruteforce(q_tokens: np.ndarray, k_tokens: np.ndarray, perm: np.ndarray,
                           S: int, q_tiles: Iterable[int], sm_scale: float) -> np.ndarray:
    """The same map by definition, for tiny inputs: materialise the full
    attention matrix A over the N real tokens (token order), then take the
    maximum of A over each (query tile, key tile) block of real tokens.
    ``perm`` maps slot -> token (-1 for padding)."""
    logits = sm_scale * (np.asarray(q_tokens, np.float64) @ np.asarray(k_tokens, np.float64).T)
    A = np.exp(logits - logits.max(axis=1, keepdims=True))
    A /= A.sum(axis=1, keepdims=True)
    n = perm.size // S
    q_tiles = list(q_tiles)
    out = np.zeros((len(q_tiles), n))
    for a, i in enumerate(q_tiles):
        qt = perm[i * S:(i + 1) * S]
        qt = qt[qt >= 0]
        for j in range(n):
            kt = perm[j * S:(j + 1) * S]
            kt = kt[kt >= 0]
            out[a, j] = A[np.ix_(qt, kt)].max()
    return out

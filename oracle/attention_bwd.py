"""Backward pass of the tile-skipping attention: dQ, dK, dV.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages train the sparse model (Veda §2.1 distillation with the sparse
path in place; Veda news: sparse attention during fine-tuning) but give no
backward kernel.  This is the derivative of ``attention.sparse_attention``
exactly as that function computes its output, written from the chain rule.
For query row r of tile i, with C the real key slots of the tiles its CSR row
lists (a tile listed twice contributes its keys twice, as in the forward):

    p_rc  = exp(sm_scale q_r.k_c - lse_r)           (the forward's softmax)
    dp_rc = do_r . v_c
    ds_rc = p_rc (dp_rc - sum_c' p_rc' dp_rc')       (softmax derivative)
    dq_r  = sm_scale sum_c ds_rc k_c
    dk_c += sm_scale ds_rc q_r,   dv_c += p_rc do_r  (summed over every row
                                                      and occurrence)

Reading:
  R28 the gradient is taken with respect to the tile-ordered Q, K, V of the
      real slots; rows of padding slots get zero gradient, and so does a query
      row whose CSR row keeps no key.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def sparse_attention_bwd(qp: np.ndarray, kp: np.ndarray, vp: np.ndarray, valid: np.ndarray,
                         S: int, row_ptr: np.ndarray, col_idx: np.ndarray, sm_scale: float,
                         dop: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of sum(o * dop) for one head, all in tile order [n*S][d]."""
    q = np.asarray(qp, np.float64)
    k = np.asarray(kp, np.float64)
    v = np.asarray(vp, np.float64)
    do = np.asarray(dop, np.float64)
    n = q.shape[0] // S
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for i in range(n):
        kept = [j for j in col_idx[row_ptr[i]:row_ptr[i + 1]] if 0 <= j < n]
        q_slots = np.arange(i * S, (i + 1) * S)
        q_slots = q_slots[valid[q_slots]]
        if not kept or q_slots.size == 0:
            continue
        key_slots = np.concatenate([np.arange(j * S, (j + 1) * S) for j in kept])
        key_slots = key_slots[valid[key_slots]]
        logits = sm_scale * (q[q_slots] @ k[key_slots].T)
        z = logits - logits.max(axis=1, keepdims=True)
        p = np.exp(z) / np.exp(z).sum(axis=1, keepdims=True)
        dp = do[q_slots] @ v[key_slots].T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        dq[q_slots] = sm_scale * ds @ k[key_slots]
        np.add.at(dk, key_slots, sm_scale * ds.T @ q[q_slots])
        np.add.at(dv, key_slots, p.T @ do[q_slots])
    return dq, dk, dv

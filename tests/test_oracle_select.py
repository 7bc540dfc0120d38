"""Pins for the oracle's keep count and top-k -> CSR.

Pinned against: hand values of the integer keep count (including the case
where a float ceil would be off by one), a brute-force rank count written with
Python's own float comparisons, and hand-worked rows with ties, signed zeros
and NaN.
"""
import math

import numpy as np
import pytest

import oracle
from workloads import random_scores


@pytest.mark.parametrize("n,s,k", [
    (720, 95, 36),     # 720*0.05 in floating point ceils to 37; integer arithmetic gives 36
    (4, 50, 2), (4, 0, 4), (336, 90, 34), (336, 95, 17), (1920, 95, 96), (1830, 95, 92),
    (630, 95, 32), (1, 100, 1), (10, 100, 1), (7, 99, 1),
])
def test_keep_count(n, s, k):
    assert oracle.keep_count(n, s) == k


def test_keep_count_float_form_differs_at_720():
    assert math.ceil(720 * (1 - 0.95)) == 37      # the trap the integer form avoids


def _brute_force(row, k):
    """Selected set by counting, for each element, how many others beat it."""
    def better(a, b):   # does a beat b?  (value desc, NaN lowest, index asc)
        va, vb = float(row[a]), float(row[b])
        if math.isnan(va) or math.isnan(vb):
            if math.isnan(va) and math.isnan(vb):
                return a < b
            return not math.isnan(va)
        if va != vb:
            return va > vb
        return a < b
    n = len(row)
    return sorted(j for j in range(n) if sum(better(o, j) for o in range(n) if o != j) < k)


@pytest.mark.parametrize("ties", [False, True])
@pytest.mark.parametrize("k", [1, 3, 17, 40])
def test_topk_matches_brute_force(ties, k):
    s = random_scores(6, 40, seed=11 + k, ties=ties)
    if ties:
        s[0, 5] = np.nan
        s[1, ::3] = np.nan
    rp, ci = oracle.select_topk(s, k)
    assert rp.tolist() == [i * k for i in range(7)]
    for i in range(6):
        assert ci[i * k:(i + 1) * k].tolist() == _brute_force(s[i], k)


def test_hand_worked_rows():
    row = np.array([[0.5, 0.7, 0.7, 0.1, np.nan, 0.7]], dtype=np.float32)
    assert oracle.select_topk(row, 3)[1].tolist() == [1, 2, 5]
    assert oracle.select_topk(row, 4)[1].tolist() == [0, 1, 2, 5]
    assert oracle.select_topk(row, 5)[1].tolist() == [0, 1, 2, 3, 5]
    assert oracle.select_topk(row, 6)[1].tolist() == [0, 1, 2, 3, 4, 5]
    z = np.array([[-0.0, 0.0, -1.0]], dtype=np.float32)
    assert oracle.select_topk(z, 1)[1].tolist() == [0]          # -0.0 ties +0.0 -> lower index
    z2 = np.array([[0.0, -0.0, -1.0]], dtype=np.float32)
    assert oracle.select_topk(z2, 1)[1].tolist() == [0]
    nn = np.array([[np.nan, np.nan, -np.inf]], dtype=np.float32)
    assert oracle.select_topk(nn, 1)[1].tolist() == [2]          # -inf beats NaN
    assert oracle.select_topk(nn, 2)[1].tolist() == [0, 2]


def test_special_cases():
    eq = np.ones((3, 9), dtype=np.float32)
    assert oracle.select_topk(eq, 4)[1].tolist() == [0, 1, 2, 3] * 3
    s = random_scores(4, 9, seed=5)
    assert oracle.select_topk(s, 9)[1].tolist() == list(range(9)) * 4
    ci = oracle.select_topk(s, 1)[1]
    assert ci.tolist() == np.argmax(s, axis=1).tolist()

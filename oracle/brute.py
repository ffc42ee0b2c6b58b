"""Brute-force top-k by rank counting, O(N^2). TEST INFRASTRUCTURE ONLY.

Independent of the sorting oracle: instead of sorting, every element counts how many
elements of the row rank strictly before it; an element is selected when fewer than k
do, and the selected elements are output in order of that count.

The order is expressed as a Python tuple key (value, copysign(1, value), -index),
compared lexicographically and taken descending: larger value first; between +0 and -0
(equal as numbers) the positive zero first; then the smaller index first.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np


def _key(v: float, j: int) -> Tuple[float, float, int]:
    return (v, math.copysign(1.0, v), -j)


def brute_topk(values: Sequence[float], k: int) -> List[int]:
    """Indices of the top-k of one row, in output order."""
    n = len(values)
    if not 1 <= k <= n:
        raise ValueError("need 1 <= k <= n")
    keys = [_key(float(v), j) for j, v in enumerate(values)]
    ahead = [sum(1 for kb in keys if kb > ka) for ka in keys]
    chosen = [j for j in range(n) if ahead[j] < k]
    chosen.sort(key=lambda j: ahead[j])
    return chosen


def brute_order_batch(values: np.ndarray) -> np.ndarray:
    """The same rank counting for a batch of short rows at once (values [R, n], float64, no
    NaN): element i of a row is preceded by element j when (v_j, sign_j, -j) > (v_i, sign_i,
    -i) lexicographically, with sign = copysign(1, v). Returns [R, n] int64: column t holds
    the index of the element with t elements ahead of it, so the first k columns are the
    top-k in output order."""
    v = np.asarray(values, np.float64)
    R, n = v.shape
    sgn = np.copysign(1.0, v)
    j = np.arange(n)
    vj, vi = v[:, :, None], v[:, None, :]  # [R, j, i]
    sj, si = sgn[:, :, None], sgn[:, None, :]
    ahead_of = (vj > vi) | ((vj == vi) & ((sj > si) | ((sj == si) & (j[:, None] < j[None, :]))))
    ahead = ahead_of.sum(axis=1)  # [R, i]: how many elements precede element i
    order = np.full((R, n), -1, np.int64)
    rr = np.repeat(np.arange(R), n)
    order[rr, ahead.reshape(-1)] = np.tile(j, R)
    if (order < 0).any():
        raise AssertionError("rank counts are not a permutation")
    return order

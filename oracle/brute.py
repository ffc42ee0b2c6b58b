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

"""Adaptive k: how many keys carry a given share of a group's estimated attention mass.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages: DSV summaries, zh §2.1 stage two, "critical KV estimation" (pt §2A, fr §2A, ko §2가):
the trained low-rank predictors estimate QK^T quickly and identify the critical KV pairs,
those that contribute more than 90 % of the attention score.
Readings (the pages give no formula):
  * a group's estimated logits are logit_scale * sigma[g][m], sigma the group score of the
    top-k estimator (SUM over members); logit_scale = scale / G is the mean member logit;
  * the attention mass of key m is its softmax weight over all S keys of the row;
  * a group's k is the smallest number of keys whose weights, largest first, reach `mass`
    of the row's total weight (the "critical" keys carry that share of the score);
  * the head's k is the largest k of its groups over the batch.

Everything is float64. The weights are exp(logit_scale * (sigma - max sigma)) (the common
factor exp(-max) cancels), the total and the prefix sums are exactly rounded (math.fsum).
`k_bracket` widens the decision by an absolute band on the prefix sums: it returns every k
that a computation of the same rule whose sums are within `band` of these would return.
"""
from __future__ import annotations

import math
from typing import Tuple

import numpy as np


def softmax_weights(sigma_row: np.ndarray, logit_scale: float) -> np.ndarray:
    """exp(logit_scale * (sigma_m - max sigma)) for every key of the row (fp64, max weight 1)."""
    s = np.asarray(sigma_row, dtype=np.float64)
    return np.exp(float(logit_scale) * (s - s.max()))


def _sorted_desc(w: np.ndarray) -> np.ndarray:
    return np.sort(w)[::-1]


def _first_reaching(wd: np.ndarray, target: float) -> int:
    """Smallest n >= 1 with fsum(wd[:n]) >= target (wd descending; len(wd) if none)."""
    S = wd.shape[0]
    c = np.cumsum(wd)                        # an estimate; corrected with exact sums below
    n = min(int(np.searchsorted(c, target)) + 1, S)
    pre = lambda j: math.fsum(wd[:j])       # noqa: E731 — exactly rounded prefix sum
    while n > 1 and pre(n - 1) >= target:
        n -= 1
    while n < S and pre(n) < target:
        n += 1
    return n


def exact_k(sigma_row: np.ndarray, logit_scale: float, mass: float) -> int:
    """Smallest number of keys whose softmax weights (largest first) reach `mass` of the
    row's total weight."""
    w = softmax_weights(sigma_row, logit_scale)
    wd = _sorted_desc(w)
    return _first_reaching(wd, mass * math.fsum(w))


def k_bracket(sigma_row: np.ndarray, logit_scale: float, mass: float,
              band: float) -> Tuple[int, int]:
    """(k_lo, k_hi): the smallest counts whose prefix sums reach mass * total - band and
    mass * total + band. exact_k lies in between, and so does the k of any evaluation of the
    rule whose prefix sums and target are each within band / 2 of the exact ones."""
    return k_with_bracket(sigma_row, logit_scale, mass, band)[1:]


def k_with_bracket(sigma_row: np.ndarray, logit_scale: float, mass: float,
                   band: float) -> Tuple[int, int, int]:
    """(exact_k, k_lo, k_hi) from one sort of the row's weights."""
    w = softmax_weights(sigma_row, logit_scale)
    wd = _sorted_desc(w)
    target = mass * math.fsum(w)
    return (_first_reaching(wd, target), _first_reaching(wd, target - band),
            _first_reaching(wd, target + band))

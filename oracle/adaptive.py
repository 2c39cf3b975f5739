"""Adaptive k: how many keys carry a given share of a group's estimated attention mass.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages: DSV summaries, zh §2.1 stage two, "critical KV estimation" (pt §2A, fr §2A, ko §2가):
the trained low-rank predictors estimate QK^T quickly and identify the critical KV pairs,
those that contribute more than 90 % of the attention score.
Readings (the pages give no formula):
  * a group's estimated logits are logit_scale * sigma[g][m], sigma the group score of the
    top-k estimator (SUM over members); logit_scale = scale / G is the mean member logit;
  * the mass of a key is its softmax weight; k is found from a histogram of the logits below
    the group maximum (bins of 1/4 logit unit, 128 bins, the last one open-ended), each key of
    bin b weighted exp(-(b + 1/2)/4) (the last bin exp(-127/4)), accumulated in bin order;
  * the head's k is the largest k of its groups over the batch.
The histogram is the exact object; only the weights are binned. `exact_k` (a full sort of the
true softmax weights) pins it within the bin width.
"""
from __future__ import annotations

import math
from typing import List, Sequence

import numpy as np

BINS = 128
PER_NAT = 4


def bin_weights() -> List[float]:
    w = [math.exp(-(b + 0.5) / PER_NAT) for b in range(BINS - 1)]
    w.append(math.exp(-(BINS - 1) / PER_NAT))
    return w


def group_bin_counts(sigma_row: np.ndarray, logit_scale: float) -> np.ndarray:
    """Histogram of a group's keys over the logit gap below the maximum. The gap and its
    product with 4 * logit_scale are taken in fp32, as the kernel does."""
    s = np.asarray(sigma_row, dtype=np.float32)
    M = s.max()
    tau_r = np.float32(logit_scale) * np.float32(PER_NAT)
    x = (M - s) * tau_r                      # fp32 subtract, then fp32 multiply
    b = np.where(x < np.float32(BINS - 1), np.floor(x), BINS - 1).astype(np.int64)
    return np.bincount(b, minlength=BINS)


def k_from_counts(counts: Sequence[int], mass: float, w: Sequence[float]) -> int:
    """Running softmax mass in bin order (fp64, one operation at a time)."""
    z = 0.0
    for c, wb in zip(counts, w):
        z = z + float(c) * wb
    target = mass * z
    cum, n = 0.0, 0
    for c, wb in zip(counts, w):
        nxt = cum + float(c) * wb
        if c != 0 and nxt >= target:
            need = math.ceil((target - cum) / wb)
            return max(n + min(need, int(c)), 1)
        cum, n = nxt, n + int(c)
    return max(n, 1)


def group_k(sigma_row: np.ndarray, logit_scale: float, mass: float) -> int:
    return k_from_counts(group_bin_counts(sigma_row, logit_scale), mass, bin_weights())


def exact_k(sigma_row: np.ndarray, logit_scale: float, mass: float) -> int:
    """Smallest number of keys whose true softmax weights (largest first) reach `mass` of the
    total, by a full sort in fp64."""
    s = np.asarray(sigma_row, dtype=np.float64) * logit_scale
    p = np.exp(s - s.max())
    p = np.sort(p)[::-1]
    c = np.cumsum(p)
    return int(np.searchsorted(c, mass * c[-1] * (1 - 1e-15)) + 1)

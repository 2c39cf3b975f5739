"""Pins for the oracle's adaptive k (CPU only): a hand-worked case, closed forms, and the
exact sort-based rule within the bin width."""
import math

import numpy as np
import pytest

from oracle import adaptive, geometry, topk


def test_hand_worked_example():
    # scores 10, 10, 9, 0 at logit scale 1: gaps 0, 0, 1, 10 -> bins 0, 0, 4, 40
    s = np.array([10.0, 10.0, 9.0, 0.0])
    counts = adaptive.group_bin_counts(s, 1.0)
    assert counts[0] == 2 and counts[4] == 1 and counts[40] == 1 and counts.sum() == 4
    # masses 2 e^-1/8 = 1.765, e^-9/8 = 0.325, e^-81/8 = 4e-5; 90 % of 2.090 needs one key of
    # bin 4: k = 3 (the true weights agree: the top two carry 84.5 %)
    assert adaptive.group_k(s, 1.0, 0.9) == 3
    assert adaptive.exact_k(s, 1.0, 0.9) == 3
    assert adaptive.group_k(s, 1.0, 0.8) == 2


def test_constant_scores_need_ceil_mass_times_S():
    s = np.zeros(1000)
    assert adaptive.group_k(s, 0.3, 0.9003) == 901
    assert adaptive.group_k(s, 0.3, 0.0004) == 1
    assert adaptive.group_k(s, 0.3, 1.0) == 1000


def test_two_levels_far_apart():
    # 37 keys at the maximum, 963 keys 1000 logit units lower (open last bin, weight e^-31.75)
    s = np.concatenate([np.full(37, 500.0), np.full(963, -500.0)])
    lo = 963 * math.exp(-127 / 4) / math.exp(-0.125)
    assert adaptive.group_k(s, 1.0, 0.9) == math.ceil(0.9 * (37 + lo))
    assert adaptive.group_k(s, 1.0, 1.0) == 1000


def test_weights_and_bins():
    w = adaptive.bin_weights()
    assert len(w) == 128 and w[0] == math.exp(-0.125) and w[-1] == math.exp(-31.75)
    assert all(a > b for a, b in zip(w, w[1:]))
    # a gap just below a bin edge stays in the lower bin (fp32 gap times fp32 4*scale)
    s = np.array([0.0, -0.2499], dtype=np.float32)
    assert adaptive.group_bin_counts(s, 1.0)[0] == 2
    s = np.array([0.0, -0.25], dtype=np.float32)
    assert adaptive.group_bin_counts(s, 1.0)[1] == 1


@pytest.mark.parametrize("seed", range(12))
def test_within_bin_width_of_the_exact_rule(seed):
    rng = np.random.default_rng(seed)
    S, G, r = 1024, 16, 16
    q = rng.integers(-7, 8, size=(S, r)).astype(np.float64)
    k = rng.integers(-7, 8, size=(S, r)).astype(np.float64)
    mem = geometry.group_members(4, 16, 16, 2, 2, 4)
    sigma = topk.group_scores_bruteforce(q, k, mem)
    scale = rng.choice([1.0 / (8 * G), 1.0 / G, 4.0 / G])
    for mass in (0.5, 0.9, 0.99):
        for g in range(0, sigma.shape[0], 7):
            kb = adaptive.group_k(sigma[g], scale, mass)
            lo = adaptive.exact_k(sigma[g], scale, mass * math.exp(-0.25))
            hi = adaptive.exact_k(sigma[g], scale, min(1.0, mass * math.exp(0.25)))
            assert lo <= kb <= hi, (g, mass, lo, kb, hi)


def test_monotone_in_mass():
    rng = np.random.default_rng(5)
    s = rng.normal(0, 40, size=4096).round()
    ks = [adaptive.group_k(s, 0.05, m) for m in (0.1, 0.3, 0.5, 0.7, 0.9, 0.99, 1.0)]
    assert ks == sorted(ks) and ks[-1] == 4096

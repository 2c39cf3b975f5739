"""Pins for the oracle's adaptive k (CPU only): a hand-worked case, brute force over key
subsets, closed forms of constant, two-level and geometric score rows, and the bracket."""
import itertools
import math

import numpy as np
import pytest

from oracle import adaptive, geometry, topk


def test_hand_worked_example():
    # scores 10, 10, 9, 0 at logit scale 1: weights 1, 1, e^-1, e^-10, total 2.367925...
    s = np.array([10.0, 10.0, 9.0, 0.0])
    # 90 %: 2.13113 > 2 (two keys), <= 2.36788 (three keys)
    assert adaptive.exact_k(s, 1.0, 0.9) == 3
    # 80 %: 1.89434 <= 2
    assert adaptive.exact_k(s, 1.0, 0.8) == 2
    # the two top keys carry 84.46 %: 0.844 needs two keys, 0.845 three
    assert adaptive.exact_k(s, 1.0, 0.844) == 2
    assert adaptive.exact_k(s, 1.0, 0.845) == 3
    # all four keys are needed beyond (2 + e^-1) / total = 99.998 %
    assert adaptive.exact_k(s, 1.0, 0.99999) == 4
    assert adaptive.exact_k(s, 1.0, 0.0001) == 1


def _brute_force_k(w, mass):
    """Smallest |A| over all key subsets A whose weights reach mass * total."""
    tot = math.fsum(w)
    for n in range(1, len(w) + 1):
        for sub in itertools.combinations(range(len(w)), n):
            if math.fsum(w[i] for i in sub) >= mass * tot:
                return n
    return len(w)


@pytest.mark.parametrize("seed", range(8))
def test_brute_force_over_subsets(seed):
    rng = np.random.default_rng(seed)
    s = rng.integers(-6, 7, size=10).astype(np.float64)   # many ties
    for ls in (0.1, 0.7, 2.0):
        w = list(np.exp(ls * (s - s.max())))
        for mass in (0.2, 0.5, 0.75, 0.9, 0.99):
            assert adaptive.exact_k(s, ls, mass) == _brute_force_k(w, mass), (ls, mass)


def test_constant_scores_need_ceil_mass_times_S():
    s = np.zeros(1000)
    assert adaptive.exact_k(s, 0.3, 0.9003) == 901
    assert adaptive.exact_k(s, 0.3, 0.0004) == 1
    assert adaptive.exact_k(s, 0.3, 1.0) == 1000


def test_two_levels():
    # 37 keys at the maximum, 963 keys 2 logit units lower: total 37 + 963 e^-2
    s = np.concatenate([np.full(37, 500.0), np.full(963, 498.0)])
    low = math.exp(-2.0)
    tot = 37 + 963 * low
    for mass in (0.2, 0.5, 0.9):
        if mass * tot <= 37:
            want = math.ceil(mass * tot)
        else:
            want = 37 + math.ceil((mass * tot - 37) / low)
        assert adaptive.exact_k(s, 1.0, mass) == want
    assert adaptive.exact_k(s, 1.0, 1.0) == 1000


@pytest.mark.parametrize("lam", [0.01, 0.05, 0.3])
def test_geometric_weights_closed_form(lam):
    # sigma_m = -m: weights e^{-lam m}; the top n carry (1 - e^{-lam n}) / (1 - e^{-lam S}),
    # so k = ceil(-ln(1 - mass (1 - e^{-lam S})) / lam)
    S = 4000
    s = -np.arange(S, dtype=np.float64)
    for mass in (0.3, 0.6, 0.9, 0.97):
        x = -math.log1p(-mass * -math.expm1(-lam * S)) / lam
        if abs(x - round(x)) < 1e-6:
            continue   # on a boundary: rounding decides, nothing to pin
        assert adaptive.exact_k(s, lam, mass) == math.ceil(x), (lam, mass, x)


def test_order_of_keys_does_not_matter():
    rng = np.random.default_rng(3)
    s = rng.normal(0, 40, size=2048).round()
    k0 = adaptive.exact_k(s, 0.05, 0.9)
    for _ in range(3):
        assert adaptive.exact_k(rng.permutation(s), 0.05, 0.9) == k0


def test_monotone_in_mass():
    rng = np.random.default_rng(5)
    s = rng.normal(0, 40, size=4096).round()
    ks = [adaptive.exact_k(s, 0.05, m) for m in (0.1, 0.3, 0.5, 0.7, 0.9, 0.99, 1.0)]
    assert ks == sorted(ks) and ks[-1] == 4096


@pytest.mark.parametrize("seed", range(6))
def test_bracket_holds_the_exact_rule(seed):
    rng = np.random.default_rng(seed)
    S, G, r = 1024, 16, 16
    q = rng.integers(-7, 8, size=(S, r)).astype(np.float64)
    k = rng.integers(-7, 8, size=(S, r)).astype(np.float64)
    mem = geometry.group_members(4, 16, 16, 2, 2, 4)
    sigma = topk.group_scores_bruteforce(q, k, mem)
    ls = [1.0 / (8 * G), 1.0 / G, 4.0 / G][seed % 3]
    for g in range(0, sigma.shape[0], 5):
        for mass in (0.5, 0.9):
            ke = adaptive.exact_k(sigma[g], ls, mass)
            assert adaptive.k_bracket(sigma[g], ls, mass, 0.0) == (ke, ke)
            lo, hi = adaptive.k_bracket(sigma[g], ls, mass, 1e-9)
            assert lo <= ke <= hi
            # a band wider than the whole row's weight admits every count
            assert adaptive.k_bracket(sigma[g], ls, mass, 1e9) == (1, S)

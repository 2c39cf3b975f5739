"""Pins for the oracle's head placement and dense-versus-sparse choice (CPU only).

The placement is checked against brute-force optimal placements (Graham's bound for the
longest-processing-time greedy), a known tight instance, and closed forms of the imbalance
ratio; the dispatch rule against its closed-form break-even k."""
import itertools
import random

import pytest

from oracle import planning


def test_lpt_tight_instance():
    # Graham's tight case for two devices: 3, 3, 2, 2, 2 -> greedy 7, optimum 6 (= 4/3 - 1/6)
    part, load = planning.lpt([3, 3, 2, 2, 2], 2)
    assert sorted(load) == [5.0, 7.0]
    assert planning.optimal_makespan([3, 3, 2, 2, 2], 2) == 6.0
    assert part == [0, 1, 0, 1, 0]


@pytest.mark.parametrize("seed", range(40))
def test_lpt_within_graham_bound_of_brute_force(seed):
    rng = random.Random(seed)
    n = rng.randint(1, 7)
    m = rng.randint(1, 3)
    costs = [float(rng.randint(1, 20)) for _ in range(n)]
    part, load = planning.lpt(costs, m)
    # every head placed once; loads are the sums of their heads
    for q in range(m):
        assert load[q] == sum(c for c, p in zip(costs, part) if p == q)
    opt = planning.optimal_makespan(costs, m)
    assert max(load) <= (4.0 / 3.0 - 1.0 / (3.0 * m)) * opt + 1e-12
    assert max(load) >= opt
    # largest-first: no device ends more than the smallest head above the least loaded one
    assert max(load) - min(load) <= max(costs) + 1e-12


def test_rho_closed_forms():
    part, load = planning.lpt([5.0] * 24, 8)
    assert load == [15.0] * 8 and planning.rho_s(load) == 1.0
    part, load = planning.lpt([1.0, 2.0, 3.0], 1)
    assert part == [0, 0, 0] and planning.rho_s(load) == 1.0
    # one huge head among small ones: rho = H * max / total for n_parts = H
    costs = [10.0, 1.0, 1.0, 1.0]
    _, load = planning.lpt(costs, 4)
    assert planning.rho_s(load) == pytest.approx(10.0 / (13.0 / 4.0))


def test_head_costs_and_ties():
    assert planning.head_costs([1, 2], 0.5, 2.0) == [2.5, 4.5]
    # equal costs: lower head first onto lower device
    part, _ = planning.lpt([1.0, 1.0, 1.0, 1.0], 2)
    assert part == [0, 1, 0, 1]


def test_dispatch_break_even_closed_form():
    S, cs, ce = 1000, 0.01, 1.0          # break-even k* = S (1 - cs/ce) = 990
    ks = [1, 500, 989, 990, 991, 1000]
    out, nd = planning.dispatch_k(ks, S, cs, ce)
    assert out == [1, 500, 989, 1000, 1000, 1000]
    assert nd == 3
    # free estimation: only k = S is dense; estimation dearer than attention: all dense
    assert planning.dispatch_k([999, 1000], S, 0.0, 1.0) == ([999, 1000], 1)
    assert planning.dispatch_k([1, 2], S, 2.0, 1.0) == ([1000, 1000], 2)

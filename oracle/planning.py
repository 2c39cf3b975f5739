"""Head placement and the dense-versus-sparse choice, as plain Python.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages:
  * DSV summaries, zh §2.3 "Head-wise CP Re-balancing" (pt §2C, fr §2C, ko §2다): the heads
    are placed on devices according to their sparsity so that the compute load balances.
  * db-SP summary, "核心方法" (core method): a head-level greedy partition balances the load
    per device; "关键观察" (key observations): the sparse imbalance ratio is the largest device
    load over the mean device load.
  * DSV summaries, zh §2.1 stage two (pt §2A, fr §2A, ko §2가): the OP Dispatcher decides,
    from the current sparsity, whether sparse attention runs.
Readings (the pages give no formulas):
  * cost of a head = fixed + per_k * k_h (the estimator's fixed cost per head plus the
    attention's cost per unit of k);
  * the greedy is longest-processing-time first: heads by decreasing cost (equal costs: lower
    head index first), each onto the least-loaded device (equal loads: lower device index);
  * a head runs dense (k_h := S, no estimation) when dense attention is not dearer than the
    estimator plus sparse attention.
"""
from __future__ import annotations

import itertools
from typing import List, Sequence, Tuple


def head_costs(k_per_head: Sequence[int], fixed: float, per_k: float) -> List[float]:
    return [fixed + per_k * float(k) for k in k_per_head]


def lpt_order(costs: Sequence[float]) -> List[int]:
    """The greedy's processing order: heads by decreasing cost, equal costs by lower index."""
    return sorted(range(len(costs)), key=lambda h: (-costs[h], h))


def lpt(costs: Sequence[float], n_parts: int) -> Tuple[List[int], List[float]]:
    """Longest-processing-time greedy: (device of each head, load of each device)."""
    order = lpt_order(costs)
    load = [0.0] * n_parts
    part = [0] * len(costs)
    for h in order:
        best = min(range(n_parts), key=lambda q: (load[q], q))
        part[h] = best
        load[best] += costs[h]
    return part, load


def rho_s(loads: Sequence[float]) -> float:
    """Sparse imbalance ratio: largest load over mean load."""
    return max(loads) / (sum(loads) / len(loads))


def optimal_makespan(costs: Sequence[float], n_parts: int) -> float:
    """Smallest possible largest load, by trying every placement (tiny inputs only)."""
    best = float("inf")
    for assign in itertools.product(range(n_parts), repeat=len(costs)):
        load = [0.0] * n_parts
        for h, q in enumerate(assign):
            load[q] += costs[h]
        best = min(best, max(load))
    return best


def dispatch_k(k_per_head: Sequence[int], S: int, topk_ns_per_score: float,
               attn_ns_per_edge: float) -> Tuple[List[int], int]:
    """Per head: S if dense attention (S edges per group) costs no more than estimation
    (S scores per group) plus sparse attention (k_h edges per group), else k_h."""
    out = []
    for k in k_per_head:
        sparse = S * topk_ns_per_score + k * attn_ns_per_edge
        dense = S * attn_ns_per_edge
        out.append(S if dense <= sparse else int(k))
    return out, sum(1 for o in out if o == S)

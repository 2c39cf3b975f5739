"""Pins for the oracle's geometry and critical-KV top-k (CPU only).

Each test checks the oracle against something other than itself: a hand-worked fixture,
brute force over all subsets, library routines, closed forms or invariants."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import geometry, topk

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- geometry
@pytest.mark.parametrize("grid,grp", [((4, 16, 16), (2, 2, 4)), ((2, 4, 6), (1, 2, 3)),
                                      ((4, 8, 8), (4, 4, 4)), ((1, 2, 4), (1, 2, 2))])
def test_groups_partition_grid_into_boxes(grid, grp):
    T, Hh, W = grid
    gt, gh, gw = grp
    mem = geometry.group_members(T, Hh, W, gt, gh, gw)
    S = T * Hh * W
    assert mem.shape == (S // (gt * gh * gw), gt * gh * gw)
    # partition
    assert np.array_equal(np.sort(mem.reshape(-1)), np.arange(S))
    # each group is a gt x gh x gw box, members listed row-major over (dt, dy, dx)
    t, rem = np.divmod(mem, Hh * W)
    y, x = np.divmod(rem, W)
    for g in range(mem.shape[0]):
        assert t[g].max() - t[g].min() == gt - 1
        assert y[g].max() - y[g].min() == gh - 1
        assert x[g].max() - x[g].min() == gw - 1
        assert t[g].min() % gt == 0 and y[g].min() % gh == 0 and x[g].min() % gw == 0
        assert np.all(np.diff(mem[g]) > 0)   # row-major member order on a row-major grid
    # boxes numbered row-major by their corner
    corners = list(zip(t.min(1), y.min(1), x.min(1)))
    assert corners == sorted(corners)


def test_groups_reject_non_dividing_extents():
    with pytest.raises(ValueError):
        geometry.group_members(4, 6, 6, 2, 4, 2)


# ---------------------------------------------------------------- hand-worked fixture
def test_toy_fixture_scores_and_rows():
    fx = json.load(open(os.path.join(GOLD, "toy_topk.json")))
    T, Hh, W = fx["grid"]
    mem = geometry.group_members(T, Hh, W, *fx["group"])
    q = np.array(fx["q_lr"], float)
    k = np.array(fx["k_lr"], float)
    sigma = topk.group_scores_bruteforce(q, k, mem)
    assert np.array_equal(sigma, np.array(fx["sigma"], float))
    for kk, rows in fx["rows"].items():
        got = topk.topk_rows_by_sort(sigma, int(kk))
        assert np.array_equal(got, np.array(rows))
    # the packed entry point on a [1,1,S,r] view gives the same rows
    packed = topk.lowrank_topk(q[None, None], k[None, None], [3], mem)
    assert np.array_equal(packed.reshape(2, 3), np.array(fx["rows"]["3"]))


# ---------------------------------------------------------------- group scores
def test_group_scores_bruteforce_matches_python_loops_and_sum_first():
    rng = np.random.default_rng(1)
    T, Hh, W, r = 2, 4, 4, 3
    mem = geometry.group_members(T, Hh, W, 1, 2, 2)
    S = T * Hh * W
    q = rng.integers(-7, 8, size=(S, r))
    k = rng.integers(-7, 8, size=(S, r))
    sig = topk.group_scores_bruteforce(q, k, mem)
    # plain Python int loops, no numpy arithmetic
    ql, kl = q.tolist(), k.tolist()
    for g in range(mem.shape[0]):
        for m in range(S):
            ref = sum(sum(ql[n][c] * kl[m][c] for c in range(r)) for n in mem[g].tolist())
            assert sig[g, m] == ref
    assert np.array_equal(sig, topk.group_scores_sum_first(q, k, mem))


def test_group_scores_exact_at_config_bound():
    """|sigma| <= G*r*49 for factors in [-7,7]: the extreme case is reproduced exactly."""
    mem = geometry.group_members(4, 4, 4, 4, 4, 4)   # one group of 64
    S, r = 64, 32
    q = np.full((S, r), 7.0)
    k = np.full((S, r), -7.0)
    sig = topk.group_scores_bruteforce(q, k, mem)
    assert np.all(sig == -64 * 32 * 49)
    assert 64 * 32 * 49 < 2 ** 24


# ---------------------------------------------------------------- top-k
def _brute_force_row(scores, k):
    """Among all k-subsets whose every member scores >= every non-member, the one that
    prefers lower indices (lexicographically smallest sorted tuple)."""
    n = len(scores)
    best = None
    for sub in itertools.combinations(range(n), k):
        inside = [scores[i] for i in sub]
        outside = [scores[i] for i in range(n) if i not in sub]
        if outside and min(inside) < max(outside):
            continue
        if best is None or sub < best:
            best = sub
    return np.array(best)


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_subset_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    scores = rng.integers(-3, 4, size=(3, 12)).astype(float)   # heavy ties
    for k in (1, 3, 6, 11, 12):
        rows = topk.topk_rows_by_sort(scores, k)
        for g in range(3):
            assert np.array_equal(rows[g], _brute_force_row(scores[g].tolist(), k))


def test_topk_special_cases():
    rng = np.random.default_rng(7)
    sig = rng.integers(-5, 6, size=(4, 40)).astype(float)
    full = topk.topk_rows_by_sort(sig, 40)
    assert np.array_equal(full, np.tile(np.arange(40), (4, 1)))
    one = topk.topk_rows_by_sort(sig, 1)
    assert np.array_equal(one[:, 0], np.argmax(sig, axis=1))   # first maximum = lowest index
    const = topk.topk_rows_by_sort(np.zeros((2, 10)), 4)
    assert np.array_equal(const, np.tile(np.arange(4), (2, 1)))
    with pytest.raises(ValueError):
        topk.topk_rows_by_sort(sig, 0)
    with pytest.raises(ValueError):
        topk.topk_rows_by_sort(sig, 41)


@pytest.mark.parametrize("seed", range(4))
def test_characterisation_agrees_with_sort_and_rejects_mistakes(seed):
    rng = np.random.default_rng(100 + seed)
    S = 300
    sig = rng.integers(-20, 21, size=(5, S)).astype(float)
    for k in (1, 17, 150, 299, 300):
        rows = topk.topk_rows_by_sort(sig, k)
        for g in range(5):
            assert topk.topk_row_is_exact(sig[g], rows[g], k)
    k = 40
    rows = topk.topk_rows_by_sort(sig, k)
    for g in range(5):
        row = rows[g]
        T = sig[g, row].min()
        ties_out = [m for m in np.flatnonzero(sig[g] == T) if m not in set(row)]
        if ties_out:   # swap the last selected tie for a later, unselected tie
            sel_ties = [m for m in row if sig[g, m] == T]
            bad = np.sort(np.array([m for m in row if m != sel_ties[-1]] + [ties_out[-1]]))
            assert not topk.topk_row_is_exact(sig[g], bad, k)
        lower = [m for m in np.flatnonzero(sig[g] < T)]
        if lower:      # replace a selected key by a strictly lower-scoring one
            bad = np.sort(np.concatenate([row[1:], [lower[0]]]))
            if len(set(bad.tolist())) == k:
                assert not topk.topk_row_is_exact(sig[g], bad, k)
        assert not topk.topk_row_is_exact(sig[g], row[::-1], k)       # not ascending
        assert not topk.topk_row_is_exact(sig[g], row[:-1], k)        # too short


@pytest.mark.parametrize("seed", range(4))
def test_batched_characterisation_equals_the_row_check(seed):
    """topk_rows_are_exact (all rows at once) gives the per-row check's verdict on the sort's
    answer and on planted mistakes: a tie swapped for a later tie, a lower-scoring key, a
    duplicate, a key out of range, a descending row, a row of the wrong length."""
    rng = np.random.default_rng(200 + seed)
    S, NG = 257, 12
    sig = rng.integers(-9, 10, size=(NG, S)).astype(np.int64)
    for k in (1, 13, 128, 256, 257):
        rows = topk.topk_rows_by_sort(sig.astype(float), k)
        assert topk.topk_rows_are_exact(sig, rows, k).all()
        assert topk.topk_rows_are_exact(sig.astype(float), rows, k).all()
    k = 50
    rows = topk.topk_rows_by_sort(sig.astype(float), k)
    planted = []
    for g in range(NG):
        row = rows[g].copy()
        T = sig[g, row].min()
        kind = g % 6
        if kind == 0:
            ties_out = [m for m in np.flatnonzero(sig[g] == T) if m not in set(row)]
            sel_ties = [m for m in row if sig[g, m] == T]
            if not ties_out:
                planted.append(row)
                continue
            row = np.sort(np.array([m for m in row if m != sel_ties[-1]] + [ties_out[-1]]))
        elif kind == 1:
            lower = np.flatnonzero(sig[g] < T)
            row = np.sort(np.concatenate([row[1:], lower[:1]]))
        elif kind == 2:
            row[5] = row[4]                       # duplicate
        elif kind == 3:
            row[-1] = S                           # out of range
        elif kind == 4:
            row = row[::-1].copy()                # descending
        else:
            pass                                  # the correct row
        planted.append(row)
    planted = np.stack(planted)
    want = np.array([topk.topk_row_is_exact(sig[g].astype(float), planted[g], k)
                     for g in range(NG)])
    got = topk.topk_rows_are_exact(sig, planted, k)
    assert np.array_equal(got, want)
    assert not want[1] and not want[2] and not want[3] and not want[4] and want[5]
    assert not topk.topk_rows_are_exact(sig, rows[:, :-1], k).any()   # wrong length


def test_packed_layout_offsets_heterogeneous_k():
    B, H, NG = 2, 3, 5
    kph = [4, 1, 7]
    offs = topk.idx_row_offsets(B, H, NG, kph)
    # blocks are contiguous, in (b, h) order, each NG*k_h long, and tile [0, total)
    spans = []
    for b in range(B):
        for h in range(H):
            spans.append((offs[b, h], offs[b, h] + NG * kph[h]))
    assert spans[0][0] == 0
    for (s0, e0), (s1, _) in zip(spans, spans[1:]):
        assert e0 == s1
    assert spans[-1][1] == B * NG * sum(kph)


# ---------------------------------------------------------------- MAX group reduction
def test_max_scores_hand_worked():
    # two members (1, 0) and (0, 2) against keys (3, 1), (-1, 1), (0, 0): per-member scores
    # (3, -1, 0) and (2, 2, 0) -> max (3, 2, 0), sum (5, 1, 0)
    q = np.array([[1.0, 0.0], [0.0, 2.0]])
    k = np.array([[3.0, 1.0], [-1.0, 1.0], [0.0, 0.0]])
    mem = np.array([[0, 1]])
    assert np.array_equal(topk.group_scores_max_bruteforce(q, k, mem), [[3.0, 2.0, 0.0]])
    assert np.array_equal(topk.group_scores_bruteforce(q, k, mem), [[5.0, 1.0, 0.0]])
    # the two readings select differently at k = 1 ... and agree at k = 2
    smax = topk.group_scores_max_bruteforce(q, k, mem)
    assert topk.topk_rows_by_sort(smax, 1).tolist() == [[0]]
    assert topk.topk_rows_by_sort(smax, 2).tolist() == [[0, 1]]


def test_max_scores_against_python_loops_and_invariants():
    rng = np.random.default_rng(7)
    q = rng.integers(-7, 8, size=(32, 4)).astype(np.float64)
    k = rng.integers(-7, 8, size=(24, 4)).astype(np.float64)
    mem = geometry.group_members(2, 4, 4, 1, 2, 2)   # 8 groups of 4
    smax = topk.group_scores_max_bruteforce(q, k, mem)
    for g in range(mem.shape[0]):
        for m in range(k.shape[0]):
            ref = max(sum(q[n, c] * k[m, c] for c in range(4)) for n in mem[g])
            assert smax[g, m] == ref
    ssum = topk.group_scores_bruteforce(q, k, mem)
    G = mem.shape[1]
    assert np.all(smax * G >= ssum)                  # max >= mean
    # members in any order give the same scores
    perm = mem[:, ::-1].copy()
    assert np.array_equal(topk.group_scores_max_bruteforce(q, k, perm), smax)
    # groups of identical members: MAX is the per-query score, SUM is G times it
    q2 = np.repeat(q[:8], 4, axis=0)
    mem2 = np.arange(32).reshape(8, 4)
    assert np.array_equal(topk.group_scores_max_bruteforce(q2, k, mem2) * 4,
                          topk.group_scores_bruteforce(q2, k, mem2))

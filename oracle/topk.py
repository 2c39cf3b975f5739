"""Critical-KV estimation: low-rank group scores and exact top-k by a full sort.

DSV summaries (gist.science/{zh,pt,fr,ko}/paper/2502.07590):
  * zh §2.1 / pt §2A / fr §2A / ko §2가: per-head low-rank factors give Q_lr K_lr^T, an
    estimate of QK^T, from which the critical KV pairs are chosen.
  * zh §2.2 / pt §2B / fr §2B / ko §2나: the low-rank MatMul and the top-k selection are one
    fused operation that never stores the S x S scores; adjacent queries form a group that
    shares one list of critical KV indices.
Readings (the pages are silent): a group's score for key m is the SUM over its queries of the
per-query low-rank scores (the MAX over them is the other reading, `group_scores_max_*`); the
row keeps the k keys with the largest group score, equal scores ranked by the lower key index;
the row is written in ascending key order.

Everything is float64 (exact for integer-valued factors below 2^53) or int64.
"""
from __future__ import annotations

import numpy as np


def group_scores_bruteforce(q_lr: np.ndarray, k_lr: np.ndarray, members: np.ndarray) -> np.ndarray:
    """sigma[g, m] = sum_{n in g} u[n, m], with u the per-query scores ([NG, S], fp64).

    Computed group by group (the per-query block of one group, then its column sums), so that
    only G x S scores exist at a time."""
    q = np.asarray(q_lr, dtype=np.float64)
    kt = np.asarray(k_lr, dtype=np.float64).T
    NG = members.shape[0]
    S = kt.shape[1]
    sigma = np.empty((NG, S), dtype=np.float64)
    for g in range(NG):
        u = q[members[g]] @ kt          # [G, S] per-query scores of this group
        sigma[g] = u.sum(axis=0)
    return sigma


def group_scores_sum_first(q_lr: np.ndarray, k_lr: np.ndarray, members: np.ndarray) -> np.ndarray:
    """(sum_{n in g} Q_lr[n]) . K_lr[m]; equal to the brute force by linearity ([NG, S])."""
    q = np.asarray(q_lr, dtype=np.float64)
    s = q[members].sum(axis=1)          # [NG, r]
    return s @ np.asarray(k_lr, dtype=np.float64).T


def group_scores_max_bruteforce(q_lr: np.ndarray, k_lr: np.ndarray,
                                members: np.ndarray) -> np.ndarray:
    """MAX reduction: sigma[g, m] = max_{n in g} u[n, m], u the per-query scores ([NG, S]).

    The other reading of how a group's members combine into one score (the pages only say
    that a group shares its critical indices): the key counts for the group as much as for the
    member that attends to it most. Computed group by group from the G x S per-query block."""
    q = np.asarray(q_lr, dtype=np.float64)
    kt = np.asarray(k_lr, dtype=np.float64).T
    NG = members.shape[0]
    sigma = np.empty((NG, kt.shape[1]), dtype=np.float64)
    for g in range(NG):
        sigma[g] = (q[members[g]] @ kt).max(axis=0)
    return sigma


def topk_rows_by_sort(sigma: np.ndarray, k: int) -> np.ndarray:
    """For each row of sigma: the k largest entries, ties to the lower index, ascending ([NG, k])."""
    S = sigma.shape[1]
    if not 1 <= k <= S:
        raise ValueError("k must lie in [1, S]")
    order = np.argsort(-sigma, axis=1, kind="stable")   # descending, equal keys keep index order
    sel = np.sort(order[:, :k], axis=1)
    return sel.astype(np.int64)


def topk_row_is_exact(sigma_row: np.ndarray, row: np.ndarray, k: int) -> bool:
    """Characterisation of the top-k row, O(S): True iff `row` is the row the sort returns.

    A row is that answer iff it is strictly ascending with k entries in [0, S), every selected
    score is >= every unselected score, and at the threshold T = min selected score, the
    selected keys with score T are exactly the lowest-index keys among all keys scoring T."""
    S = sigma_row.shape[0]
    row = np.asarray(row, dtype=np.int64)
    if row.shape != (k,):
        return False
    if k and (row[0] < 0 or row[-1] >= S):
        return False
    if np.any(np.diff(row) <= 0):
        return False
    mask = np.zeros(S, dtype=bool)
    mask[row] = True
    sel = sigma_row[mask]
    uns = sigma_row[~mask]
    T = sel.min()
    if uns.size and uns.max() > T:
        return False
    ties_all = np.flatnonzero(sigma_row == T)
    ties_sel = np.flatnonzero(mask & (sigma_row == T))
    return bool(np.array_equal(ties_sel, ties_all[: ties_sel.size]))


def topk_rows_are_exact(sigma: np.ndarray, rows: np.ndarray, k: int) -> np.ndarray:
    """topk_row_is_exact for every row at once ([NG] bool), in a few passes over sigma.

    With T the smallest selected score of a row: the row is the sort's answer iff it is strictly
    ascending with k entries in [0, S), every key scoring above T is selected (as many keys
    above T in the whole row as among the selected), and the selected keys scoring T are all
    the keys scoring T up to the largest selected one (then they are the lowest-index ties)."""
    sigma = np.asarray(sigma)
    NG, S = sigma.shape
    rows = np.asarray(rows, dtype=np.int64)
    if rows.shape != (NG, k):
        return np.zeros(NG, dtype=bool)
    ok = np.all(np.diff(rows, axis=1) > 0, axis=1) & (rows[:, 0] >= 0) & (rows[:, -1] < S)
    rc = np.clip(rows, 0, S - 1)
    sel = np.take_along_axis(sigma, rc, axis=1)
    T = sel.min(axis=1)[:, None]
    above_all = np.count_nonzero(sigma > T, axis=1)
    above_sel = np.count_nonzero(sel > T, axis=1)
    tie_sel = sel == T
    n_tie_sel = np.count_nonzero(tie_sel, axis=1)
    last_tie = np.where(tie_sel, rc, -1).max(axis=1)[:, None]
    n_tie_upto = np.count_nonzero((sigma == T) & (np.arange(S)[None, :] <= last_tie), axis=1)
    return ok & (above_all == above_sel) & (n_tie_upto == n_tie_sel)


def idx_row_offsets(B: int, H: int, NG: int, k_per_head) -> np.ndarray:
    """int64 [B, H]: start of the (b, h) block in the packed idx array (rows of k_h, no padding)."""
    k = np.asarray(k_per_head, dtype=np.int64)
    ksum = int(k.sum())
    pre = np.concatenate([[0], np.cumsum(k)[:-1]])
    return np.asarray([[NG * (b * ksum + pre[h]) for h in range(H)] for b in range(B)],
                      dtype=np.int64)


def lowrank_topk(q_lr: np.ndarray, k_lr: np.ndarray, k_per_head, members: np.ndarray,
                 heads_subset=None, reduce: str = "sum") -> np.ndarray:
    """Packed int32 idx for inputs [B, H, S, r]: brute-force group scores (SUM or MAX over the
    members), then a full sort.

    `heads_subset` (list of (b, h)) limits the work to those heads; other rows are left -1."""
    scores = {"sum": group_scores_bruteforce, "max": group_scores_max_bruteforce}[reduce]
    B, H, S, _ = q_lr.shape
    NG = members.shape[0]
    k = [int(x) for x in k_per_head]
    offs = idx_row_offsets(B, H, NG, k)
    out = np.full(B * NG * sum(k), -1, dtype=np.int64)
    todo = heads_subset if heads_subset is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        sigma = scores(q_lr[b, h], k_lr[b, h], members)
        rows = topk_rows_by_sort(sigma, k[h])
        o = offs[b, h]
        out[o:o + NG * k[h]] = rows.reshape(-1)
    return out.astype(np.int32)


def rows_of(idx: np.ndarray, B: int, H: int, NG: int, k_per_head, b: int, h: int) -> np.ndarray:
    """View the (b, h) block of a packed idx array as [NG, k_h]."""
    offs = idx_row_offsets(B, H, NG, k_per_head)
    kh = int(k_per_head[h])
    o = offs[b, h]
    return np.asarray(idx[o:o + NG * kh]).reshape(NG, kh)

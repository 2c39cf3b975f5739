"""Exact softmax attention restricted to each query group's selected keys (float64).

DSV summaries (gist.science/{zh,pt,fr,ko}/paper/2502.07590), zh §2.1 "sparse computation" /
pt §2A / fr §2A / ko §2가: once the critical KV pairs are known, full attention is computed
on those pairs only; zh §2.2 "Query Grouping": all queries of a group use the group's list.
Training (zh §4, "training throughput") needs the backward too; the pages do not describe
it, so the standard softmax-attention gradients are written out here, with the index lists
held constant (no gradient reaches the low-rank factors).

Readings: scale = 1/sqrt(d) unless given; no causal mask; LSE is the natural log of the row's
softmax denominator with the scale included. Inputs are the stored values (bf16 inputs are
upcast exactly by the caller).

Two forms of the same mathematics:
  * dense_masked_*: S x S scores with -inf outside each group's list (small S only).
  * gathered_*:    per group, the G x k block of selected columns; identical up to rounding,
                   because masked entries contribute exact zeros.
"""
from __future__ import annotations

import numpy as np


def _mask(S: int, members: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """Boolean [S, S]: True where key m is in the list of query n's group."""
    allowed = np.zeros((S, S), dtype=bool)
    for g in range(members.shape[0]):
        allowed[np.ix_(members[g], rows[g])] = True
    return allowed


def dense_masked_forward(q, k, v, members, rows, scale):
    """O [S, d] and LSE [S] for one (b, h): z = scale q k^T, -inf off the lists, softmax, P V."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    S = q.shape[0]
    z = scale * (q @ k.T)
    allowed = _mask(S, members, rows)
    z = np.where(allowed, z, -np.inf)
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    den = e.sum(axis=1, keepdims=True)
    lse = (np.log(den) + zmax)[:, 0]
    p = e / den
    return p @ v, lse, p


def dense_masked_backward(q, k, v, do, members, rows, scale):
    """dQ, dK, dV [S, d] for one (b, h), with the index lists held constant.

    Delta_n = dO_n . O_n; dP = dO V^T; dS = P * (dP - Delta); dQ = scale dS K;
    dK = scale dS^T Q; dV = P^T dO."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    o, _, p = dense_masked_forward(q, k, v, members, rows, scale)
    delta = (do * o).sum(axis=1, keepdims=True)
    dp = do @ v.T
    ds = p * (dp - delta)
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    dv = p.T @ do
    return dq, dk, dv


def gathered_forward(q, k, v, members, rows, scale, groups=None):
    """Same result as dense_masked_forward, one G x k block per group.

    `groups` limits the work to a subset of groups; other outputs stay NaN."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    S, d = q.shape
    o = np.full((S, d), np.nan)
    lse = np.full(S, np.nan)
    for g in (range(members.shape[0]) if groups is None else groups):
        mem = members[g]
        sel = rows[g]
        z = scale * (q[mem] @ k[sel].T)                  # [G, k]
        zmax = z.max(axis=1, keepdims=True)
        e = np.exp(z - zmax)
        den = e.sum(axis=1, keepdims=True)
        o[mem] = (e / den) @ v[sel]
        lse[mem] = (np.log(den) + zmax)[:, 0]
    return o, lse


def gathered_backward(q, k, v, do, members, rows, scale, groups=None):
    """Same result as dense_masked_backward; dK/dV are summed over the groups that chose a key.

    With `groups`, dQ rows of other groups stay NaN and dK/dV hold only those groups' share."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    S, d = q.shape
    dq = np.full((S, d), np.nan)
    dk = np.zeros((S, d))
    dv = np.zeros((S, d))
    for g in (range(members.shape[0]) if groups is None else groups):
        mem = members[g]
        sel = rows[g]
        qg, dog = q[mem], do[mem]
        kg, vg = k[sel], v[sel]
        z = scale * (qg @ kg.T)
        zmax = z.max(axis=1, keepdims=True)
        e = np.exp(z - zmax)
        p = e / e.sum(axis=1, keepdims=True)
        og = p @ vg
        delta = (dog * og).sum(axis=1, keepdims=True)
        dp = dog @ vg.T
        ds = p * (dp - delta)
        dq[mem] = scale * (ds @ kg)
        # rows are strictly ascending, so `sel` has no repeats and += adds each key once
        assert np.all(np.diff(sel) > 0)
        dk[sel] += scale * (ds.T @ qg)
        dv[sel] += p.T @ dog
    return dq, dk, dv

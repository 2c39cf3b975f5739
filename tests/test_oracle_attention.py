"""Pins for the oracle's sparse attention forward and backward (CPU only).

Library routines (torch CPU float64 SDPA and autograd), central finite differences, a
hand-worked fixture, closed forms and invariants; none re-types the oracle's formulas."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention, geometry, topk

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _setup(seed, grid=(2, 4, 4), grp=(1, 2, 2), d=8, k=5, full=False):
    rng = np.random.default_rng(seed)
    T, Hh, W = grid
    mem = geometry.group_members(T, Hh, W, *grp)
    S = T * Hh * W
    NG = mem.shape[0]
    if full:
        rows = np.tile(np.arange(S), (NG, 1))
    else:
        rows = np.stack([np.sort(rng.choice(S, size=k, replace=False)) for _ in range(NG)])
    q, kk, v, do = (rng.standard_normal((S, d)) for _ in range(4))
    return mem, rows, q, kk, v, do


def test_hand_worked_fixture():
    fx = json.load(open(os.path.join(GOLD, "toy_attention.json")))
    T, Hh, W = fx["grid"]
    mem = geometry.group_members(T, Hh, W, *fx["group"])
    rows = np.array(fx["rows"])
    S, d = T * Hh * W, 2
    rng = np.random.default_rng(0)
    q, k, v = (rng.standard_normal((S, d)) for _ in range(3))
    q[0] = [math.log(3.0), 0.0]
    for key, val in fx["k"].items():
        k[int(key)] = val
    for key, val in fx["v"].items():
        v[int(key)] = val
    o, lse, _ = attention.dense_masked_forward(q, k, v, mem, rows, fx["scale"])
    assert np.allclose(o[0], fx["o0"], atol=1e-14, rtol=0)
    assert abs(lse[0] - math.log(4.0)) < 1e-14
    og, lseg = attention.gathered_forward(q, k, v, mem, rows, fx["scale"])
    assert np.allclose(og[0], fx["o0"], atol=1e-14, rtol=0)


@pytest.mark.parametrize("seed", range(3))
def test_full_selection_equals_library_sdpa(seed):
    mem, rows, q, k, v, do = _setup(seed, full=True)
    scale = 1 / math.sqrt(q.shape[1])
    o, lse, _ = attention.dense_masked_forward(q, k, v, mem, rows, scale)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq[None, None], tk[None, None], tv[None, None], scale=scale)[0, 0].numpy()
    assert np.max(np.abs(o - ref)) < 1e-12
    ref_lse = torch.logsumexp(scale * (tq @ tk.T), dim=1).numpy()
    assert np.max(np.abs(lse - ref_lse)) < 1e-12
    og, lg = attention.gathered_forward(q, k, v, mem, rows, scale)
    assert np.max(np.abs(og - ref)) < 1e-12 and np.max(np.abs(lg - ref_lse)) < 1e-12


@pytest.mark.parametrize("seed", range(3))
def test_full_selection_backward_equals_autograd(seed):
    mem, rows, q, k, v, do = _setup(seed, full=True)
    scale = 0.37
    dq, dk, dv = attention.dense_masked_backward(q, k, v, do, mem, rows, scale)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq[None, None], tk[None, None], tv[None, None], scale=scale)[0, 0]
    out.backward(torch.tensor(do))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.max(np.abs(mine - ref.numpy())) < 1e-12


def test_softmax_rows_sum_to_one_and_respect_lists():
    mem, rows, q, k, v, _ = _setup(3)
    _, _, p = attention.dense_masked_forward(q, k, v, mem, rows, 0.5)
    assert np.max(np.abs(p.sum(axis=1) - 1)) < 1e-12
    g_of = geometry.group_of_token(mem, q.shape[0])
    for n in range(q.shape[0]):
        off = np.setdiff1d(np.arange(q.shape[0]), rows[g_of[n]])
        assert np.all(p[n, off] == 0)
        assert np.all(p[n, rows[g_of[n]]] > 0)


def test_single_key_closed_form():
    mem, rows, q, k, v, do = _setup(4, k=1)
    scale = 0.3
    o, lse, _ = attention.dense_masked_forward(q, k, v, mem, rows, scale)
    g_of = geometry.group_of_token(mem, q.shape[0])
    for n in range(q.shape[0]):
        m = rows[g_of[n], 0]
        assert np.allclose(o[n], v[m], atol=1e-14, rtol=0)
        assert abs(lse[n] - scale * q[n] @ k[m]) < 1e-13
    dq, dk, dv = attention.dense_masked_backward(q, k, v, do, mem, rows, scale)
    assert np.max(np.abs(dq)) < 1e-13 and np.max(np.abs(dk)) < 1e-13
    ref_dv = np.zeros_like(dv)
    for g in range(mem.shape[0]):
        ref_dv[rows[g, 0]] += do[mem[g]].sum(axis=0)
    assert np.max(np.abs(dv - ref_dv)) < 1e-13


def test_zero_queries_average_selected_values():
    mem, rows, q, k, v, _ = _setup(5, k=6)
    q[:] = 0
    o, lse, _ = attention.dense_masked_forward(q, k, v, mem, rows, 0.7)
    g_of = geometry.group_of_token(mem, q.shape[0])
    for n in range(q.shape[0]):
        assert np.allclose(o[n], v[rows[g_of[n]]].mean(axis=0), atol=1e-14, rtol=0)
        assert abs(lse[n] - math.log(6)) < 1e-14


def test_shift_invariances():
    mem, rows, q, k, v, _ = _setup(6)
    o, _, _ = attention.dense_masked_forward(q, k, v, mem, rows, 0.4)
    o_k, _, _ = attention.dense_masked_forward(q, k + 2.5, v, mem, rows, 0.4)
    o_v, _, _ = attention.dense_masked_forward(q, k, v - 1.25, mem, rows, 0.4)
    assert np.max(np.abs(o_k - o)) < 1e-12
    assert np.max(np.abs(o_v - (o - 1.25))) < 1e-12


def _loss(q, k, v, do, mem, rows, scale):
    o, _, _ = attention.dense_masked_forward(q, k, v, mem, rows, scale)
    return float((o * do).sum())


@pytest.mark.parametrize("seed", range(2))
def test_backward_matches_central_differences(seed):
    mem, rows, q, k, v, do = _setup(10 + seed, d=4, k=4)
    scale = 0.6
    dq, dk, dv = attention.dense_masked_backward(q, k, v, do, mem, rows, scale)
    h = 1e-6
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + h
            fp = _loss(q, k, v, do, mem, rows, scale)
            arr[idx] = keep - h
            fm = _loss(q, k, v, do, mem, rows, scale)
            arr[idx] = keep
            num[idx] = (fp - fm) / (2 * h)
        assert np.max(np.abs(num - grad)) < 1e-7, name


def test_backward_sum_rules_and_unselected_keys():
    mem, rows, q, k, v, do = _setup(20, k=3)
    dq, dk, dv = attention.dense_masked_backward(q, k, v, do, mem, rows, 0.5)
    assert np.max(np.abs(dv.sum(axis=0) - do.sum(axis=0))) < 1e-12
    assert np.max(np.abs(dk.sum(axis=0))) < 1e-12
    unsel = np.setdiff1d(np.arange(q.shape[0]), np.unique(rows))
    assert unsel.size > 0
    assert np.all(dk[unsel] == 0) and np.all(dv[unsel] == 0)


@pytest.mark.parametrize("seed", range(2))
def test_gathered_equals_dense(seed):
    mem, rows, q, k, v, do = _setup(30 + seed, grid=(2, 4, 8), grp=(2, 2, 2), d=16, k=9)
    scale = 0.25
    o, lse, _ = attention.dense_masked_forward(q, k, v, mem, rows, scale)
    og, lg = attention.gathered_forward(q, k, v, mem, rows, scale)
    assert np.max(np.abs(o - og)) < 1e-13 and np.max(np.abs(lse - lg)) < 1e-13
    d1 = attention.dense_masked_backward(q, k, v, do, mem, rows, scale)
    d2 = attention.gathered_backward(q, k, v, do, mem, rows, scale)
    for a, b in zip(d1, d2):
        assert np.max(np.abs(a - b)) < 1e-13
    # a group subset reproduces those groups' rows
    og2, _ = attention.gathered_forward(q, k, v, mem, rows, scale, groups=[1, 3])
    for g in (1, 3):
        assert np.max(np.abs(og2[mem[g]] - o[mem[g]])) < 1e-13


def test_end_to_end_tiny_selection_is_a_top_k_of_low_rank_scores():
    """topk + attention chained as the hot path chains them, on a small grid."""
    rng = np.random.default_rng(40)
    T, Hh, W, r, d = 2, 4, 8, 4, 8
    mem = geometry.group_members(T, Hh, W, 1, 2, 4)
    S = T * Hh * W
    ql = rng.integers(-7, 8, size=(1, 1, S, r)).astype(float)
    kl = rng.integers(-7, 8, size=(1, 1, S, r)).astype(float)
    idx = topk.lowrank_topk(ql, kl, [10], mem)
    rows = topk.rows_of(idx, 1, 1, mem.shape[0], [10], 0, 0)
    sig = topk.group_scores_sum_first(ql[0, 0], kl[0, 0], mem)
    for g in range(mem.shape[0]):
        assert topk.topk_row_is_exact(sig[g], rows[g], 10)
    q, k, v = (rng.standard_normal((S, d)) for _ in range(3))
    o, _, p = attention.dense_masked_forward(q, k, v, mem, rows, 1 / math.sqrt(d))
    assert np.all(np.isfinite(o))

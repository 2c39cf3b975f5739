"""The library's host-side planning (head placement, cost model, dense-versus-sparse choice)
against the oracle, and its argument checks. CPU only: no HIP call is made."""
import ctypes
import random

import pytest

import dynamic_sparse_attention_rank_amd as dsv
from oracle import planning


@pytest.mark.parametrize("seed", range(30))
def test_plan_heads_matches_oracle(seed):
    rng = random.Random(seed)
    H = rng.randint(1, 48)
    m = rng.randint(1, 9)
    ks = [rng.choice([2621, 6554, 13107, 26214, rng.randint(1, 65536)]) for _ in range(H)]
    fixed, per_k = rng.choice([(0.0, 1.0), (0.1, 3.1e-4), (5.0, 0.0)])
    part, load, rho = dsv.plan_heads(ks, m, fixed, per_k)
    opart, oload = planning.lpt(planning.head_costs(ks, fixed, per_k), m)
    assert part == opart
    assert load == pytest.approx(oload, rel=1e-15, abs=0.0)
    assert rho == pytest.approx(planning.rho_s(oload), rel=1e-15)


@pytest.mark.parametrize("seed", range(10))
def test_plan_order_matches_oracle(seed):
    rng = random.Random(100 + seed)
    H = rng.randint(1, 64)
    ks = [rng.choice([2621, 6554, 13107, 26214]) for _ in range(H)]
    fixed, per_k = rng.choice([(0.0, 1.0), (0.3, 2e-4), (1.0, 0.0)])
    assert dsv.plan_order(ks, fixed, per_k) == \
        planning.lpt_order(planning.head_costs(ks, fixed, per_k))


def test_plan_order_is_the_one_device_placement_order():
    # on one device the greedy places every head, in its processing order
    ks = [2621, 26214, 6554, 26214, 13107, 2621]
    order = dsv.plan_order(ks)
    assert order == [1, 3, 4, 2, 0, 5]
    part, load, rho = dsv.plan_heads(ks, 1, 0.0, 1.0)
    assert part == [0] * 6 and rho == 1.0


def test_plan_heads_long_workload():
    # the heterogeneous-k workload (S = 128K, k in {2%, 5%, 10%, 20%} of S, 16 heads) on 8
    # devices; a round-robin placement (heads 0..15 -> devices h % 8) for comparison
    ks = [2621, 6554, 13107, 26214] * 4
    part, load, rho = dsv.plan_heads(ks, 8, 0.0, 1.0)
    assert rho == pytest.approx(planning.rho_s(planning.lpt([float(k) for k in ks], 8)[1]))
    rr = [sum(k for h, k in enumerate(ks) if h % 8 == q) for q in range(8)]
    assert rho < planning.rho_s(rr)
    assert rho >= max(ks) / (sum(ks) / 8)


def test_plan_heads_rejects_bad_arguments():
    L = dsv.lib()
    ks = (ctypes.c_int32 * 2)(1, 2)
    out = (ctypes.c_int32 * 2)()
    assert dsv.STATUS[L.dsv_plan_heads(None, 2, 2, 0.0, 1.0, out, None, None)] == "DSV_ERR_NULL"
    assert dsv.STATUS[L.dsv_plan_heads(ks, 0, 2, 0.0, 1.0, out, None, None)] == "DSV_ERR_SHAPE"
    assert dsv.STATUS[L.dsv_plan_heads(ks, 2, 0, 0.0, 1.0, out, None, None)] == "DSV_ERR_SHAPE"
    assert dsv.STATUS[L.dsv_plan_heads(ks, 2, 2, 0.0, 0.0, out, None, None)] == "DSV_ERR_SHAPE"
    assert dsv.STATUS[L.dsv_plan_heads(ks, 2, 2, -1.0, 1.0, out, None, None)] == "DSV_ERR_SHAPE"
    bad = (ctypes.c_int32 * 2)(1, 0)
    assert dsv.STATUS[L.dsv_plan_heads(bad, 2, 2, 0.0, 1.0, out, None, None)] == "DSV_ERR_K"


def test_cost_model_scales_with_the_work():
    mid = dsv.problem(1, 24, 16, 64, 64, 128, 32, (4, 4, 4), "bf16")
    small = dsv.problem(1, 16, 16, 32, 32, 64, 16, (4, 4, 4), "bf16")
    a, b = dsv.default_cost_model(mid), dsv.default_cost_model(small)
    assert b.attn_ns_per_edge == pytest.approx(a.attn_ns_per_edge / 2)   # d 128 -> 64
    assert b.topk_ns_per_score == pytest.approx(a.topk_ns_per_score / 2)  # r 32 -> 16
    f = dsv.default_cost_model(mid, with_backward=False)
    assert 0 < f.attn_ns_per_edge < a.attn_ns_per_edge


@pytest.mark.parametrize("seed", range(10))
def test_dispatch_matches_oracle(seed):
    rng = random.Random(seed)
    p = dsv.problem(1, 8, 4, 16, 16, 64, 16, (2, 2, 4), "bf16")
    S = p.seq
    cm = dsv.CostModel(rng.uniform(0.0, 0.5), rng.uniform(0.5, 2.0))
    ks = [rng.randint(1, S) for _ in range(8)]
    ks[0] = S
    out, nd = dsv.dispatch_k(p, ks, cm)
    oout, ond = planning.dispatch_k(ks, S, cm.topk_ns_per_score, cm.attn_ns_per_edge)
    assert out == oout and nd == ond and out[0] == S


def test_dispatch_default_model_only_near_dense_goes_dense():
    p = dsv.problem(1, 24, 16, 64, 64, 128, 32, (4, 4, 4), "bf16")
    S = p.seq
    out, nd = dsv.dispatch_k(p, [6554] * 23 + [S])
    assert nd == 1 and out[-1] == S and out[:-1] == [6554] * 23
    cm = dsv.default_cost_model(p)
    kstar = S * (1 - cm.topk_ns_per_score / cm.attn_ns_per_edge)
    assert 0.99 * S < kstar < S
    with pytest.raises(dsv.DsvError):
        dsv.dispatch_k(p, [0] * 24)

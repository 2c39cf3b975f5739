"""GPU parity of the MAX group reduction (dsv_lowrank_topk with DSV_GROUP_MAX) against the
oracle's brute-force per-member scores and full sort: idx bit-exact."""
import numpy as np
import pytest
import torch

import dynamic_sparse_attention_rank_amd as dsv
from oracle import topk as otopk
from parity_util import f64, gpu_inputs, gpu_rows, members, say, workload

pytestmark = pytest.mark.gpu

CASES = [
    # (label, workload, overrides, k_per_head or None)
    ("tiny-fp32", "tiny", {}, None),
    ("small", "small", dict(heads=4), None),
    ("k1-kS", "small", dict(heads=2, frames=2, height=8, width=8, group=(2, 2, 4), rank=32),
     [1, 128]),
    ("ragged-k", "small", dict(heads=3, frames=4, height=8, width=12, group=(2, 2, 4), rank=32),
     [7, 45, 100]),
    ("G32-r48", "small", dict(heads=2, frames=4, height=8, width=16, group=(2, 4, 4), rank=48),
     [33, 60]),
    ("G48-r64", "small", dict(heads=2, frames=3, height=8, width=16, group=(3, 4, 4), rank=64),
     [50, 9]),
    ("NG36", "small", dict(heads=2, frames=4, height=12, width=12, group=(2, 2, 4), rank=16),
     [71, 200]),
    ("fp32-r32", "small", dict(heads=2, frames=4, height=8, width=8, group=(2, 2, 4), rank=32,
                               dtype="fp32"), [19, 64]),
]


def _max_rows(cfg, x, b, h, mem):
    sig = otopk.group_scores_max_bruteforce(f64(x["q_lr"][b, h]), f64(x["k_lr"][b, h]), mem)
    return otopk.topk_rows_by_sort(sig, int(x["k_per_head"][h]))


@pytest.mark.parametrize("label,name,over,ks", CASES, ids=[c[0] for c in CASES])
def test_topk_max_bit_exact(label, name, over, ks):
    cfg = workload(name, **over)
    say(f"[topk-max] {label}")
    x = gpu_inputs(cfg, backward=False, k_per_head=ks)
    p = dsv.problem_for(cfg)
    idx = dsv.lowrank_topk(p, x["q_lr"], x["k_lr"], x["k_per_head"], reduce=dsv.DSV_GROUP_MAX)
    torch.cuda.synchronize()
    mem = members(cfg)
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            got = gpu_rows(cfg, x, idx, b, h)
            ref = _max_rows(cfg, x, b, h, mem)
            assert np.array_equal(got, ref), (b, h, np.argwhere(got != ref)[:5])


def test_topk_max_differs_from_sum_and_repeats():
    cfg = workload("small", heads=2)
    x = gpu_inputs(cfg, backward=False)
    p = dsv.problem_for(cfg)
    a = dsv.lowrank_topk(p, x["q_lr"], x["k_lr"], x["k_per_head"], reduce=dsv.DSV_GROUP_MAX)
    b2 = dsv.lowrank_topk(p, x["q_lr"], x["k_lr"], x["k_per_head"], reduce=dsv.DSV_GROUP_MAX)
    s = dsv.lowrank_topk(p, x["q_lr"], x["k_lr"], x["k_per_head"], reduce=dsv.DSV_GROUP_SUM)
    torch.cuda.synchronize()
    assert torch.equal(a, b2)
    assert not torch.equal(a, s)   # the two readings select different keys on these inputs


def _cache_ws(p, slots):
    return torch.empty(dsv.topk_max_cache_bytes(p) * slots, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("label,name,over,ks", CASES, ids=[c[0] for c in CASES])
def test_topk_max_cached_bit_exact(label, name, over, ks):
    """Group scores kept in the workspace between passes: same rows as the oracle."""
    cfg = workload(name, **over)
    say(f"[topk-max cached] {label}")
    x = gpu_inputs(cfg, backward=False, k_per_head=ks)
    p = dsv.problem_for(cfg)
    ws = _cache_ws(p, cfg.batch * cfg.heads)
    idx = dsv.lowrank_topk(p, x["q_lr"], x["k_lr"], x["k_per_head"], reduce=dsv.DSV_GROUP_MAX,
                           ws=ws)
    torch.cuda.synchronize()
    mem = members(cfg)
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            got = gpu_rows(cfg, x, idx, b, h)
            ref = _max_rows(cfg, x, b, h, mem)
            assert np.array_equal(got, ref), (b, h, np.argwhere(got != ref)[:5])


@pytest.mark.parametrize("slots", [1, 2, 5, 6])
def test_topk_max_cache_chunks(slots):
    """Workspaces for fewer slots than B*H (launches of `slots` slots, the last one short), one
    just short of a slot and one not 256-byte aligned (no cache): bit-identical to the
    recomputing kernel."""
    cfg = workload("small", batch=2, heads=3, frames=4, height=8, width=12, group=(2, 2, 4),
                   rank=32)
    say(f"[topk-max cache chunks] slots={slots}")
    x = gpu_inputs(cfg, backward=False, k_per_head=[7, 45, 100])
    p = dsv.problem_for(cfg)
    ref = dsv.lowrank_topk(p, x["q_lr"], x["k_lr"], x["k_per_head"], reduce=dsv.DSV_GROUP_MAX)
    ws = _cache_ws(p, slots)
    got = dsv.lowrank_topk(p, x["q_lr"], x["k_lr"], x["k_per_head"], reduce=dsv.DSV_GROUP_MAX,
                           ws=ws)
    short = dsv.lowrank_topk(p, x["q_lr"], x["k_lr"], x["k_per_head"],
                             reduce=dsv.DSV_GROUP_MAX, ws=ws[:dsv.topk_max_cache_bytes(p) - 256])
    # not 256-byte aligned: the scores are recomputed instead of cached
    skew = torch.empty(dsv.topk_max_cache_bytes(p) * slots + 64, dtype=torch.uint8, device="cuda")
    odd = dsv.lowrank_topk(p, x["q_lr"], x["k_lr"], x["k_per_head"], reduce=dsv.DSV_GROUP_MAX,
                           ws=skew[64:])
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    assert torch.equal(short, ref)
    assert torch.equal(odd, ref)

"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

The oracle cannot run every output at these sizes in seconds, so:
  * top-k: every row of every head is checked with the exact characterisation (pinned to the
    brute-force sort by the CPU tests), plus brute force on sampled groups;
  * forward: sampled groups of every head against the gathered fp64 oracle;
  * backward: dQ on sampled groups, dK/dV of one full head (all groups' contributions), and
    the sum rules on every head.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import dynamic_sparse_attention_rank_amd as dsv
from oracle import topk as otopk
from parity_util import (TOL, characterise_all_rows, f64, gpu_inputs, gpu_rows, maxerr,
                         members, oracle_bwd, oracle_fwd, run_bwd, run_fwd, run_topk, say,
                         workload)

pytestmark = pytest.mark.gpu


def _sampled_groups(NG, n, seed):
    rng = np.random.default_rng(seed)
    return sorted(set([0, NG - 1] + rng.choice(NG, size=n, replace=False).tolist()))


def _characterise_heads(cfg, x, idx, heads, mem):
    """The exact characterisation on every row of the given (b, h) slots, 8 host threads."""
    with ThreadPoolExecutor(max_workers=8) as ex:
        bad = list(ex.map(lambda bh: characterise_all_rows(cfg, x, idx, bh[0], bh[1], mem),
                          heads))
    for (b, h), nb in zip(heads, bad):
        assert nb == 0, (b, h, nb)


def _topk_checks(cfg, x, idx, heads=None, brute_groups=3, seed=0):
    mem = members(cfg)
    heads = [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)] if heads is None else heads
    _characterise_heads(cfg, x, idx, heads, mem)
    b, h = heads[0]
    rows = gpu_rows(cfg, x, idx, b, h)
    for g in _sampled_groups(cfg.n_groups, brute_groups, seed):
        sig = otopk.group_scores_bruteforce(f64(x["q_lr"][b, h]), f64(x["k_lr"][b, h]),
                                            mem[g:g + 1])
        ref = otopk.topk_rows_by_sort(sig, int(x["k_per_head"][h]))[0]
        assert np.array_equal(rows[g], ref), (b, h, g)


def _fwd_sampled(cfg, x, idx, o, lse, n_groups=6, seed=1):
    mem = members(cfg)
    worst = 0.0
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            groups = _sampled_groups(cfg.n_groups, n_groups, seed + 31 * h + b)
            rows = gpu_rows(cfg, x, idx, b, h)
            ro, rl = oracle_fwd(cfg, x, rows, b, h, groups=groups, mem=mem)
            eo, el = maxerr(f64(o[b, h]), ro), maxerr(f64(lse[b, h]), rl)
            worst = max(worst, eo, el)
            assert eo <= TOL[cfg.dtype] and el <= TOL[cfg.dtype], (b, h, eo, el)
    say(f"   fwd sampled worst max-abs-err {worst:.3e}")


def test_mid_topk_fwd_bwd():
    cfg = workload("mid")
    say("[full] mid: top-k + fwd + bwd at S=65536, 24 heads")
    x = gpu_inputs(cfg, backward=True)
    idx = run_topk(cfg, x)
    torch.cuda.synchronize()
    _topk_checks(cfg, x, idx)
    o, lse = run_fwd(cfg, x, idx)
    # the launch configuration bench.py times: room for every slot (one launch of 24 heads)
    # within a third of the device's memory; the default (one head per launch) must give the
    # same bits
    p = dsv.problem_for(cfg)
    one = dsv.workspace_bytes(dsv.DSV_OP_BWD, p, x["k_per_head"])
    cap = torch.cuda.get_device_properties(0).total_memory // 3
    ws = torch.empty(one * max(1, min(cfg.batch * cfg.heads + 1, cap // one)), dtype=torch.uint8,
                     device="cuda")
    say(f"   bwd workspace {ws.numel() / 1e9:.1f} GB, "
        f"{dsv.bwd_chunks(p, x['k_per_head'], ws.numel())} launch(es)")
    dq, dk, dv = dsv.sparse_attn_bwd(p, x["q"], x["k"], x["v"], o, x["do"], lse, idx,
                                     x["k_per_head"], x["scale"], ws=ws)
    del ws
    d1 = run_bwd(cfg, x, idx, o, lse)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip((dq, dk, dv), d1))
    del d1
    _fwd_sampled(cfg, x, idx, o, lse, n_groups=4)
    mem = members(cfg)
    # dQ on sampled groups of three heads; dK/dV of head 5 over all its groups
    for h in (0, 11, 23):
        groups = _sampled_groups(cfg.n_groups, 3, 100 + h)
        rows = gpu_rows(cfg, x, idx, 0, h)
        rq, _, _ = oracle_bwd(cfg, x, rows, 0, h, groups=groups, mem=mem)
        e = maxerr(f64(dq[0, h]), rq)
        assert e <= TOL["bf16"], (h, e)
    h = 5
    rows = gpu_rows(cfg, x, idx, 0, h)
    rq, rk, rv = oracle_bwd(cfg, x, rows, 0, h, mem=mem)
    e = (maxerr(f64(dq[0, h]), rq), maxerr(f64(dk[0, h]), rk), maxerr(f64(dv[0, h]), rv))
    say(f"   bwd head {h} max-abs-err dq/dk/dv {e}")
    assert max(e) <= TOL["bf16"], e
    s_dv = dv.double().sum(dim=2)
    s_do = x["do"].double().sum(dim=2)
    assert float((s_dv - s_do).abs().max()) < 1.0
    assert float(dk.double().sum(dim=2).abs().max()) < 1.0


def test_long_heterogeneous_topk_fwd():
    cfg = workload("long")
    say("[full] long: S=131072, per-head k drawn from {2,5,10,20}%")
    x = gpu_inputs(cfg, backward=False)
    ks = x["k_per_head"]
    say(f"   k_per_head = {ks}")
    assert len(set(ks)) > 1
    idx = run_topk(cfg, x)
    torch.cuda.synchronize()
    # every row of every head (the heaviest first for the brute-force samples)
    heavy = int(np.argmax(ks))
    _topk_checks(cfg, x, idx, heads=[(0, heavy)] + [(0, h) for h in range(cfg.heads)
                                                     if h != heavy])
    o, lse = run_fwd(cfg, x, idx)
    torch.cuda.synchronize()
    _fwd_sampled(cfg, x, idx, o, lse, n_groups=3)


@pytest.mark.timeout(1200)
def test_training_steps():
    """20 seeded steps with fresh inputs: every row of every (b, h) slot characterised on every
    step; the forward on sampled groups of two slots per step; the backward of one slot per
    step against the gathered oracle (the slot rotating over the steps): dQ, dK and dV of the
    whole slot on steps 0, 5, 10, 15 and 19, dQ of sampled groups on the others."""
    cfg = workload("training")
    say("[full] training: 2 x S=61440, 24 heads, k=5%, 20 seeded steps")
    mem = members(cfg)
    slots = [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)]
    worst = {"fwd": 0.0, "dq": 0.0, "dk": 0.0, "dv": 0.0}
    for step in range(cfg.steps):
        x = gpu_inputs(cfg, step=step, backward=True)
        idx = run_topk(cfg, x)
        o, lse = run_fwd(cfg, x, idx)
        dq, dk, dv = run_bwd(cfg, x, idx, o, lse)
        torch.cuda.synchronize()
        _characterise_heads(cfg, x, idx, slots, mem)
        if step == 0:   # brute-force group scores on sampled groups of one slot
            _topk_checks(cfg, x, idx, heads=[slots[0]], brute_groups=2)
        for b, h in (slots[(5 * step) % len(slots)], slots[(5 * step + 29) % len(slots)]):
            rows = gpu_rows(cfg, x, idx, b, h)
            groups = _sampled_groups(cfg.n_groups, 2, 400 + step)
            ro, rl = oracle_fwd(cfg, x, rows, b, h, groups=groups, mem=mem)
            e = max(maxerr(f64(o[b, h]), ro), maxerr(f64(lse[b, h]), rl))
            worst["fwd"] = max(worst["fwd"], e)
            assert e <= TOL["bf16"], (step, b, h, e)
        b, h = slots[(7 * step + 3) % len(slots)]
        rows = gpu_rows(cfg, x, idx, b, h)
        if step % 5 == 0 or step == cfg.steps - 1:   # the whole slot: dQ, dK and dV
            rq, rk, rv = oracle_bwd(cfg, x, rows, b, h, mem=mem)
            e = (maxerr(f64(dq[b, h]), rq), maxerr(f64(dk[b, h]), rk),
                 maxerr(f64(dv[b, h]), rv))
        else:                                      # dQ of sampled groups
            groups = _sampled_groups(cfg.n_groups, 3, 500 + step)
            rq, _, _ = oracle_bwd(cfg, x, rows, b, h, groups=groups, mem=mem)
            e = (maxerr(f64(dq[b, h]), rq),)
        for name, v in zip(("dq", "dk", "dv"), e):
            worst[name] = max(worst[name], v)
        assert max(e) <= TOL["bf16"], (step, b, h, e)
        say(f"   step {step}: 48 slots characterised; bwd (b={b}, h={h}) max-abs-err {e}")
        del x, idx, o, lse, dq, dk, dv
        torch.cuda.empty_cache()
    say(f"   worst over 20 steps: {worst}")


def test_mid_adaptive_k_sampled_groups():
    """Adaptive k at S=65536: sampled groups of three heads against the oracle's sort rule
    (equal outside the rounding band); the head k is the largest group k."""
    import math
    from oracle import adaptive as oad
    from parity_util import adaptive_band
    cfg = workload("mid")
    say("[full] mid: adaptive k, mass 0.9")
    x = gpu_inputs(cfg, backward=False)
    p = dsv.problem_for(cfg)
    kh, kg = dsv.adaptive_k(p, x["q_lr"], x["k_lr"], mass=0.9)
    torch.cuda.synchronize()
    kg = kg.cpu().numpy()
    assert np.array_equal(kh.cpu().numpy(), kg.max(axis=(0, 2)))
    ls32 = float(np.float32(1.0 / (math.sqrt(cfg.head_dim) * p.group_size)))
    mem = members(cfg)
    band = adaptive_band(p.seq)
    for h in (0, 7, 23):
        for g in _sampled_groups(cfg.n_groups, 4, 200 + h):
            sig = otopk.group_scores_sum_first(f64(x["q_lr"][0, h]), f64(x["k_lr"][0, h]),
                                               mem[g:g + 1])[0]
            ke, lo, hi = oad.k_with_bracket(sig, ls32, 0.9, band)
            got = int(kg[0, h, g])
            assert lo <= got <= hi and (lo != hi or got == ke), (h, g, got, ke, lo, hi)


def test_mid_topk_max_sampled_groups():
    """MAX top-k at S=65536: sampled groups of two heads against the brute-force oracle."""
    cfg = workload("mid")
    say("[full] mid: top-k with the MAX group reduction")
    x = gpu_inputs(cfg, backward=False)
    p = dsv.problem_for(cfg)
    idx = dsv.lowrank_topk(p, x["q_lr"], x["k_lr"], x["k_per_head"], reduce=dsv.DSV_GROUP_MAX)
    # the configuration bench.py times: every slot's group scores cached in the workspace
    ws = torch.empty(dsv.topk_max_cache_bytes(p) * cfg.batch * cfg.heads, dtype=torch.uint8,
                     device="cuda")
    idx_c = dsv.lowrank_topk(p, x["q_lr"], x["k_lr"], x["k_per_head"],
                             reduce=dsv.DSV_GROUP_MAX, ws=ws)
    torch.cuda.synchronize()
    del ws
    assert torch.equal(idx_c, idx)
    mem = members(cfg)
    for h in (0, 17):
        rows = gpu_rows(cfg, x, idx, 0, h)
        for g in _sampled_groups(cfg.n_groups, 3, 300 + h):
            sig = otopk.group_scores_max_bruteforce(f64(x["q_lr"][0, h]), f64(x["k_lr"][0, h]),
                                                    mem[g:g + 1])
            ref = otopk.topk_rows_by_sort(sig, int(x["k_per_head"][h]))[0]
            assert np.array_equal(rows[g], ref), (h, g)

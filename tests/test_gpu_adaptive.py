"""GPU parity of the adaptive k (dsv_adaptive_k) against the oracle's plain rule (fp64 softmax
weights, full sort, exactly rounded prefix sums): every group's k equal to it wherever no
prefix sum lies within the kernel's stated rounding band of the target, and inside the band's
bracket everywhere; the head's k their maximum; repeatable bit for bit."""
import math

import numpy as np
import pytest
import torch

import dynamic_sparse_attention_rank_amd as dsv
from oracle import adaptive as oad
from oracle import topk as otopk
from parity_util import adaptive_band, f64, gpu_inputs, members, say, workload

pytestmark = pytest.mark.gpu

CASES = [
    # (label, workload, overrides, mass, logit scale factor on 1/(sqrt(d) G))
    ("tiny-fp32", "tiny", {}, 0.9, 1.0),
    ("small", "small", {}, 0.9, 1.0),
    ("small-sharp", "small", dict(heads=4), 0.9, 16.0),
    ("small-m50", "small", dict(heads=4), 0.5, 4.0),
    ("ragged-r48", "small", dict(heads=2, frames=4, height=8, width=16, group=(2, 4, 4),
                                 rank=48), 0.95, 2.0),
    ("G48-r64", "small", dict(heads=2, frames=3, height=8, width=16, group=(3, 4, 4),
                              rank=64), 0.9, 8.0),
    ("mass1", "small", dict(heads=2, frames=4, height=8, width=8, group=(2, 2, 4)), 1.0, 1.0),
]


@pytest.mark.parametrize("label,name,over,mass,fac", CASES, ids=[c[0] for c in CASES])
def test_adaptive_k_bit_exact(label, name, over, mass, fac):
    cfg = workload(name, **over)
    say(f"[adaptive-k] {label}")
    x = gpu_inputs(cfg, backward=False)
    p = dsv.problem_for(cfg)
    ls = fac / (math.sqrt(cfg.head_dim) * p.group_size)
    ls32 = float(np.float32(ls))
    kh, kg = dsv.adaptive_k(p, x["q_lr"], x["k_lr"], mass=mass, logit_scale=ls)
    torch.cuda.synchronize()
    kg = kg.cpu().numpy()
    kh = kh.cpu().numpy()
    mem = members(cfg)
    band = adaptive_band(p.seq)
    n_amb = 0
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            sig = otopk.group_scores_sum_first(f64(x["q_lr"][b, h]), f64(x["k_lr"][b, h]), mem)
            for g in range(sig.shape[0]):
                ke, lo, hi = oad.k_with_bracket(sig[g], ls32, mass, band)
                got = int(kg[b, h, g])
                assert lo <= got <= hi, (b, h, g, got, ke, lo, hi)
                if lo == hi:
                    assert got == ke, (b, h, g, got, ke)
                else:
                    n_amb += 1
    say(f"   {kg.size} groups, {n_amb} within the rounding band of the target")
    assert np.array_equal(kh, kg.max(axis=(0, 2)))
    if mass == 1.0:
        assert np.all(kg == p.seq)
    kh2, kg2 = dsv.adaptive_k(p, x["q_lr"], x["k_lr"], mass=mass, logit_scale=ls)
    assert torch.equal(kh2.cpu(), torch.from_numpy(kh)) and np.array_equal(kg2.cpu().numpy(), kg)


def test_adaptive_k_feeds_topk():
    """The head k from the estimator drives the top-k and the forward in the same process."""
    cfg = workload("small", heads=2)
    x = gpu_inputs(cfg, backward=False)
    p = dsv.problem_for(cfg)
    kh, _ = dsv.adaptive_k(p, x["q_lr"], x["k_lr"], mass=0.9)
    ks = [int(v) for v in kh.cpu()]
    assert all(1 <= k <= p.seq for k in ks)
    idx = dsv.lowrank_topk(p, x["q_lr"], x["k_lr"], ks)
    o, lse = dsv.sparse_attn_fwd(p, x["q"], x["k"], x["v"], idx, ks, x["scale"])
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()

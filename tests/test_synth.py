"""The seeded input generator: determinism, value laws and shapes (CPU only)."""
import dataclasses

import numpy as np
import torch

from synth import CONFIGS, make_inputs, draw_k_per_head


def test_configs_match_their_stated_sizes():
    t, s, m, lg, tr = (CONFIGS[n] for n in ("tiny", "small", "mid", "long", "training"))
    assert (t.seq, t.group_size, t.n_groups, t.k_uniform()) == (1024, 16, 64, 128)
    assert (s.seq, s.group_size, s.n_groups, s.k_uniform()) == (16384, 64, 256, 1638)
    assert (m.seq, m.n_groups, m.k_uniform()) == (65536, 1024, 6554)
    assert (lg.seq, lg.n_groups, lg.k_uniform()) == (131072, 2048, None)
    assert (tr.seq, tr.batch, tr.n_groups, tr.k_uniform()) == (61440, 2, 960, 3072)


def test_long_k_draw_is_seeded_and_from_the_set():
    lg = CONFIGS["long"]
    a = draw_k_per_head(lg, 3000)
    assert a == draw_k_per_head(lg, 3000)
    assert set(a) <= {2621, 6554, 13107, 26214} and len(a) == 16


def test_tiny_inputs_deterministic_and_lawful():
    cfg = CONFIGS["tiny"]
    a = make_inputs(cfg, device="cpu", backward=True)
    b = make_inputs(cfg, device="cpu", backward=True)
    for key in ("q", "k", "v", "q_lr", "k_lr", "do"):
        assert torch.equal(a[key], b[key]), key
    assert a["q"].dtype == torch.float32 and a["q"].shape == (1, 2, 1024, 64)
    for key in ("q", "v"):
        assert abs(float(a[key].std()) - 1.0) < 1e-3
    lr = a["q_lr"].numpy()
    assert np.array_equal(lr, np.round(lr)) and lr.min() >= -7 and lr.max() <= 7
    assert a["k_per_head"] == [128, 128]
    c = make_inputs(cfg, step=1, device="cpu")
    assert not torch.equal(a["q"], c["q"])


def test_blur_makes_neighbours_correlated_and_clusters_scale_keys():
    cfg = dataclasses.replace(CONFIGS["small"], heads=2, frames=4, clusters=3)
    x = make_inputs(cfg, device="cpu")
    q = x["q"].float()[0, 0].reshape(4, 32, 32, 64)
    corr = float((q[:, :, 1:] * q[:, :, :-1]).mean() / (q * q).mean())
    assert corr > 0.5            # sigma=1 smoothing correlates adjacent tokens strongly
    assert x["q"].dtype == torch.bfloat16 and x["k_lr"].dtype == torch.bfloat16
    base = dataclasses.replace(cfg, clusters=0)
    y = make_inputs(base, device="cpu")
    diff = (x["k"].float() - y["k"].float()).abs().sum(-1)[0]
    changed = int((diff > 0).sum())
    assert 32 <= changed <= 2 * 3 * 32   # 3 blocks of 2x4x4 tokens per head, may overlap

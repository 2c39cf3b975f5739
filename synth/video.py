"""Seeded generator of video-token attention inputs.

Recipe (all draws come from torch generators seeded from `seed = 1000*index + step`, one
independent sub-stream per component so that adding a component never shifts another):

* Q, K, V: per (b, h, channel) an iid N(0,1) field on the (T, Hh, W) token grid, smoothed by a
  separable Gaussian of sigma = 1 token along t, h and w (7 taps, +-3 sigma, normalised,
  reflect boundary without edge repeat), then the whole tensor is divided by its standard
  deviation (unit variance).
* Salient key clusters (Small: 8 per head, Mid/Long/Training: 16): a random 2x4x4 token block
  and a random unit direction u per cluster; the block's keys get their component along u
  multiplied by 3 (K += 2 (K.u) u). Blocks may overlap; clusters are applied in draw order.
* Q_lr, K_lr: iid integers uniform on [-7, 7] (exactly representable in fp32 and bf16).
* dO: iid N(0,1) ("iid") or the same blurred, renormalised field as Q/K/V ("blur").
* Long: per-head k drawn iid uniformly from {2,5,10,20}% of S, k = round(p*S).
Values are produced in fp32 and stored in the workload dtype (bf16 by round-to-nearest-even).
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional

import torch

from .configs import Workload

_SUB = {"q": 1, "k": 2, "v": 3, "do": 4, "q_lr": 5, "k_lr": 6, "clusters": 7, "kdraw": 8}


def _gen(seed: int, comp: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 64 + _SUB[comp])
    return g


def _gauss_taps(sigma: float = 1.0, radius: int = 3) -> List[float]:
    w = [math.exp(-0.5 * (t / sigma) ** 2) for t in range(-radius, radius + 1)]
    s = sum(w)
    return [x / s for x in w]


def _blur_axis(x: torch.Tensor, dim: int, taps: List[float]) -> torch.Tensor:
    """Separable 1-D smoothing along `dim` with reflect padding (x[-1] = x[1])."""
    r = len(taps) // 2
    n = x.shape[dim]
    if n == 1:
        return x
    # reflect index map (x[-1] = x[1]), folded repeatedly for grids shorter than the taps
    period = 2 * (n - 1)

    def fold(i):
        j = i % period
        return period - j if j >= n else j

    idx = [fold(i) for i in range(-r, n + r)]
    idx_t = torch.tensor(idx, device=x.device)
    xp = x.index_select(dim, idx_t)
    out = torch.zeros_like(x)
    for t, w in enumerate(taps):
        out.add_(xp.narrow(dim, t, n), alpha=w)
    return out


def blurred_field(shape, T: int, Hh: int, W: int, gen: torch.Generator, device) -> torch.Tensor:
    """[B, H, S, d] fp32 field, smoothed over (t, h, w) and renormalised to unit variance."""
    B, H, S, d = shape
    x = torch.randn((B, H, T, Hh, W, d), generator=gen, device=device, dtype=torch.float32)
    taps = _gauss_taps()
    for dim in (2, 3, 4):
        x = _blur_axis(x, dim, taps)
    x = x.reshape(B, H, S, d)
    x /= x.std()
    return x


def plant_clusters(k: torch.Tensor, cfg: Workload, gen: torch.Generator) -> None:
    """In place: scale the component of K along a random unit direction by 3 on random blocks."""
    if cfg.clusters <= 0:
        return
    B, H, S, d = k.shape
    bt, bh, bw = cfg.cluster_block
    T, Hh, W = cfg.frames, cfg.height, cfg.width
    kv = k.view(B, H, T, Hh, W, d)
    dev = k.device
    n = B * H * cfg.clusters
    t0 = torch.randint(0, T - bt + 1, (n,), generator=gen, device=dev).tolist()
    y0 = torch.randint(0, Hh - bh + 1, (n,), generator=gen, device=dev).tolist()
    x0 = torch.randint(0, W - bw + 1, (n,), generator=gen, device=dev).tolist()
    u = torch.randn((n, d), generator=gen, device=dev, dtype=torch.float32)
    u = u / u.norm(dim=1, keepdim=True)
    c = 0
    for b in range(B):
        for h in range(H):
            for _ in range(cfg.clusters):
                blk = kv[b, h, t0[c]:t0[c] + bt, y0[c]:y0[c] + bh, x0[c]:x0[c] + bw, :]
                proj = (blk * u[c]).sum(-1, keepdim=True)
                blk.add_(2.0 * proj * u[c])
                c += 1


def draw_k_per_head(cfg: Workload, seed: int) -> List[int]:
    S = cfg.seq
    ku = cfg.k_uniform()
    if ku is not None:
        return [ku] * cfg.heads
    g = _gen(seed, "kdraw", "cpu")
    ch = torch.randint(0, len(cfg.k_choices), (cfg.heads,), generator=g).tolist()
    return [int(round(cfg.k_choices[c] * S)) for c in ch]


def group_members_count(cfg: Workload) -> int:
    return cfg.group_size


def storage_dtype(cfg: Workload) -> torch.dtype:
    return torch.float32 if cfg.dtype == "fp32" else torch.bfloat16


def make_inputs(cfg: Workload, step: int = 0, device="cpu", backward: Optional[bool] = None,
                seed: Optional[int] = None) -> Dict[str, object]:
    """Draw one batch of inputs for `cfg` on `device`; tensors are in the storage dtype."""
    if seed is None:
        seed = 1000 * cfg.index + step
    if backward is None:
        backward = cfg.backward
    B, H, S, d, r = cfg.batch, cfg.heads, cfg.seq, cfg.head_dim, cfg.rank
    T, Hh, W = cfg.frames, cfg.height, cfg.width
    dt = storage_dtype(cfg)
    out: Dict[str, object] = {"seed": seed, "device": str(device), "config": cfg.name}
    q = blurred_field((B, H, S, d), T, Hh, W, _gen(seed, "q", device), device)
    out["q"] = q.to(dt)
    del q
    k = blurred_field((B, H, S, d), T, Hh, W, _gen(seed, "k", device), device)
    plant_clusters(k, cfg, _gen(seed, "clusters", device))
    out["k"] = k.to(dt)
    del k
    v = blurred_field((B, H, S, d), T, Hh, W, _gen(seed, "v", device), device)
    out["v"] = v.to(dt)
    del v
    glr = _gen(seed, "q_lr", device)
    out["q_lr"] = torch.randint(-7, 8, (B, H, S, r), generator=glr, device=device).to(dt)
    glr = _gen(seed, "k_lr", device)
    out["k_lr"] = torch.randint(-7, 8, (B, H, S, r), generator=glr, device=device).to(dt)
    if backward:
        if cfg.do_law == "blur":
            do = blurred_field((B, H, S, d), T, Hh, W, _gen(seed, "do", device), device)
        else:
            do = torch.randn((B, H, S, d), generator=_gen(seed, "do", device), device=device,
                             dtype=torch.float32)
        out["do"] = do.to(dt)
        del do
    out["k_per_head"] = draw_k_per_head(cfg, seed)
    out["scale"] = 1.0 / math.sqrt(d)
    return out

"""The five synthetic video-token workloads.

Each is a latent video of T x Hh x W tokens (row-major t,h,w) with per-head low-rank factors
of rank r and query groups of gt x gh x gw adjacent tokens. The DSV summaries
(gist.science/{zh,pt,fr,ko}/paper/2502.07590, §1 and §4) describe video DiTs with 100k-520k
tokens per sample trained on UCF-101/WebVid/VideoGen/OpenVid; those datasets are not used
here: seeded random fields of these shapes stand in for them.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    index: int                 # seed base = 1000 * index + step
    batch: int
    heads: int
    frames: int
    height: int
    width: int
    head_dim: int
    rank: int
    group: Tuple[int, int, int]   # (gt, gh, gw)
    k_frac: Optional[float]       # fixed fraction of S (None: drawn per head)
    k_fixed: Optional[int]        # explicit k (Tiny prints k=128)
    k_choices: Tuple[float, ...] = ()   # per-head draw set (Long)
    dtype: str = "bf16"           # storage / compute dtype of Q,K,V,dO,Q_lr,K_lr
    clusters: int = 0             # planted salient key clusters per head
    cluster_block: Tuple[int, int, int] = (2, 4, 4)
    do_law: str = "iid"           # "iid" N(0,1) or "blur" (same generator as Q/K/V)
    backward: bool = True
    steps: int = 1                # Training: 20 seeded steps with fresh inputs
    note: str = ""

    @property
    def seq(self) -> int:
        return self.frames * self.height * self.width

    @property
    def group_size(self) -> int:
        gt, gh, gw = self.group
        return gt * gh * gw

    @property
    def n_groups(self) -> int:
        return self.seq // self.group_size

    def k_uniform(self) -> Optional[int]:
        if self.k_fixed is not None:
            return self.k_fixed
        if self.k_frac is not None:
            return int(round(self.k_frac * self.seq))
        return None


CONFIGS = {
    "tiny": Workload(
        name="tiny", index=0, batch=1, heads=2, frames=4, height=16, width=16,
        head_dim=64, rank=16, group=(2, 2, 4), k_frac=None, k_fixed=128, dtype="fp32",
        clusters=0, backward=False,
        note="S=1024, 2 heads, d=64, r=16, group 2x2x4, k=128 (12.5%), fp32, forward only"),
    "small": Workload(
        name="small", index=1, batch=1, heads=16, frames=16, height=32, width=32,
        head_dim=64, rank=16, group=(4, 4, 4), k_frac=0.10, k_fixed=None, dtype="bf16",
        clusters=8, do_law="iid",
        note="S=16384, 16 heads, d=64, r=16, group 4x4x4, k=1638 (10%), bf16, fwd+bwd"),
    "mid": Workload(
        name="mid", index=2, batch=1, heads=24, frames=16, height=64, width=64,
        head_dim=128, rank=32, group=(4, 4, 4), k_frac=0.10, k_fixed=None, dtype="bf16",
        clusters=16, do_law="iid",
        note="S=65536, 24 heads, d=128, r=32, group 4x4x4, k=6554 (10%), bf16, fwd+bwd"),
    "long": Workload(
        name="long", index=3, batch=1, heads=16, frames=32, height=64, width=64,
        head_dim=128, rank=32, group=(4, 4, 4), k_frac=None, k_fixed=None,
        k_choices=(0.02, 0.05, 0.10, 0.20), dtype="bf16", clusters=16, backward=False,
        note="S=131072, 16 heads, d=128, r=32, per-head k in {2,5,10,20}% of S, bf16, fwd"),
    "training": Workload(
        name="training", index=4, batch=2, heads=24, frames=16, height=48, width=80,
        head_dim=128, rank=32, group=(4, 4, 4), k_frac=0.05, k_fixed=None, dtype="bf16",
        clusters=16, do_law="blur", steps=20,
        note="2 x S=61440, 24 heads, d=128, r=32, group 4x4x4, k=3072 (5%), bf16, "
             "topk+fwd+bwd, 20 seeded steps"),
}


def get_config(name: str) -> Workload:
    return CONFIGS[name]

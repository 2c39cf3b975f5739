"""Seeded synthetic video-token workloads for the DSV hot path.

This package only draws inputs (random fields, planted clusters, integer low-rank factors,
per-head k). It contains none of the method's arithmetic, and both the HIP path and the
CPU oracle consume what it produces.
"""
from .configs import CONFIGS, Workload, get_config  # noqa: F401
from .video import make_inputs, draw_k_per_head, group_members_count  # noqa: F401

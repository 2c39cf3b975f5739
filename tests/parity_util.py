"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI binding and the
oracle on the same seeded inputs. Nothing here computes any part of the method."""
from __future__ import annotations

import dataclasses
import math
import sys

import numpy as np

import dynamic_sparse_attention_rank_amd as dsv
from oracle import attention as oatt
from oracle import geometry as ogeo
from oracle import topk as otopk
from synth import CONFIGS, make_inputs

TOL = {"fp32": 1e-3, "bf16": 2e-2}   # max-abs-err bars for outputs and gradients


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def workload(name="small", **kw):
    return dataclasses.replace(CONFIGS[name], **kw)


def members(cfg) -> np.ndarray:
    return ogeo.group_members(cfg.frames, cfg.height, cfg.width, *cfg.group)


def gpu_inputs(cfg, step=0, backward=None, k_per_head=None):
    x = make_inputs(cfg, step=step, device="cuda", backward=backward)
    if k_per_head is not None:
        x["k_per_head"] = list(k_per_head)
    return x


def run_topk(cfg, x):
    p = dsv.problem_for(cfg)
    return dsv.lowrank_topk(p, x["q_lr"], x["k_lr"], x["k_per_head"])


def oracle_rows(cfg, x, b, h, mem=None):
    mem = members(cfg) if mem is None else mem
    sig = otopk.group_scores_bruteforce(f64(x["q_lr"][b, h]), f64(x["k_lr"][b, h]), mem)
    return otopk.topk_rows_by_sort(sig, int(x["k_per_head"][h]))


def gpu_rows(cfg, x, idx, b, h):
    p = dsv.problem_for(cfg)
    return dsv.idx_rows(idx, p, x["k_per_head"], b, h).cpu().numpy()


def characterise_all_rows(cfg, x, idx, b, h, mem=None) -> int:
    """Number of rows of (b, h) that fail the exact top-k characterisation
    (oracle.topk.topk_rows_are_exact on sum-first scores, which the CPU tests pin to the
    brute-force definition; the integer scores are held as int32, exactly)."""
    mem = members(cfg) if mem is None else mem
    sig = otopk.group_scores_sum_first(f64(x["q_lr"][b, h]), f64(x["k_lr"][b, h]), mem)
    if np.all(sig == np.round(sig)) and np.abs(sig).max() < 2 ** 31:
        sig = sig.astype(np.int32)
    rows = gpu_rows(cfg, x, idx, b, h)
    kh = int(x["k_per_head"][h])
    return int(np.count_nonzero(~otopk.topk_rows_are_exact(sig, rows, kh)))


def run_fwd(cfg, x, idx):
    p = dsv.problem_for(cfg)
    return dsv.sparse_attn_fwd(p, x["q"], x["k"], x["v"], idx, x["k_per_head"], x["scale"])


def run_bwd(cfg, x, idx, o, lse):
    p = dsv.problem_for(cfg)
    return dsv.sparse_attn_bwd(p, x["q"], x["k"], x["v"], o, x["do"], lse, idx,
                               x["k_per_head"], x["scale"])


def oracle_fwd(cfg, x, rows, b, h, groups=None, mem=None):
    mem = members(cfg) if mem is None else mem
    return oatt.gathered_forward(f64(x["q"][b, h]), f64(x["k"][b, h]), f64(x["v"][b, h]), mem,
                                 rows, x["scale"], groups=groups)


def oracle_bwd(cfg, x, rows, b, h, groups=None, mem=None):
    mem = members(cfg) if mem is None else mem
    return oatt.gathered_backward(f64(x["q"][b, h]), f64(x["k"][b, h]), f64(x["v"][b, h]),
                                  f64(x["do"][b, h]), mem, rows, x["scale"], groups=groups)


def adaptive_band(S: int) -> float:
    """Absolute band on the prefix sums within which dsv_adaptive_k may decide differently from
    the exact rule (include/dsv.h): twice the per-sum bound of its fixed-point weights, plus
    fp64 roundings of sums of at most S weights <= 1, with a wide margin."""
    P = 62 - int(S).bit_length()
    return 2.0 * (S * 2.0 ** -(P + 1) + 2.0 ** -P) + S * 2.0 ** -46


def maxerr(a, b) -> float:
    a = np.asarray(a)
    b = np.asarray(b)
    ok = ~np.isnan(b)
    return float(np.max(np.abs(a[ok] - b[ok]))) if ok.any() else 0.0

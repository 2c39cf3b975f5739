"""Benchmark of the DSV hot path on one MI355X.

One step = the whole hot path on one batch of synthetic video tokens already resident in
HBM: dsv_lowrank_topk (fused low-rank group scoring + exact top-k), dsv_sparse_attn_fwd and
dsv_sparse_attn_bwd. Default workload: the 16x64x64-token video (S = 65,536), 24 heads,
d = 128, r = 32, 4x4x4 query groups, k = 6,554 (10%), bf16.

Prints one JSON line. `value` is the selected-KV attention TFLOP/s of the whole step
(fwd + bwd FLOPs over the step time, top-k time included); the per-op times, the attention-only
and dense-equivalent rates, the top-k time, the dominant kernel's roofline and the oracle's
rate on the host cores are reported beside it.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK = {"bf16_mfma_tflops": 2500.0, "fp32_mfma_tflops": 157.3, "hbm_gbs": 8000.0}


def flops(cfg, ks):
    """Algorithmic FLOPs: forward 4*S*k*d per (b,h) (two GEMMs), backward 2.5x (five GEMMs)."""
    S, d, B = cfg.seq, cfg.head_dim, cfg.batch
    fwd = 4.0 * B * S * d * sum(ks)
    dense_fwd = 4.0 * B * cfg.heads * S * S * d
    return fwd, 2.5 * fwd, dense_fwd, 2.5 * dense_fwd


def topk_units(cfg, ks):
    """Top-k algorithmic work: one exact group score per (group, key) and the bytes it must
    move: K_lr and Q_lr once, idx written once."""
    B, H, S, r = cfg.batch, cfg.heads, cfg.seq, cfg.rank
    esz = 4 if cfg.dtype == "fp32" else 2
    scores = B * H * cfg.n_groups * S
    bytes_ = 2 * B * H * S * r * esz + 4 * B * cfg.n_groups * sum(ks)
    return scores, bytes_


def cpu_baseline(cfg, x, idx_rows_h0, seconds=12.0):
    """The oracle, as it is, on a bounded sample: groups of (b=0, h=0), timed on host cores."""
    import numpy as np
    from oracle import attention as oatt
    from oracle import geometry as ogeo
    from oracle import topk as otopk

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    mem = ogeo.group_members(cfg.frames, cfg.height, cfg.width, *cfg.group)
    f64 = lambda t: t.detach().float().cpu().double().numpy()  # noqa: E731
    qlr, klr = f64(x["q_lr"][0, 0]), f64(x["k_lr"][0, 0])
    q, k, v, do = (f64(x[n][0, 0]) for n in ("q", "k", "v", "do"))
    kh = int(x["k_per_head"][0])
    rows = idx_rows_h0
    t0 = time.perf_counter()
    n = 0
    while True:
        g = n
        sig = otopk.group_scores_bruteforce(qlr, klr, mem[g:g + 1])
        otopk.topk_rows_by_sort(sig, kh)
        oatt.gathered_forward(q, k, v, mem, rows, x["scale"], groups=[g])
        oatt.gathered_backward(q, k, v, do, mem, rows, x["scale"], groups=[g])
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or n >= cfg.n_groups:
            break
    sel_flops = 3.5 * 4.0 * cfg.group_size * kh * cfg.head_dim * n
    return {"value": sel_flops / el / 1e12, "unit": "TFLOP/s (selected-KV fwd+bwd, top-k incl.)",
            "cores": int(threads), "kind": "oracle",
            "sample": f"{n} query groups of head 0 (of {cfg.batch * cfg.heads * cfg.n_groups}): "
                      f"brute-force group scores + full sort, gathered fp64 fwd + bwd; "
                      f"{el:.1f} s on {threads} BLAS threads"}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="mid")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the DSV hot path is measured on one GPU's share "
              "of the work (no sharding or collectives in this build); use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import dynamic_sparse_attention_rank_amd as dsv
    from synth import CONFIGS, make_inputs

    cfg = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"generating {cfg.name} inputs on {dev}")
    x = make_inputs(cfg, step=0, device=dev, backward=True)
    ks = x["k_per_head"]
    p = dsv.problem_for(cfg)
    shp = (cfg.batch, cfg.heads, cfg.seq, cfg.head_dim)
    dt = torch.float32 if cfg.dtype == "fp32" else torch.bfloat16
    idx = torch.zeros(dsv.idx_elems(p, ks), dtype=torch.int32, device=dev)
    o = torch.empty(shp, dtype=dt, device=dev)
    lse = torch.empty(shp[:3], dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty(shp, dtype=torch.float32, device=dev) for _ in range(3))
    # the backward's minimum workspace covers one (b, h) slot; four slots per launch
    ws_n = dsv.workspace_bytes(dsv.DSV_OP_BWD, p, ks) * min(4, cfg.batch * cfg.heads)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        dsv.lowrank_topk(p, x["q_lr"], x["k_lr"], ks, idx=idx, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        dsv.sparse_attn_fwd(p, x["q"], x["k"], x["v"], idx, ks, x["scale"], o=o, lse=lse,
                            stream=stream)
        if ev is not None:
            ev[2].record(stream)
        dsv.sparse_attn_bwd(p, x["q"], x["k"], x["v"], o, x["do"], lse, idx, ks, x["scale"],
                            dq=dq, dk=dk, dv=dv, ws=ws, stream=stream)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps); timing {args.steps} steps")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    t_topk = [e[0].elapsed_time(e[1]) for e in evs]
    t_fwd = [e[1].elapsed_time(e[2]) for e in evs]
    t_bwd = [e[2].elapsed_time(e[3]) for e in evs]
    mean = lambda a: sum(a) / len(a)  # noqa: E731
    med = lambda a: sorted(a)[len(a) // 2]  # noqa: E731
    f_fwd, f_bwd, fd_fwd, fd_bwd = flops(cfg, ks)
    ms_attn = mean(t_fwd) + mean(t_bwd)
    sel_step = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12
    sel_attn = (f_fwd + f_bwd) / (ms_attn * 1e-3) / 1e12
    dense_attn = (fd_fwd + fd_bwd) / (ms_attn * 1e-3) / 1e12
    scores, tk_bytes = topk_units(cfg, ks)

    kernels = {
        "lowrank_topk": {"ms_mean": mean(t_topk), "ms_median": med(t_topk),
                         "scores_per_s": scores / (mean(t_topk) * 1e-3),
                         "hbm_gbs_algorithmic": tk_bytes / (mean(t_topk) * 1e-3) / 1e9},
        "sparse_attn_fwd": {"ms_mean": mean(t_fwd), "ms_median": med(t_fwd),
                            "tflops": f_fwd / (mean(t_fwd) * 1e-3) / 1e12},
        "sparse_attn_bwd": {"ms_mean": mean(t_bwd), "ms_median": med(t_bwd),
                            "tflops": f_bwd / (mean(t_bwd) * 1e-3) / 1e12,
                            "note": "call = per chunk of (b,h) slots: bucket count + scan + "
                                    "backward kernel + bucket reduce"},
    }
    dom = max(kernels, key=lambda kname: kernels[kname]["ms_mean"])
    peak = PEAK["bf16_mfma_tflops"] if cfg.dtype == "bf16" else PEAK["fp32_mfma_tflops"]
    if dom == "lowrank_topk":
        ach = tk_bytes / (kernels[dom]["ms_mean"] * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": ach, "peak": PEAK["hbm_gbs"],
                "unit": "GB/s", "frac": ach / PEAK["hbm_gbs"], "traffic": None}
    else:
        fl = f_fwd if dom == "sparse_attn_fwd" else f_bwd
        ach = fl / (kernels[dom]["ms_mean"] * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": ach, "peak": peak,
                "unit": "TFLOP/s", "frac": ach / peak, "traffic": None}

    out = {
        "metric": "sparse attn fwd+bwd TFLOP/s (selected-KV & dense-equiv) + top-k ms, S=64K",
        "value": sel_step,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded blurred video-token fields, integer low-rank factors)",
        "config": {"workload": cfg.name, "batch": cfg.batch, "heads": cfg.heads,
                   "grid": [cfg.frames, cfg.height, cfg.width], "seq_len": cfg.seq,
                   "head_dim": cfg.head_dim, "rank": cfg.rank, "group": list(cfg.group),
                   "k_per_head": sorted(set(ks)), "parallelism": "single GPU"},
        "selected_tflops_attn": sel_attn,
        "dense_equiv_tflops_attn": dense_attn,
        "topk_ms": mean(t_topk),
        "fwd_ms": mean(t_fwd),
        "bwd_ms": mean(t_bwd),
        "kernels": kernels,
        "roofline": roof,
        "cpu_baseline": None,
    }
    log(f"timed: {ms_step:.3f} ms/step (top-k {mean(t_topk):.3f}, fwd {mean(t_fwd):.3f}, "
        f"bwd {mean(t_bwd):.3f} ms)")
    if not args.no_cpu_baseline:
        log(f"oracle on host cores for ~{args.cpu_seconds:.0f} s")
        rows = dsv.idx_rows(idx, p, ks, 0, 0).cpu().numpy()
        out["cpu_baseline"] = cpu_baseline(cfg, x, rows, seconds=args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the DSV hot path on one MI355X.

One step = the whole hot path on one batch of synthetic video tokens already resident in
HBM: dsv_lowrank_topk (fused low-rank group scoring + exact top-k), dsv_sparse_attn_fwd and,
for the workloads with a backward, dsv_sparse_attn_bwd. Workloads (--config):
  mid       (default) 16x64x64 tokens (S = 65,536), 24 heads, d = 128, r = 32, 4x4x4 groups,
            k = 6,554 (10%), bf16: top-k + fwd + bwd;
  small     16x32x32 tokens, 16 heads, d = 64, r = 16, k = 1,638: top-k + fwd + bwd;
  long      32x64x64 tokens (S = 131,072), 16 heads, per-head k drawn from {2,5,10,20}% of S:
            top-k + fwd (selection and attention timed apart), heads launched in the
            planner's order; the planner's placement over 8 parts is also timed part by part;
  training  2 x 16x48x80 tokens, 24 heads, k = 5%: top-k + fwd + bwd, every step on fresh
            inputs (all of them generated before the timed region);
  tiny      4x16x16 tokens, 2 heads, fp32, forward only.

Prints one JSON line. `value` is the selected-KV attention TFLOP/s of the whole step (the
step's attention FLOPs over the step time, top-k time included); per-op times, attention-only
and dense-equivalent rates, per-kernel times, the dominant kernel's roofline, the top-k
against its own roofline and the oracle's rate on the host cores are reported beside it.

Timing: HIP events on the launch stream around every op (torch events) and, inside the
backward, around every head chunk's stages (raw hipEvent_t handles passed to
dsv_sparse_attn_bwd_profiled), so each kernel's average launch duration is measured live.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published peaks; the integer VALU rate is 256 CUs x 64 lanes x 2.4 GHz
PEAK = {"bf16_mfma_tflops": 2500.0, "fp32_mfma_tflops": 157.3, "hbm_gbs": 8000.0,
        "valu_tops": 39.3}
METRIC = "sparse attn fwd+bwd TFLOP/s (selected-KV & dense-equiv) + top-k ms, S=64K"


def flops(cfg, ks):
    """Algorithmic FLOPs: forward 4*S*k*d per (b,h) (two GEMMs), backward 2.5x (five GEMMs)."""
    S, d, B = cfg.seq, cfg.head_dim, cfg.batch
    fwd = 4.0 * B * S * d * sum(ks)
    dense_fwd = 4.0 * B * cfg.heads * S * S * d
    return fwd, 2.5 * fwd, dense_fwd, 2.5 * dense_fwd


def n_edges(cfg, ks):
    """(group, selected key) pairs of the whole batch."""
    return cfg.batch * cfg.n_groups * sum(ks)


def bwd_stage_bytes(cfg, ks, share8=0.0):
    """HBM bytes of the staged backward design per step (backward kernel, reduce).

    A staged edge writes a dV row and a dK row: d bytes each as 8-bit codes (the share share8
    of the rows) or 2d bytes each in fp16, plus block factors, E/2 bytes. Backward kernel (per
    (b,h) slot, E = NG*k edges): the staging rows and factors, idx reads, 4E, Q, K, V, O and dO
    read once, 10*S*d, LSE, 4*S, and dQ written once, 4*S*d. Reduce: staging rows and factors
    read once, its edge list, 4E, dK and dV written once, 8*S*d."""
    B, S, d, NG = cfg.batch, cfg.seq, cfg.head_dim, cfg.n_groups
    row = share8 * 2 * d + (1.0 - share8) * 4 * d + 0.5
    k1 = red = 0
    for kh in ks:
        E = NG * kh
        k1 += B * (E * row + 4 * E + 10 * S * d + 4 * S + 4 * S * d)
        red += B * (E * row + 4 * E + 8 * S * d)
    return k1, red


def staged_8bit_share(p, cfg, ks, xi, o, lse, idx):
    """Share of the backward's staging rows written as 8-bit codes, read from the block factor
    table (sign bit set: 8-bit) that a backward with a one-slot workspace leaves for its last
    slot (the last in launch order). Layout as pinned by the ABI tests; None for the fp32 path."""
    import torch

    import dynamic_sparse_attention_rank_amd as dsv
    if cfg.dtype != "bf16":
        return None
    need = dsv.workspace_bytes(dsv.DSV_OP_BWD, p, ks)
    ws = torch.zeros(need, dtype=torch.uint8, device=o.device)
    dsv.sparse_attn_bwd(p, xi["q"], xi["k"], xi["v"], o, xi["do"], lse, idx, ks, xi["scale"],
                        ws=ws)
    torch.cuda.synchronize()
    al = lambda v: -(-v // 256) * 256  # noqa: E731
    NG, nb = cfg.n_groups, -(-cfg.seq // 32)
    pad = lambda k: -(-k // 32) * 32  # noqa: E731
    e = NG * pad(max(ks))
    off = 2 * al(NG * (nb + 1) * 4) + 2 * al((nb + 1) * 4) + al(e * 4)
    last = dsv.plan_order(list(ks))[-1]
    blocks = NG * pad(ks[last]) // 16
    fac = ws[off:off + e // 16 * 8].view(torch.float32).view(-1, 2)[:blocks, 0]
    return float(torch.signbit(fac).float().mean())


def topk_roofline(cfg, ks):
    """The selection's roofline: one exact score per (group, key), the bytes it must move
    (Q_lr and K_lr once, idx written once) and the MFMA work of the score tiles (two bf16
    terms per group sum); its time is the largest of the three at the chip's peaks."""
    B, H, S, r = cfg.batch, cfg.heads, cfg.seq, cfg.rank
    esz = 4 if cfg.dtype == "fp32" else 2
    scores = B * H * cfg.n_groups * S
    nbytes = 2 * B * H * S * r * esz + 4 * B * cfg.n_groups * sum(ks)
    mfma = 2.0 * r * scores * (1 if cfg.dtype == "fp32" else 2)
    mpeak = PEAK["fp32_mfma_tflops"] if cfg.dtype == "fp32" else PEAK["bf16_mfma_tflops"]
    t = {"hbm": nbytes / (PEAK["hbm_gbs"] * 1e9), "alu": scores / (PEAK["valu_tops"] * 1e12),
         "mfma": mfma / (mpeak * 1e12)}
    bound = max(t, key=t.get)
    return {"scores": scores, "bytes": nbytes, "bound": bound, "ms": t[bound] * 1e3,
            "ms_hbm": t["hbm"] * 1e3, "ms_alu": t["alu"] * 1e3, "ms_mfma": t["mfma"] * 1e3}


def hip_events(n):
    """n raw hipEvent_t handles (timing enabled) from the HIP runtime libdsv uses."""
    import dynamic_sparse_attention_rank_amd as dsv
    L = dsv.lib()
    L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    L.hipEventCreate.restype = ctypes.c_int
    out = []
    for _ in range(n):
        e = ctypes.c_void_p()
        if L.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        out.append(e.value)
    return out


def hip_elapsed_ms(a, b):
    import dynamic_sparse_attention_rank_amd as dsv
    L = dsv.lib()
    L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                      ctypes.c_void_p]
    L.hipEventElapsedTime.restype = ctypes.c_int
    ms = ctypes.c_float()
    if L.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
        raise RuntimeError("hipEventElapsedTime failed")
    return ms.value


def hip_destroy(evs):
    import dynamic_sparse_attention_rank_amd as dsv
    L = dsv.lib()
    L.hipEventDestroy.argtypes = [ctypes.c_void_p]
    for e in evs:
        L.hipEventDestroy(e)


def kernel_sources_sha256(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "dynamic_sparse_attention_rank_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_summary(kernel, workload, launches):
    """The kernel's block of the committed rocprofv3 counter summary
    profiles/counters_<workload>.txt as a dict, or None if there is none, its sources have
    changed since, or it was taken with another number of launches per step."""
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals, cur = {}, None
    for line in open(path):
        line = line.strip()
        if line.startswith("kernel:"):
            cur = line.split(":", 1)[1].strip()
            vals[cur] = {}
        elif cur and ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            vals[cur][key.strip()] = val.strip()
    v = vals.get(kernel)
    if not v or v.get("sources_sha256") != kernel_sources_sha256(v.get("sources", "").split()):
        return None
    if int(v.get("launches_per_step", -1)) != launches:
        return None
    return v


def counter_traffic(kernel, workload, launches):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated) from the counter summary."""
    v = counter_summary(kernel, workload, launches)
    if not v or "fetch_bytes_per_launch" not in v:
        return None
    return float(v["fetch_bytes_per_launch"]) + float(v["write_bytes_per_launch"])


def cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = None
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return {"os_cpu_count": os.cpu_count(), "affinity": aff, "blas_threads": blas}


def cpu_baseline(cfg, x, rows_h0, backward, seconds=12.0):
    """The oracle, as it is, on a bounded sample of the workload: query groups of (b=0, h=0),
    top-k (brute-force group scores + full sort), forward and backward (gathered fp64) each
    timed on their own share of the budget, then scaled to the whole workload."""
    import numpy as np
    from oracle import attention as oatt
    from oracle import geometry as ogeo
    from oracle import topk as otopk

    thr = cpu_threads()
    mem = ogeo.group_members(cfg.frames, cfg.height, cfg.width, *cfg.group)
    f64 = lambda t: t.detach().float().cpu().double().numpy()  # noqa: E731
    qlr, klr = f64(x["q_lr"][0, 0]), f64(x["k_lr"][0, 0])
    q, k, v = (f64(x[n][0, 0]) for n in ("q", "k", "v"))
    do = f64(x["do"][0, 0]) if backward else None
    kh = int(x["k_per_head"][0])
    groups_total = cfg.batch * cfg.heads * cfg.n_groups
    parts = ["topk", "fwd"] + (["bwd"] if backward else [])
    budget = seconds / len(parts)

    def timed(fn):
        t0 = time.perf_counter()
        n = 0
        while n < cfg.n_groups:
            fn(n)
            n += 1
            if time.perf_counter() - t0 >= budget:
                break
        return n, time.perf_counter() - t0

    out = {}
    n, el = timed(lambda g: otopk.topk_rows_by_sort(
        otopk.group_scores_bruteforce(qlr, klr, mem[g:g + 1]), kh))
    out["topk"] = {"groups": n, "s": el, "ms_whole_workload": el / n * groups_total * 1e3}
    n, el = timed(lambda g: oatt.gathered_forward(q, k, v, mem, rows_h0, x["scale"],
                                                  groups=[g]))
    fl = 4.0 * cfg.group_size * kh * cfg.head_dim
    out["fwd"] = {"groups": n, "s": el, "tflops": fl * n / el / 1e12}
    if backward:
        n, el = timed(lambda g: oatt.gathered_backward(q, k, v, do, mem, rows_h0, x["scale"],
                                                       groups=[g]))
        out["bwd"] = {"groups": n, "s": el, "tflops": 2.5 * fl * n / el / 1e12}
    # the whole workload at these rates: top-k time plus attention time (FLOPs / rate)
    f_fwd, f_bwd, _, _ = flops(cfg, x["k_per_head"])
    t_all = out["topk"]["ms_whole_workload"] * 1e-3 + f_fwd / (out["fwd"]["tflops"] * 1e12)
    sel = f_fwd
    if backward:
        t_all += f_bwd / (out["bwd"]["tflops"] * 1e12)
        sel += f_bwd
    return {"value": sel / t_all / 1e12,
            "unit": "TFLOP/s (selected-KV attention of the step, top-k time included)",
            "cores": thr["blas_threads"] or thr["affinity"] or thr["os_cpu_count"],
            "kind": "oracle", "threads": thr, "parts": out,
            "sample": f"query groups of head 0 (of {groups_total} in the workload): "
                      f"brute-force group scores + full sort ({out['topk']['groups']} groups), "
                      f"gathered fp64 forward ({out['fwd']['groups']})"
                      + (f" and backward ({out['bwd']['groups']})" if backward else "")
                      + f", about {budget:.0f} s each, scaled to the whole workload"}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 10; training: 20, one fresh input set each)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="mid", choices=["tiny", "small", "mid", "long",
                                                         "training"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the measurements outside the step (MAX top-k, adaptive k, plans)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run one plain fp32 copy kernel of this many MiB (read "
                         "and written once): the reference for scaling HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the DSV hot path is measured on one GPU's share "
              "of the work (the library has no sharded path and makes no collective calls); "
              "use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import dynamic_sparse_attention_rank_amd as dsv
    from synth import CONFIGS, make_inputs

    cfg = CONFIGS[args.config]
    fresh = cfg.steps > 1                       # training: fresh inputs every step
    steps = args.steps if args.steps is not None else (cfg.steps if fresh else 10)
    backward = cfg.backward
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n_sets = steps if fresh else 1
    log(f"generating {cfg.name} inputs on {dev} ({n_sets} set(s))")
    xs = [make_inputs(cfg, step=i, device=dev, backward=backward) for i in range(n_sets)]
    x = xs[0]
    ks = x["k_per_head"]
    p = dsv.problem_for(cfg)
    shp = (cfg.batch, cfg.heads, cfg.seq, cfg.head_dim)
    dt = torch.float32 if cfg.dtype == "fp32" else torch.bfloat16
    idx = torch.empty(dsv.idx_elems(p, ks), dtype=torch.int32, device=dev)
    o = torch.empty(shp, dtype=dt, device=dev)
    lse = torch.empty(shp[:3], dtype=torch.float32, device=dev)
    staged = backward and cfg.dtype == "bf16"   # per-stage backward events: bf16 path
    nch = 0
    if backward:
        dq, dk, dv = (torch.empty(shp, dtype=torch.float32, device=dev) for _ in range(3))
        # The backward's minimum workspace covers one (b, h) slot. Room for every slot lets one
        # launch take them all, which leaves one tail per kernel instead of one per launch:
        # against launches of two slots, 0.6 ms less per step at S = 64K (24 slots, 87 GB) and
        # 2.5 ms at 2 x 61440 (48 slots, 75 GB). Capped at a third of the device's memory.
        one_slot = dsv.workspace_bytes(dsv.DSV_OP_BWD, p, ks)
        cap = torch.cuda.get_device_properties(dev).total_memory // 3
        # (one slot more than the slots: the per-slot tables and row capacity round up)
        ws_n = one_slot * max(1, min(cfg.batch * cfg.heads + 1, cap // max(one_slot, 1)))
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)
        nch = dsv.bwd_chunks(p, ks, ws.numel()) if staged else 0
    stage_ev = hip_events(4 * nch * steps) if staged else []
    stream = torch.cuda.current_stream()

    def step(xi, ev=None, sev=None):
        if ev is not None:
            ev[0].record(stream)
        dsv.lowrank_topk(p, xi["q_lr"], xi["k_lr"], ks, idx=idx, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        dsv.sparse_attn_fwd(p, xi["q"], xi["k"], xi["v"], idx, ks, xi["scale"], o=o, lse=lse,
                            stream=stream)
        if ev is not None:
            ev[2].record(stream)
        if backward:
            dsv.sparse_attn_bwd(p, xi["q"], xi["k"], xi["v"], o, xi["do"], lse, idx, ks,
                                xi["scale"], dq=dq, dk=dk, dv=dv, ws=ws, stream=stream,
                                events=sev)
        if ev is not None:
            ev[3].record(stream)

    for i in range(args.warmup):
        step(xs[i % n_sets])
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps); timing {steps} steps")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(xs[i % n_sets], evs[i], stage_ev[4 * nch * i:4 * nch * (i + 1)] if staged else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / steps
    t_topk = [e[0].elapsed_time(e[1]) for e in evs]
    t_fwd = [e[1].elapsed_time(e[2]) for e in evs]
    t_bwd = [e[2].elapsed_time(e[3]) for e in evs]
    mean = lambda a: sum(a) / len(a)  # noqa: E731
    med = lambda a: sorted(a)[len(a) // 2]  # noqa: E731
    f_fwd, f_bwd, fd_fwd, fd_bwd = flops(cfg, ks)
    if not backward:
        f_bwd = fd_bwd = 0.0
    ms_attn = mean(t_fwd) + (mean(t_bwd) if backward else 0.0)
    sel_step = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12
    sel_attn = (f_fwd + f_bwd) / (ms_attn * 1e-3) / 1e12
    dense_attn = (fd_fwd + fd_bwd) / (ms_attn * 1e-3) / 1e12
    E = n_edges(cfg, ks)
    row2 = 2 * cfg.head_dim * (4 if cfg.dtype == "fp32" else 2)   # gathered K + V row bytes
    tk = topk_roofline(cfg, ks)
    peak = PEAK["bf16_mfma_tflops"] if cfg.dtype == "bf16" else PEAK["fp32_mfma_tflops"]
    fwd_name = "attn_fwd_bf16" if cfg.dtype == "bf16" else "attn_fwd_f32"

    # per-kernel table: launches per step, average launch duration, per-step total and the
    # algorithmic work of one average launch with the roofline it is held to: sparse attention
    # against MFMA over 4*G*d (fwd) and 10*G*d (bwd) FLOPs per edge, the top-k against its
    # roofline time (topk_roofline), the reduce against HBM over its staged bytes
    kernels = {
        "topk_kernel": {"op": "dsv_lowrank_topk", "launches_per_step": 1,
                        "ms_per_launch": mean(t_topk), "ms_median": med(t_topk),
                        "bound": tk["bound"], "roofline_ms": tk["ms"],
                        "scores_per_s": tk["scores"] / (mean(t_topk) * 1e-3)},
        fwd_name: {"op": "dsv_sparse_attn_fwd", "launches_per_step": 1,
                   "ms_per_launch": mean(t_fwd), "ms_median": med(t_fwd), "bound": "mfma",
                   "units_per_launch": f_fwd},
    }
    if staged:
        pre, p1, red = [], [], []
        for i in range(steps):
            e = stage_ev[4 * nch * i:4 * nch * (i + 1)]
            for c in range(nch):
                pre.append(hip_elapsed_ms(e[4 * c], e[4 * c + 1]))
                p1.append(hip_elapsed_ms(e[4 * c + 1], e[4 * c + 2]))
                red.append(hip_elapsed_ms(e[4 * c + 2], e[4 * c + 3]))
        # the last step's inputs, which idx, o and lse still hold (an extra backward: skipped
        # with --no-extras, as in the profiling runs; the reduce is then priced as fp16 rows)
        share8 = (None if args.no_extras else
                  staged_8bit_share(p, cfg, ks, xs[(steps - 1) % n_sets], o, lse, idx))
        _, b2 = bwd_stage_bytes(cfg, ks, share8 or 0.0)
        kernels["attn_bwd_bf16"] = {"op": "dsv_sparse_attn_bwd", "launches_per_step": nch,
                                    "ms_per_launch": mean(p1), "ms_median": med(p1),
                                    "bound": "mfma", "units_per_launch": f_bwd / nch}
        kernels["bucket_reduce"] = {"op": "dsv_sparse_attn_bwd", "launches_per_step": nch,
                                    "ms_per_launch": mean(red), "ms_median": med(red),
                                    "bound": "hbm", "units_per_launch": b2 / nch,
                                    "staged_8bit_share": share8,
                                    "note": "bytes of the staged design: rows (8-bit codes "
                                            "or fp16) and block factors read once"}
        kernels["bwd_index_prepasses"] = {
            "op": "dsv_sparse_attn_bwd", "launches_per_step": nch, "ms_per_launch": mean(pre),
            "ms_median": med(pre), "bound": None,
            "note": "row_bucket_starts + transpose_rs + bucket_totals + bucket_offsets + "
                    "bucket_perm"}
        hip_destroy(stage_ev)
    elif backward:
        kernels["attn_bwd_f32"] = {"op": "dsv_sparse_attn_bwd", "launches_per_step": 1,
                                   "ms_per_launch": mean(t_bwd), "ms_median": med(t_bwd),
                                   "bound": "mfma", "units_per_launch": f_bwd}
    for kn, kv in kernels.items():
        kv["ms_per_step"] = kv["ms_per_launch"] * kv["launches_per_step"]
        sec = kv["ms_per_launch"] * 1e-3
        if "roofline_ms" in kv:   # the top-k: its roofline time over its measured time
            kv["frac"] = kv["roofline_ms"] / kv["ms_per_launch"]
        elif kv["bound"] == "mfma":
            kv["tflops"] = kv["units_per_launch"] / sec / 1e12
            kv["frac"] = kv["tflops"] / peak
        elif kv["bound"] == "hbm":
            kv["gbs"] = kv["units_per_launch"] / sec / 1e9
            kv["frac"] = kv["gbs"] / PEAK["hbm_gbs"]
    dom = max((kn for kn in kernels if kernels[kn]["bound"]),
              key=lambda kn: kernels[kn]["ms_per_step"])
    kd = kernels[dom]
    sec = kd["ms_per_launch"] * 1e-3
    if "roofline_ms" in kd:   # the top-k: the roofline's own unit
        roof = {"kernel": dom, "bound": kd["bound"], "achieved": tk["ms"] / kd["frac"],
                "peak": tk["ms"], "unit": "ms", "frac": kd["frac"]}
    elif kd["bound"] == "mfma":
        roof = {"kernel": dom, "bound": "mfma", "achieved": kd["tflops"], "peak": peak,
                "unit": "TFLOP/s", "frac": kd["frac"],
                "per_unit": "4*G*d FLOPs per edge (fwd), 10*G*d (bwd)",
                "units_per_launch": kd["units_per_launch"]}
    else:
        roof = {"kernel": dom, "bound": "hbm", "achieved": kd["gbs"], "peak": PEAK["hbm_gbs"],
                "unit": "GB/s", "frac": kd["frac"], "units_per_launch": kd["units_per_launch"]}
    roof["traffic"] = counter_traffic(dom, cfg.name, kd["launches_per_step"])
    cs = counter_summary(dom, cfg.name, kd["launches_per_step"])
    if cs:
        roof["counters"] = {k2: float(v2) for k2, v2 in cs.items()
                            if k2.endswith(("_pct", "_gbs"))}
        if roof["traffic"] is not None:
            roof["counters"]["hbm_gbs"] = roof["traffic"] / sec / 1e9

    out = {
        "metric": METRIC,
        "value": sel_step,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded blurred video-token fields, integer low-rank factors)"
                + ("; fresh inputs every step" if fresh else ""),
        "config": {"workload": cfg.name, "batch": cfg.batch, "heads": cfg.heads,
                   "grid": [cfg.frames, cfg.height, cfg.width], "seq_len": cfg.seq,
                   "head_dim": cfg.head_dim, "rank": cfg.rank, "group": list(cfg.group),
                   "k_per_head": list(ks), "ops": "topk+fwd" + ("+bwd" if backward else ""),
                   "parallelism": "single GPU"},
        "selected_tflops_attn": sel_attn,
        "dense_equiv_tflops_attn": dense_attn,
        "mfma_frac_attn": sel_attn / peak,
        "topk_ms": mean(t_topk),
        "topk_roofline": {**tk, "frac": tk["ms"] / mean(t_topk)},
        "fwd_ms": mean(t_fwd),
        "bwd_ms": mean(t_bwd) if backward else None,
        "gather": {"bytes_per_edge": row2, "fwd_gbs": row2 * E / (mean(t_fwd) * 1e-3) / 1e9},
        "kernels": kernels,
        "bwd_chunks": nch,
        "bwd_workspace_gb": (ws.numel() / 1e9) if backward else None,
        "roofline": roof,
        "cpu_baseline": None,
    }
    if backward:
        out["gather"]["bwd_gbs"] = row2 * E / (mean(t_bwd) * 1e-3) / 1e9
        # the cross-group dK/dV sum: 2*d fp32 values per edge; the whole backward against
        # that traffic at the HBM peak
        acc = 8.0 * cfg.head_dim * E
        out["bwd_byte_view"] = {"accumulation_bytes": acc,
                                "ms_at_hbm_peak": acc / (PEAK["hbm_gbs"] * 1e9) * 1e3,
                                "frac": acc / (PEAK["hbm_gbs"] * 1e9) / (mean(t_bwd) * 1e-3)}
    log(f"timed: {ms_step:.3f} ms/step (top-k {mean(t_topk):.3f}, fwd {mean(t_fwd):.3f}"
        + (f", bwd {mean(t_bwd):.3f}" if backward else "") + " ms)")

    extras = {}
    if not args.no_extras:
        extras = run_extras(args, cfg, p, x, ks, peak, tk, stream, dev)
    out["extras"] = extras
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)   # one elementwise kernel: n*4 bytes read, n*4 written
        torch.cuda.synchronize()
        log(f"calibration copy: {args.calib_copy_mib} MiB read + {args.calib_copy_mib} MiB "
            f"written by one kernel")
        del src, dst
    if not args.no_cpu_baseline:
        log(f"oracle on host cores for ~{args.cpu_seconds:.0f} s")
        # the rows of step 0's selection (the timed loop's last step may use other inputs)
        step(x)
        torch.cuda.synchronize()
        rows = dsv.idx_rows(idx, p, ks, 0, 0).cpu().numpy()
        out["cpu_baseline"] = cpu_baseline(cfg, x, rows, backward, seconds=args.cpu_seconds)
    print(json.dumps(out), flush=True)


def run_extras(args, cfg, p, x, ks, peak, tk, stream, dev):
    """Measurements outside the step, on the step's inputs but with buffers of their own."""
    import torch

    import dynamic_sparse_attention_rank_amd as dsv

    extras = {}

    def timed(fn, reps):
        fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(reps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    # the head placement the planner gives for this workload over 8 devices, with the
    # measured cost model (estimation per head + attention per unit of k)
    cm = dsv.default_cost_model(p, with_backward=cfg.backward)
    fixed = cfg.seq * p.n_groups * cm.topk_ns_per_score * 1e-6
    per_k = p.n_groups * cm.attn_ns_per_edge * 1e-6
    part, load, rho = dsv.plan_heads(ks, 8, fixed, per_k)
    kd_out, n_dense = dsv.dispatch_k(p, ks, cm)
    extras["head_plan_8"] = {"rho_s": rho, "max_load_ms": max(load), "part_of_head": part}
    extras["dispatch"] = {"dense_heads": n_dense,
                          "break_even_k_over_S": 1 - cm.topk_ns_per_score / cm.attn_ns_per_edge}
    if cfg.name == "long":
        extras["head_plan_8"].update(measure_plan(cfg, p, x, ks, part, stream, timed))
    if cfg.name != "mid":
        return extras

    # adaptive k on the same inputs
    kg = torch.empty((cfg.batch, cfg.heads, p.n_groups), dtype=torch.int32, device=dev)
    res = {}

    def ak():
        res["kh"] = dsv.adaptive_k(p, x["q_lr"], x["k_lr"], mass=0.9, k_group=kg,
                                   stream=stream)[0]
    ak_ms = timed(ak, 5)
    kh_t = res["kh"]
    extras["adaptive_k"] = {"ms": ak_ms, "mass": 0.9,
                            "scores_per_s": tk["scores"] / (ak_ms * 1e-3),
                            "k_head_min_max": [int(kh_t.min()), int(kh_t.max())]}
    # the MAX group reduction (the other reading of the group score), in its own idx buffer:
    # recomputing the member products in every selection pass (memory O(S*k), the fused
    # form), and with every slot's NG x S group scores kept in a workspace between passes
    idx_max = torch.empty(dsv.idx_elems(p, ks), dtype=torch.int32, device=dev)
    re_ms = timed(lambda: dsv.lowrank_topk(p, x["q_lr"], x["k_lr"], ks, idx=idx_max,
                                           reduce=dsv.DSV_GROUP_MAX, stream=stream), 2)
    cache_b = dsv.topk_max_cache_bytes(p) * cfg.batch * cfg.heads
    ws_max = torch.empty(cache_b, dtype=torch.uint8, device=dev)
    ca_ms = timed(lambda: dsv.lowrank_topk(p, x["q_lr"], x["k_lr"], ks, idx=idx_max,
                                           reduce=dsv.DSV_GROUP_MAX, stream=stream,
                                           ws=ws_max), 3)
    del ws_max, idx_max
    member_flop = 2.0 * cfg.batch * cfg.heads * cfg.seq * cfg.seq * cfg.rank   # S x S x r
    mx_tf = member_flop / (re_ms * 1e-3) / 1e12
    extras["topk_max"] = {
        "ms": re_ms, "memory": "O(S*k): member products recomputed in every selection pass",
        "member_score_tflops_per_pass": mx_tf,
        "ms_cached_scores": ca_ms, "cache_bytes": cache_b,
        "cached_note": "stores every slot's NG x S group scores in a caller workspace",
        # one S x S x r member-score product per pass over the keys
        "roofline": {"bound": "mfma", "peak": peak, "unit": "TFLOP/s",
                     "achieved_one_product": mx_tf, "frac_one_product": mx_tf / peak}}
    log(f"adaptive k: {ak_ms:.3f} ms; top-k with MAX: {re_ms:.3f} ms (recomputed), "
        f"{ca_ms:.3f} ms (scores cached)")
    return extras


def measure_plan(cfg, p, x, ks, part, stream, timed):
    """Head-parallel placement emulated on one GPU: each part's heads copied into tensors of
    their own and run (top-k + forward) as their own problem; measured part times give the
    measured imbalance ratio beside the planned one."""
    import torch

    import dynamic_sparse_attention_rank_amd as dsv

    n_parts = max(part) + 1
    ms = []
    for pi in range(n_parts):
        heads = [h for h in range(cfg.heads) if part[h] == pi]
        if not heads:
            ms.append(0.0)
            continue
        sub = {n: x[n][:, heads].contiguous() for n in ("q", "k", "v", "q_lr", "k_lr")}
        kp = [ks[h] for h in heads]
        pp = dsv.problem(cfg.batch, len(heads), cfg.frames, cfg.height, cfg.width,
                         cfg.head_dim, cfg.rank, cfg.group, cfg.dtype)
        idx = torch.empty(dsv.idx_elems(pp, kp), dtype=torch.int32, device=x["q"].device)

        def run():
            dsv.lowrank_topk(pp, sub["q_lr"], sub["k_lr"], kp, idx=idx, stream=stream)
            dsv.sparse_attn_fwd(pp, sub["q"], sub["k"], sub["v"], idx, kp, x["scale"],
                                stream=stream)
        ms.append(timed(run, 2))
        del sub, idx
    mean_ms = sum(ms) / len(ms)
    return {"measured_part_ms": ms, "measured_rho_s": max(ms) / mean_ms if mean_ms else None}


if __name__ == "__main__":
    main()

"""GPU parity: the HIP path through the C ABI against the oracle, element by element.

Bars: idx bit-exact; O, dQ, dK, dV within max-abs-err 1e-3 (fp32 path) / 2e-2 (bf16 path);
LSE within the same bar. Sizes are chosen so the oracle finishes in seconds while spanning
several tiles and a ragged tail."""
import numpy as np
import pytest
import torch

import dynamic_sparse_attention_rank_amd as dsv
from oracle import attention as oatt
from parity_util import (TOL, characterise_all_rows, f64, gpu_inputs, gpu_rows, maxerr,
                         members, oracle_bwd, oracle_fwd, oracle_rows, run_bwd, run_fwd,
                         run_topk, say, workload)

pytestmark = pytest.mark.gpu


# --------------------------------------------------------------------------------- top-k
@pytest.mark.parametrize("name", ["tiny", "small"])
def test_topk_bit_exact_full_config(name):
    cfg = workload(name)
    say(f"[topk] {name}")
    x = gpu_inputs(cfg, backward=False)
    idx = run_topk(cfg, x)
    torch.cuda.synchronize()
    mem = members(cfg)
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            ref = oracle_rows(cfg, x, b, h, mem)
            got = gpu_rows(cfg, x, idx, b, h)
            assert np.array_equal(got, ref), (b, h, np.argwhere(got != ref)[:5])


TOPK_CASES = [
    # (label, overrides, k_per_head)
    ("k1", dict(heads=2, frames=4, height=8, width=8, group=(2, 2, 4), rank=32), [1, 1]),
    ("kS", dict(heads=2, frames=2, height=8, width=8, group=(2, 2, 4), rank=32), [128, 128]),
    ("ragged-k", dict(heads=3, frames=4, height=8, width=12, group=(2, 2, 4), rank=32),
     [7, 45, 100]),
    ("G32-r48", dict(heads=2, frames=4, height=8, width=16, group=(2, 4, 4), rank=48), [33, 60]),
    ("G48-r64", dict(heads=2, frames=3, height=8, width=16, group=(3, 4, 4), rank=64), [50, 9]),
    ("NG36", dict(heads=2, frames=4, height=12, width=12, group=(2, 2, 4), rank=16), [71, 200]),
    ("fp32-r32", dict(heads=2, frames=4, height=8, width=8, group=(2, 2, 4), rank=32,
                      dtype="fp32"), [19, 64]),
    ("fp32-r48", dict(heads=1, frames=4, height=8, width=8, group=(1, 4, 4), rank=48,
                      dtype="fp32"), [100]),
    # dense heads (k = S: every key, no scoring) next to sparse ones in one call
    ("mixed-dense", dict(heads=3, frames=4, height=8, width=8, group=(2, 2, 4), rank=32),
     [256, 40, 256]),
    ("fp32-dense", dict(heads=2, frames=4, height=8, width=8, group=(2, 2, 4), rank=16,
                        dtype="fp32"), [3, 256]),
]


@pytest.mark.parametrize("label,over,ks", TOPK_CASES, ids=[c[0] for c in TOPK_CASES])
def test_topk_edge_cases_bit_exact(label, over, ks):
    cfg = workload("small", **over)
    say(f"[topk-edge] {label}")
    x = gpu_inputs(cfg, backward=False, k_per_head=ks)
    idx = run_topk(cfg, x)
    torch.cuda.synchronize()
    for h in range(cfg.heads):
        assert np.array_equal(gpu_rows(cfg, x, idx, 0, h), oracle_rows(cfg, x, 0, h)), h


def test_topk_all_ties_takes_lowest_indices():
    cfg = workload("small", heads=1, frames=4, height=8, width=8, group=(2, 2, 4), rank=32)
    x = gpu_inputs(cfg, backward=False, k_per_head=[37])
    x["q_lr"].zero_()
    idx = run_topk(cfg, x)
    rows = gpu_rows(cfg, x, idx, 0, 0)
    assert np.array_equal(rows, np.tile(np.arange(37), (rows.shape[0], 1)))


def _sampled_key_mask(S):
    """Keys of the tiles the top-k samples for its threshold window: 8 tiles of 512 keys, tile
    j * (S // 512 // 8) (include/dsv.h: selection by a sampled window, radix otherwise)."""
    nfull = S // 512
    ns = min(8, nfull)
    mask = np.zeros(S, dtype=bool)
    for j in range(ns):
        t = j * (nfull // ns)
        mask[512 * t:512 * (t + 1)] = True
    return mask


def test_topk_window_misses_fall_back_to_radix():
    """Sampled key tiles unrepresentative (their K_lr rows zero, scores 0) so the threshold
    window misses for groups with nonzero sums; groups whose Q_lr is zero (all scores tie at
    0) resolve in the window. Both kinds of row bit-exact against the oracle."""
    cfg = workload("small", heads=2)
    say("[topk] window misses -> radix passes")
    x = gpu_inputs(cfg, backward=False, k_per_head=[1638, 200])
    mask = torch.from_numpy(_sampled_key_mask(cfg.seq)).to(x["k_lr"].device)
    x["k_lr"][:, :, mask, :] = 0
    mem = torch.from_numpy(members(cfg)).to(x["q_lr"].device)
    for g in range(0, cfg.n_groups, 5):   # every fifth group: all its scores tie at 0
        x["q_lr"][:, :, mem[g], :] = 0
    idx = run_topk(cfg, x)
    torch.cuda.synchronize()
    for h in range(cfg.heads):
        assert np.array_equal(gpu_rows(cfg, x, idx, 0, h), oracle_rows(cfg, x, 0, h)), h


def test_topk_half_integer_scores_verify_and_retry():
    """Half-integer K_lr entries make scores that share a one-unit window bin without being
    equal: the window's count check fails and the rows are redone by the radix passes. The
    scores are still exact (multiples of 1/2), so the rows are compared bit for bit."""
    cfg = workload("small", heads=2, frames=8, height=16, width=16)
    say("[topk] half-integer scores -> verified retry")
    x = gpu_inputs(cfg, backward=False, k_per_head=[256, 61])
    g = torch.Generator(device=x["k_lr"].device)
    g.manual_seed(5)
    half = torch.rand(x["k_lr"].shape, generator=g, device=x["k_lr"].device) < 0.3
    x["k_lr"] = torch.where(half, x["k_lr"] + 0.5, x["k_lr"]).contiguous()
    idx = run_topk(cfg, x)
    torch.cuda.synchronize()
    for h in range(cfg.heads):
        assert np.array_equal(gpu_rows(cfg, x, idx, 0, h), oracle_rows(cfg, x, 0, h)), h


def test_topk_repeatable_bitwise():
    cfg = workload("small", heads=4)
    x = gpu_inputs(cfg, backward=False)
    a = run_topk(cfg, x).clone()
    b = run_topk(cfg, x)
    assert torch.equal(a, b)
    assert characterise_all_rows(cfg, x, b, 0, 3) == 0


# ------------------------------------------------------------------------------- forward
def _fwd_check(cfg, x, idx, heads=None, groups=None):
    o, lse = run_fwd(cfg, x, idx)
    torch.cuda.synchronize()
    tol = TOL[cfg.dtype]
    mem = members(cfg)
    worst = 0.0
    for b in range(cfg.batch):
        for h in (range(cfg.heads) if heads is None else heads):
            rows = gpu_rows(cfg, x, idx, b, h)
            ro, rl = oracle_fwd(cfg, x, rows, b, h, groups=groups, mem=mem)
            eo = maxerr(f64(o[b, h]), ro)
            el = maxerr(f64(lse[b, h]), rl)
            worst = max(worst, eo, el)
            assert eo <= tol and el <= tol, (b, h, eo, el)
    say(f"   worst max-abs-err {worst:.3e} (bar {tol})")
    return o, lse


def test_fwd_tiny_fp32_vs_dense_oracle():
    cfg = workload("tiny")
    say("[fwd] tiny fp32")
    x = gpu_inputs(cfg, backward=False)
    idx = run_topk(cfg, x)
    o, lse = run_fwd(cfg, x, idx)
    torch.cuda.synchronize()
    mem = members(cfg)
    for h in range(cfg.heads):
        rows = gpu_rows(cfg, x, idx, 0, h)
        ro, rl, _ = oatt.dense_masked_forward(f64(x["q"][0, h]), f64(x["k"][0, h]),
                                              f64(x["v"][0, h]), mem, rows, x["scale"])
        assert maxerr(f64(o[0, h]), ro) <= 1e-3
        assert maxerr(f64(lse[0, h]), rl) <= 1e-3


def test_fwd_small_bf16_all_groups():
    cfg = workload("small")
    say("[fwd] small bf16")
    x = gpu_inputs(cfg, backward=False)
    idx = run_topk(cfg, x)
    _fwd_check(cfg, x, idx)


FWD_CASES = [
    ("bf16-d128-G64", dict(heads=2, frames=4, height=16, width=16, head_dim=128, rank=32),
     [300, 77]),
    ("bf16-d64-G16", dict(heads=2, frames=4, height=16, width=16, group=(2, 2, 4)), [1, 45]),
    ("bf16-d128-G32", dict(heads=2, frames=4, height=8, width=16, group=(2, 4, 4),
                           head_dim=128, rank=32), [33, 512]),
    ("bf16-d64-G48-kS", dict(heads=1, frames=3, height=8, width=16, group=(3, 4, 4)), [384]),
    ("fp32-d128-G64", dict(heads=2, frames=4, height=8, width=8, head_dim=128, rank=32,
                           dtype="fp32"), [17, 256]),
    ("fp32-d64-G16-k1", dict(heads=1, frames=4, height=8, width=8, group=(2, 2, 4),
                             dtype="fp32"), [1]),
    # the remaining (head dim, query blocks) instances of the bf16 kernel
    ("bf16-d128-G16", dict(heads=2, frames=4, height=8, width=16, group=(2, 2, 4),
                           head_dim=128, rank=32), [70, 129]),
    ("bf16-d128-G48", dict(heads=1, frames=3, height=8, width=16, group=(3, 4, 4),
                           head_dim=128, rank=32), [95]),
    ("bf16-d64-G32", dict(heads=2, frames=2, height=8, width=16, group=(2, 4, 4)), [31, 200]),
    # the remaining (head dim, query blocks) instances of the fp32 MFMA kernel
    ("fp32-d128-G16", dict(heads=1, frames=4, height=8, width=8, group=(2, 2, 4),
                           head_dim=128, rank=32, dtype="fp32"), [45]),
    ("fp32-d128-G32", dict(heads=1, frames=4, height=8, width=8, group=(2, 4, 4),
                           head_dim=128, rank=32, dtype="fp32"), [100]),
    ("fp32-d128-G48", dict(heads=1, frames=3, height=8, width=16, group=(3, 4, 4),
                           head_dim=128, rank=32, dtype="fp32"), [31]),
    ("fp32-d64-G32", dict(heads=2, frames=2, height=8, width=16, group=(2, 4, 4),
                          dtype="fp32"), [16, 256]),
    ("fp32-d64-G48", dict(heads=1, frames=3, height=8, width=16, group=(3, 4, 4),
                          dtype="fp32"), [200]),
    ("fp32-d64-G64", dict(heads=1, frames=4, height=8, width=16, dtype="fp32"), [77]),
]


@pytest.mark.parametrize("label,over,ks", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_fwd_edge_cases(label, over, ks):
    cfg = workload("small", **over)
    say(f"[fwd-edge] {label}")
    x = gpu_inputs(cfg, backward=False, k_per_head=ks)
    idx = run_topk(cfg, x)
    o, lse = _fwd_check(cfg, x, idx)
    if ks[0] == 1:   # one key: O is that key's V row (stored dtype)
        rows = gpu_rows(cfg, x, idx, 0, 0)
        mem = members(cfg)
        for g in range(rows.shape[0]):
            ref = f64(x["v"][0, 0, rows[g, 0]])
            assert np.max(np.abs(f64(o[0, 0, mem[g]]) - ref)) <= TOL[cfg.dtype]


def test_fwd_repeatable_bitwise():
    cfg = workload("small", heads=4)
    x = gpu_inputs(cfg, backward=False)
    idx = run_topk(cfg, x)
    o1, l1 = run_fwd(cfg, x, idx)
    o1, l1 = o1.clone(), l1.clone()
    o2, l2 = run_fwd(cfg, x, idx)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ------------------------------------------------------------------------------ backward
def _bwd_check(cfg, x, idx, heads=None):
    o, lse = run_fwd(cfg, x, idx)
    dq, dk, dv = run_bwd(cfg, x, idx, o, lse)
    torch.cuda.synchronize()
    tol = TOL[cfg.dtype]
    worst = 0.0
    mem = members(cfg)
    for b in range(cfg.batch):
        for h in (range(cfg.heads) if heads is None else heads):
            rows = gpu_rows(cfg, x, idx, b, h)
            rq, rk, rv = oracle_bwd(cfg, x, rows, b, h, mem=mem)
            e = (maxerr(f64(dq[b, h]), rq), maxerr(f64(dk[b, h]), rk), maxerr(f64(dv[b, h]), rv))
            worst = max(worst, *e)
            assert max(e) <= tol, (b, h, e)
            # unselected keys receive exactly zero
            unsel = np.setdiff1d(np.arange(cfg.seq), np.unique(rows))
            if unsel.size:
                assert not dk[b, h, unsel].any() and not dv[b, h, unsel].any()
    say(f"   worst max-abs-err {worst:.3e} (bar {tol})")
    return dq, dk, dv


def test_bwd_tiny_shape_fp32():
    cfg = workload("tiny")
    say("[bwd] tiny fp32")
    x = gpu_inputs(cfg, backward=True)
    idx = run_topk(cfg, x)
    _bwd_check(cfg, x, idx)


def test_bwd_fp32_repeatable_bitwise():
    """fp32 dK/dV are summed as fixed-point integers: the same bits on every run, although
    the groups' atomics land in whatever order the scheduling gives."""
    cfg = workload("tiny", heads=2, head_dim=128, rank=32, k_fixed=256)
    say("[bwd] fp32 repeatable")
    x = gpu_inputs(cfg, backward=True)
    idx = run_topk(cfg, x)
    o, lse = run_fwd(cfg, x, idx)
    first = [t.clone() for t in run_bwd(cfg, x, idx, o, lse)]
    for _ in range(3):
        again = run_bwd(cfg, x, idx, o, lse)
        assert all(torch.equal(a, b) for a, b in zip(first, again))


def test_bwd_small_bf16_all_heads():
    cfg = workload("small")
    say("[bwd] small bf16")
    x = gpu_inputs(cfg, backward=True)
    idx = run_topk(cfg, x)
    dq, dk, dv = _bwd_check(cfg, x, idx)
    # sum rules per (b, h): sum_m dV_m = sum_n dO_n, sum_m dK_m = 0
    s_dv = dv.double().sum(dim=2)
    s_do = x["do"].double().sum(dim=2)
    assert float((s_dv - s_do).abs().max()) < 0.5
    assert float(dk.double().sum(dim=2).abs().max()) < 0.5


BWD_CASES = [
    ("bf16-d128-G64", dict(heads=2, frames=4, height=16, width=16, head_dim=128, rank=32),
     [300, 77]),
    ("bf16-d64-G16", dict(heads=2, frames=4, height=16, width=16, group=(2, 2, 4)), [1, 45]),
    ("bf16-d128-G48", dict(heads=1, frames=3, height=8, width=16, group=(3, 4, 4),
                           head_dim=128, rank=32), [100]),
    ("bf16-d64-G32-kS", dict(heads=1, frames=2, height=8, width=16, group=(2, 4, 4)), [256]),
    ("fp32-d128-G64", dict(heads=2, frames=4, height=8, width=8, head_dim=128, rank=32,
                           dtype="fp32"), [17, 256]),
    ("fp32-d64-G32-k1", dict(heads=1, frames=4, height=8, width=8, group=(2, 4, 4),
                             dtype="fp32"), [1]),
    # the remaining (head dim, query blocks) instances of the bf16 kernel
    ("bf16-d128-G16", dict(heads=2, frames=4, height=8, width=16, group=(2, 2, 4),
                           head_dim=128, rank=32), [70, 129]),
    ("bf16-d128-G32", dict(heads=2, frames=4, height=8, width=16, group=(2, 4, 4),
                           head_dim=128, rank=32), [33, 257]),
    ("bf16-d64-G48", dict(heads=1, frames=3, height=8, width=16, group=(3, 4, 4)), [130]),
    # the remaining (head dim, query blocks) instances of the fp32 MFMA kernel
    ("fp32-d128-G16", dict(heads=1, frames=4, height=8, width=8, group=(2, 2, 4),
                           head_dim=128, rank=32, dtype="fp32"), [45]),
    ("fp32-d128-G32", dict(heads=2, frames=4, height=8, width=8, group=(2, 4, 4),
                           head_dim=128, rank=32, dtype="fp32"), [100, 31]),
    ("fp32-d128-G48", dict(heads=1, frames=3, height=8, width=16, group=(3, 4, 4),
                           head_dim=128, rank=32, dtype="fp32"), [33]),
    ("fp32-d64-G16", dict(heads=1, frames=4, height=8, width=8, group=(2, 2, 4),
                          dtype="fp32"), [256]),
    ("fp32-d64-G48", dict(heads=1, frames=3, height=8, width=16, group=(3, 4, 4),
                          dtype="fp32"), [200]),
    ("fp32-d64-G64", dict(heads=1, frames=4, height=8, width=16, dtype="fp32"), [77]),
]


@pytest.mark.parametrize("label,over,ks", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_bwd_edge_cases(label, over, ks):
    cfg = workload("small", **over)
    say(f"[bwd-edge] {label}")
    x = gpu_inputs(cfg, backward=True, k_per_head=ks)
    idx = run_topk(cfg, x)
    dq, dk, dv = _bwd_check(cfg, x, idx)
    if ks[0] == 1:   # a single key per group: dQ = dK = 0
        assert float(dq[0, 0].abs().max()) <= TOL[cfg.dtype]
        assert float(dk[0, 0].abs().max()) <= TOL[cfg.dtype]


def test_bwd_mixed_staging_formats():
    """d = 128: 16-key blocks whose largest dV (dK: after the softmax scale) entry is at most
    0.125 are staged in 8 bits, the others in fp16. At k = 1400 of 4096 keys about 95% of
    head 1's dV blocks take 8 bits, so one launch holds both kinds (read back from the block
    factor table of the workspace: sign bit set = 8-bit) and the reduce runs its mixed steps;
    every output still meets the bf16 bar against the oracle."""
    cfg = workload("small", heads=2, frames=4, height=32, width=32, head_dim=128, rank=32)
    say("[bwd] mixed staging formats")
    x = gpu_inputs(cfg, backward=True, k_per_head=[2048, 1400])
    idx = run_topk(cfg, x)
    p = dsv.problem_for(cfg)
    o, lse = dsv.sparse_attn_fwd(p, x["q"], x["k"], x["v"], idx, x["k_per_head"], x["scale"])
    need = dsv.workspace_bytes(dsv.DSV_OP_BWD, p, x["k_per_head"])
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")   # one slot per chunk
    dq, dk, dv = dsv.sparse_attn_bwd(p, x["q"], x["k"], x["v"], o, x["do"], lse, idx,
                                     x["k_per_head"], x["scale"], ws=ws)
    torch.cuda.synchronize()
    # the last chunk's block factors (layout pinned in test_abi): heads run heaviest k first,
    # so the last chunk is head 1 (k = 1400, 44 chunks = 88 blocks per group)
    al = lambda v: -(-v // 256) * 256
    NG, nb = p.n_groups, -(-p.seq // 32)
    e = NG * (-(-max(x["k_per_head"]) // 32) * 32)
    off = 2 * al(NG * (nb + 1) * 4) + 2 * al((nb + 1) * 4) + al(e * 4)
    fac = ws[off:off + e // 16 * 8].view(torch.float32).view(-1, 2).cpu()
    neg = torch.signbit(fac[:NG * 88, 0])
    say(f"   8-bit blocks of head 1: {float(neg.float().mean()):.2f}")
    assert bool(neg.any()) and bool((~neg).any()), float(neg.float().mean())
    tol = TOL[cfg.dtype]
    mem = members(cfg)
    for h in range(cfg.heads):
        rows = gpu_rows(cfg, x, idx, 0, h)
        rdq, rdk, rdv = oracle_bwd(cfg, x, rows, 0, h, mem=mem)
        e3 = (maxerr(dq[0, h].cpu().numpy(), rdq), maxerr(dk[0, h].cpu().numpy(), rdk),
              maxerr(dv[0, h].cpu().numpy(), rdv))
        say(f"   head {h}: max-abs-err dQ {e3[0]:.2e} dK {e3[1]:.2e} dV {e3[2]:.2e}")
        assert max(e3) <= tol, (h, e3)


def test_bwd_profiled_matches_plain_bitwise():
    """dsv_sparse_attn_bwd_profiled does the same work: bitwise-equal dQ/dK/dV, and its stage
    events are ordered on the stream."""
    import ctypes
    import torch
    cfg = workload("small", heads=4)
    say("[bwd] profiled entry point, small x 4 heads")
    x = gpu_inputs(cfg, backward=True)
    idx = run_topk(cfg, x)
    o, lse = run_fwd(cfg, x, idx)
    p = dsv.problem_for(cfg)
    ks = x["k_per_head"]
    need = dsv.workspace_bytes(dsv.DSV_OP_BWD, p, ks)
    ws = torch.empty(2 * need, dtype=torch.uint8, device="cuda")
    nch = dsv.bwd_chunks(p, ks, ws.numel())
    assert nch >= 2
    ref = dsv.sparse_attn_bwd(p, x["q"], x["k"], x["v"], o, x["do"], lse, idx, ks, ws=ws)
    ref = [t.clone() for t in ref]
    L = dsv.lib()
    L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                      ctypes.c_void_p]
    L.hipEventDestroy.argtypes = [ctypes.c_void_p]
    evs = []
    for _ in range(4 * nch):
        e = ctypes.c_void_p()
        assert L.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    got = dsv.sparse_attn_bwd(p, x["q"], x["k"], x["v"], o, x["do"], lse, idx, ks, ws=ws,
                              events=evs)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    ms = ctypes.c_float()
    for i in range(len(evs) - 1):
        assert L.hipEventElapsedTime(ctypes.byref(ms), evs[i], evs[i + 1]) == 0
        assert ms.value >= 0.0
    for e in evs:
        L.hipEventDestroy(e)


def test_malformed_index_rows_are_memory_safe():
    """Index rows with keys outside [0, S), a repeated key and a descending row: the forward
    follows the clamped lists as listed (against the oracle on the clamped rows, repeats
    counted twice), dQ of the well-formed and the reordered rows matches the oracle, and every
    output (dK/dV are unspecified for such lists) is finite."""
    cfg = workload("small", heads=2, frames=4, height=16, width=16, head_dim=128, rank=32)
    say("[malformed idx] keys out of range, repeated, descending")
    x = gpu_inputs(cfg, backward=True, k_per_head=[100, 77])
    idx = run_topk(cfg, x)
    torch.cuda.synchronize()
    p = dsv.problem_for(cfg)
    S, k0 = cfg.seq, x["k_per_head"][0]
    h_idx = idx.cpu().numpy().copy()
    off0 = dsv.idx_row_offset(p, x["k_per_head"], 0, 0, 0)
    row = lambda g: slice(off0 + g * k0, off0 + (g + 1) * k0)
    h_idx[row(0)][[3, 10, k0 - 1]] = [-5, S + 7, 2**31 - 1]   # out of range
    h_idx[row(1)][20:30] = h_idx[row(1)][20]                    # one key ten times
    h_idx[row(2)] = h_idx[row(2)][::-1].copy()                  # descending
    bad = torch.from_numpy(h_idx).to(idx.device)
    o, lse = run_fwd(cfg, x, bad)
    dq, dk, dv = run_bwd(cfg, x, bad, o, lse)
    torch.cuda.synchronize()
    for t in (o, lse, dq, dk, dv):
        assert bool(torch.isfinite(t.float()).all())
    mem = members(cfg)
    for h in range(cfg.heads):
        # the kernels' clamp: any key outside [0, S), negative ones included, reads S - 1
        rows = gpu_rows(cfg, x, bad, 0, h).astype(np.int64)
        rows = np.where((rows < 0) | (rows >= S), S - 1, rows)
        ro, rl = oracle_fwd(cfg, x, rows, 0, h, mem=mem)   # any list: repeats count twice
        e = (maxerr(f64(o[0, h]), ro), maxerr(f64(lse[0, h]), rl))
        assert max(e) <= TOL[cfg.dtype], (h, e)
        # dQ does not depend on the order of a list: the descending row is checked in
        # ascending order; the rows with out-of-range or repeated keys only for finiteness
        groups = list(range(2 if h == 0 else 0, cfg.n_groups))
        rows[2] = np.sort(rows[2])
        rq, _, _ = oracle_bwd(cfg, x, rows, 0, h, groups=groups, mem=mem)
        tok = mem[groups].ravel()
        eq = maxerr(f64(dq[0, h])[tok], rq[tok])
        assert eq <= TOL[cfg.dtype], (h, eq)


def test_pipeline_on_a_side_stream_matches_the_current_stream():
    """The binding allocates its outputs and the backward's workspace on the launch stream:
    top-k, forward and backward launched on a side stream (default priority) give the same
    bits as on the current stream, while the current stream allocates and fills other memory
    meanwhile."""
    cfg = workload("small", heads=4)
    say("[stream] full pipeline on a side stream")
    x = gpu_inputs(cfg, backward=True)
    p = dsv.problem_for(cfg)
    ks = x["k_per_head"]

    def run(stream):
        idx = dsv.lowrank_topk(p, x["q_lr"], x["k_lr"], ks, stream=stream)
        o, lse = dsv.sparse_attn_fwd(p, x["q"], x["k"], x["v"], idx, ks, x["scale"],
                                     stream=stream)
        d = dsv.sparse_attn_bwd(p, x["q"], x["k"], x["v"], o, x["do"], lse, idx, ks,
                                x["scale"], stream=stream)
        return (idx, o, lse) + tuple(d)

    ref = run(None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got = run(side)
    # the current stream keeps allocating and writing while the side stream works
    junk = [torch.full((1 << 22,), 7.0, device="cuda") for _ in range(8)]
    del junk
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)

"""The no-allocation backward (dsv_sparse_attn_bwd_noalloc), called through the C ABI, against
the workspace entry point dsv_sparse_attn_bwd on the same inputs: the same bits on two calls
in a row, the second on a smaller problem (the shared scratch then holds the first call's
contents), no change in the device's free memory across the later calls, and the outputs
within the bar of the oracle; a third call runs the fp32 path on the same scratch."""
import ctypes

import pytest
import torch

import dynamic_sparse_attention_rank_amd as dsv
from parity_util import (TOL, f64, gpu_inputs, gpu_rows, maxerr, members, oracle_bwd, run_fwd,
                         run_topk, say, workload)

pytestmark = pytest.mark.gpu


def _free_bytes():
    L = dsv.lib()
    L.hipMemGetInfo.argtypes = [ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
    L.hipMemGetInfo.restype = ctypes.c_int
    free, total = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.hipMemGetInfo(ctypes.byref(free), ctypes.byref(total)) == 0
    return free.value


def _noalloc(p, x, o, lse, idx, ks, outs):
    L = dsv.lib()
    dq, dk, dv = outs
    return L.dsv_sparse_attn_bwd_noalloc(
        ctypes.byref(p), x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(), o.data_ptr(),
        x["do"].data_ptr(), lse.data_ptr(), idx.data_ptr(), dsv._kph(ks), float(x["scale"]),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
        torch.cuda.current_stream().cuda_stream)


CASES = [
    # (label, workload overrides, k per head): the first needs two head chunks of the scratch
    ("small-4heads", dict(heads=4), None),
    ("smaller-ragged", dict(heads=3, frames=4, height=16, width=16, head_dim=128, rank=32),
     [201, 77, 40]),
    # fp32: the scratch holds the fixed-point dV/dK accumulators instead
    ("fp32", dict(heads=2, frames=4, height=16, width=16, group=(2, 2, 4), dtype="fp32"),
     [128, 37]),
]


def test_noalloc_bwd_matches_workspace_entry_point_twice():
    for i, (label, over, ks) in enumerate(CASES):
        cfg = workload("small", **over)
        say(f"[no-alloc bwd] call {i + 1}: {label}")
        x = gpu_inputs(cfg, backward=True, k_per_head=ks)
        ks = x["k_per_head"]
        p = dsv.problem_for(cfg)
        need = dsv.workspace_bytes(dsv.DSV_OP_BWD, p, ks)
        assert 0 < need <= 256 * 1024 * 1024
        if i == 0:   # the heads take more than one chunk of the scratch
            assert dsv.bwd_chunks(p, ks, 256 * 1024 * 1024) >= 2
        idx = run_topk(cfg, x)
        o, lse = run_fwd(cfg, x, idx)
        ref = dsv.sparse_attn_bwd(p, x["q"], x["k"], x["v"], o, x["do"], lse, idx, ks,
                                  x["scale"])
        shp = (cfg.batch, cfg.heads, cfg.seq, cfg.head_dim)
        outs = [torch.full(shp, float("nan"), dtype=torch.float32, device="cuda")
                for _ in range(3)]
        torch.cuda.synchronize()
        free0 = _free_bytes()
        st = _noalloc(p, x, o, lse, idx, ks, outs)
        assert st == 0, dsv.last_error()
        torch.cuda.synchronize()
        if i > 0:   # after the first call on the device: nothing is allocated
            assert _free_bytes() == free0
        for a, b in zip(ref, outs):
            assert torch.equal(a, b)
        mem = members(cfg)
        rows = gpu_rows(cfg, x, idx, 0, 0)
        rq, rk, rv = oracle_bwd(cfg, x, rows, 0, 0, mem=mem)
        e = (maxerr(f64(outs[0][0, 0]), rq), maxerr(f64(outs[1][0, 0]), rk),
             maxerr(f64(outs[2][0, 0]), rv))
        say(f"   head 0 max-abs-err dq/dk/dv {e}")
        assert max(e) <= TOL[cfg.dtype], e

"""The C ABI on the CPU: the library loads, exports every declared symbol, validates
arguments before touching HIP, and agrees with the oracle on the packed index layout.
No compute call is made here."""
import ctypes
import os
import re

import numpy as np
import pytest

import dynamic_sparse_attention_rank_amd as dsv
from oracle import topk as otopk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsv_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = dsv.lib()
    names = declared_functions()
    assert {"dsv_lowrank_topk", "dsv_sparse_attn_fwd", "dsv_sparse_attn_bwd"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(dsv.EXPORTED)
    assert re.fullmatch(r"\d+\.\d+\.\d+", dsv.version())


def mid():
    return dsv.problem(1, 24, 16, 64, 64, 128, 32, (4, 4, 4), "bf16")


FAKE = 1 << 20   # a non-NULL, 16-byte aligned value; never dereferenced by validation


def test_validation_accepts_the_workloads():
    p = mid()
    assert dsv.validate(dsv.DSV_OP_TOPK, p, [6554] * 24, [FAKE] * 3) == 0
    assert dsv.validate(dsv.DSV_OP_FWD, p, [6554] * 24, [FAKE] * 6) == 0
    need = dsv.workspace_bytes(dsv.DSV_OP_BWD, p, [6554] * 24)
    assert dsv.validate(dsv.DSV_OP_BWD, p, [6554] * 24, [FAKE] * 10, ws_bytes=need) == 0
    tiny = dsv.problem(1, 2, 4, 16, 16, 64, 16, (2, 2, 4), "fp32")
    assert dsv.validate(dsv.DSV_OP_FWD, tiny, [128, 128], [FAKE] * 6) == 0


@pytest.mark.parametrize("mutate,code", [
    (lambda p: setattr(p, "gt", 3), "DSV_ERR_SHAPE"),
    (lambda p: setattr(p, "batch", 0), "DSV_ERR_SHAPE"),
    (lambda p: setattr(p, "dtype", 7), "DSV_ERR_DTYPE"),
    (lambda p: setattr(p, "head_dim", 96), "DSV_ERR_UNSUPPORTED"),
    (lambda p: setattr(p, "rank", 24), "DSV_ERR_UNSUPPORTED"),
    (lambda p: setattr(p, "gw", 8), "DSV_ERR_UNSUPPORTED"),     # G = 128
    (lambda p: setattr(p, "heads", 200), "DSV_ERR_UNSUPPORTED"),
])
def test_validation_rejects_bad_problems(mutate, code):
    p = mid()
    mutate(p)
    st = dsv.validate(dsv.DSV_OP_FWD, p, [6554] * max(p.heads, 1), [FAKE] * 6)
    assert dsv.STATUS[st] == code, dsv.last_error()
    assert dsv.last_error()


def test_validation_rejects_bad_k_pointers_and_reduce():
    p = mid()
    ks = [6554] * 24
    assert dsv.STATUS[dsv.validate(dsv.DSV_OP_FWD, p, [0] + ks[1:], [FAKE] * 6)] == "DSV_ERR_K"
    assert dsv.STATUS[dsv.validate(dsv.DSV_OP_FWD, p, [65537] + ks[1:], [FAKE] * 6)] == "DSV_ERR_K"
    assert dsv.validate(dsv.DSV_OP_FWD, p, [65536] + ks[1:], [FAKE] * 6) == 0   # k = S: dense
    ptrs = [FAKE] * 6
    ptrs[2] = 0
    assert dsv.STATUS[dsv.validate(dsv.DSV_OP_FWD, p, ks, ptrs)] == "DSV_ERR_NULL"
    ptrs[2] = FAKE + 8
    assert dsv.STATUS[dsv.validate(dsv.DSV_OP_FWD, p, ks, ptrs)] == "DSV_ERR_ALIGN"
    ptrs = [FAKE] * 3
    assert dsv.validate(dsv.DSV_OP_TOPK, p, ks, ptrs, reduce=dsv.DSV_GROUP_MAX) == 0
    assert dsv.STATUS[dsv.validate(dsv.DSV_OP_TOPK, p, ks, ptrs, reduce=5)] == \
        "DSV_ERR_UNSUPPORTED"
    assert dsv.STATUS[dsv.validate(dsv.DSV_OP_TOPK, p, ks, [FAKE] * 2)] == "DSV_ERR_NULL"


def test_entry_points_reject_before_any_hip_call():
    """Invalid arguments come back as status codes without a GPU being touched."""
    L = dsv.lib()
    p = mid()
    p.gt = 3
    ks = (ctypes.c_int32 * 24)(*([6554] * 24))
    st = L.dsv_lowrank_topk(ctypes.byref(p), FAKE, FAKE, ks, 0, FAKE, None, 0, None)
    assert dsv.STATUS[st] == "DSV_ERR_SHAPE"
    p = mid()
    st = L.dsv_sparse_attn_fwd(ctypes.byref(p), FAKE, 0, FAKE, FAKE, ks, 0.1, FAKE, FAKE,
                               None, 0, None)
    assert dsv.STATUS[st] == "DSV_ERR_NULL"
    st = L.dsv_sparse_attn_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                               0.1, FAKE, FAKE, FAKE, None, 0, None)
    assert dsv.STATUS[st] == "DSV_ERR_NULL"


@pytest.mark.parametrize("scale", [0.0, -0.125, float("inf"), float("nan")])
def test_attention_rejects_a_scale_that_is_not_positive_and_finite(scale):
    """The kernels order logits by raw q.k: a scale <= 0 or not finite is refused before any
    HIP call (forward and backward)."""
    L = dsv.lib()
    p = mid()
    ks = (ctypes.c_int32 * 24)(*([6554] * 24))
    st = L.dsv_sparse_attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, ks, scale, FAKE, FAKE,
                               None, 0, None)
    assert dsv.STATUS[st] == "DSV_ERR_SHAPE" and "scale" in dsv.last_error()
    need = dsv.workspace_bytes(dsv.DSV_OP_BWD, p, list(ks))
    st = L.dsv_sparse_attn_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ks,
                               scale, FAKE, FAKE, FAKE, FAKE, need, None)
    assert dsv.STATUS[st] == "DSV_ERR_SHAPE" and "scale" in dsv.last_error()


def test_workspace_and_idx_layout_agree_with_oracle():
    p = dsv.problem(2, 3, 4, 8, 8, 64, 16, (2, 2, 4), "bf16")
    ks = [5, 17, 3]
    for op in (dsv.DSV_OP_TOPK, dsv.DSV_OP_FWD):
        assert dsv.workspace_bytes(op, p, ks) == 0
    # backward (bf16), for one (b, h) slot: per-row bucket entry points NG x (nB+1) u32 and
    # their transpose, bucket totals and offsets (nB+1) u32 each, then per staging row of the heaviest slot
    # (NG * max k rounded up to 32): a bucket-list entry (u32), a d-entry fp16 dV row and a
    # d-entry fp16 dK row (an 8-bit row uses the first d bytes), plus two fp32 factors per 16
    # rows
    al = lambda x: -(-x // 256) * 256
    nb = -(-p.seq // 32)
    NG = p.n_groups
    e = NG * (-(-max(ks) // 32) * 32)
    need = (2 * al(NG * (nb + 1) * 4) + 2 * al((nb + 1) * 4) + al(e * 4) + al(e // 16 * 8)
            + al(e * 64 * 2) + e * 64 * 2)
    assert dsv.workspace_bytes(dsv.DSV_OP_BWD, p, ks) == need
    pf = dsv.problem(2, 3, 4, 8, 8, 64, 16, (2, 2, 4), "fp32")
    # fp32: fixed-point dV and dK accumulators, 8 bytes per element each (S = 4 * 8 * 8)
    assert dsv.workspace_bytes(dsv.DSV_OP_BWD, pf, ks) == 2 * 3 * 256 * 64 * 2 * 8
    assert dsv.validate(dsv.DSV_OP_BWD, p, ks, [FAKE] * 10, ws_bytes=need) == 0
    assert dsv.STATUS[dsv.validate(dsv.DSV_OP_BWD, p, ks, [FAKE] * 10, ws_bytes=need - 1)] \
        == "DSV_ERR_WORKSPACE"
    NG = p.n_groups
    assert dsv.idx_elems(p, ks) == 2 * NG * sum(ks)
    offs = otopk.idx_row_offsets(2, 3, NG, ks)
    for b in range(2):
        for h in range(3):
            for g in (0, 1, NG - 1):
                assert dsv.idx_row_offset(p, ks, b, h, g) == offs[b, h] + g * ks[h]
    assert dsv.idx_row_offset(p, ks, 2, 0, 0) == -1
    bad = dsv.problem(2, 3, 4, 8, 8, 64, 16, (3, 2, 4), "bf16")
    assert dsv.idx_elems(bad, ks) == 0
    assert dsv.workspace_bytes(dsv.DSV_OP_FWD, bad, ks) == np.iinfo(np.uint64).max


def test_bwd_chunks_and_profiled_entry_point_validation():
    """Chunk count follows the workspace; the profiling variant rejects a wrong event count,
    NULL events and the fp32 path before any HIP call."""
    L = dsv.lib()
    p = mid()
    ks = [6554] * 24
    need = dsv.workspace_bytes(dsv.DSV_OP_BWD, p, ks)
    assert dsv.bwd_chunks(p, ks, need) == 24          # the minimum holds one (b, h) slot
    assert dsv.bwd_chunks(p, ks, need - 1) == -1
    big = dsv.bwd_chunks(p, ks, 4 * need)
    assert 1 <= big < 24
    assert dsv.bwd_chunks(p, ks, 64 * need) == 1
    kp = (ctypes.c_int32 * 24)(*ks)
    args = [ctypes.byref(p)] + [FAKE] * 7 + [kp, 0.1, FAKE, FAKE, FAKE, FAKE, need, None]
    ev = (ctypes.c_void_p * 96)(*([FAKE] * 96))
    st = L.dsv_sparse_attn_bwd_profiled(*args, ev, 95)
    assert dsv.STATUS[st] == "DSV_ERR_NULL" and "stage events" in dsv.last_error()
    st = L.dsv_sparse_attn_bwd_profiled(*args, None, 96)
    assert dsv.STATUS[st] == "DSV_ERR_NULL"
    ev[3] = None
    st = L.dsv_sparse_attn_bwd_profiled(*args, ev, 96)
    assert dsv.STATUS[st] == "DSV_ERR_NULL"
    pf = dsv.problem(1, 2, 4, 16, 16, 64, 16, (2, 2, 4), "fp32")
    kf = (ctypes.c_int32 * 2)(128, 128)
    need_f = dsv.workspace_bytes(dsv.DSV_OP_BWD, pf, [128, 128])   # fixed-point accumulators
    st = L.dsv_sparse_attn_bwd_profiled(ctypes.byref(pf), *([FAKE] * 7), kf, 0.1, FAKE, FAKE,
                                        FAKE, FAKE, need_f, None, ev, 4)
    assert dsv.STATUS[st] == "DSV_ERR_UNSUPPORTED"


def test_topk_max_cache_bytes():
    """Per-slot bytes of the MAX score cache: NG rows of S keys rounded up to 128, 4 bytes
    each, the total rounded up to 256; a bad problem raises (the C call returns SIZE_MAX)."""
    al = lambda x: -(-x // 256) * 256
    for p in (mid(), dsv.problem(2, 3, 4, 8, 8, 64, 16, (2, 2, 4), "bf16"),
              dsv.problem(1, 2, 3, 8, 12, 64, 16, (1, 4, 4), "fp32")):
        row = -(-p.seq // 128) * 128
        assert dsv.topk_max_cache_bytes(p) == al(p.n_groups * row * 4)
    assert dsv.topk_max_cache_bytes(mid()) == 1024 * 65536 * 4
    with pytest.raises(ValueError):
        dsv.topk_max_cache_bytes(dsv.problem(2, 3, 4, 8, 8, 64, 16, (3, 2, 4), "bf16"))


def test_noalloc_bwd_validates_before_any_hip_call():
    """The no-allocation backward refuses, before touching HIP, a problem whose heaviest head
    does not fit its fixed scratch (S = 64K, d = 128, k = 10%), and bad arguments as the
    workspace entry point does."""
    L = dsv.lib()
    p = dsv.problem(1, 1, 16, 64, 64, 128, 32, (4, 4, 4), "bf16")
    ks = (ctypes.c_int32 * 1)(6554)
    assert dsv.workspace_bytes(dsv.DSV_OP_BWD, p, [6554]) > 256 * 1024 * 1024
    args = [FAKE] * 7
    st = L.dsv_sparse_attn_bwd_noalloc(ctypes.byref(p), *args, ks, 0.088, FAKE, FAKE, FAKE, None)
    assert dsv.STATUS[st] == "DSV_ERR_WORKSPACE" and "scratch" in dsv.last_error()
    small = dsv.problem(1, 1, 16, 32, 32, 64, 16, (4, 4, 4), "bf16")
    ks1 = (ctypes.c_int32 * 1)(1638)
    st = L.dsv_sparse_attn_bwd_noalloc(ctypes.byref(small), FAKE, 0, *[FAKE] * 5, ks1, 0.125,
                                       FAKE, FAKE, FAKE, None)
    assert dsv.STATUS[st] == "DSV_ERR_NULL"
    st = L.dsv_sparse_attn_bwd_noalloc(ctypes.byref(small), *[FAKE] * 7, ks1, 0.0, FAKE, FAKE,
                                       FAKE, None)
    assert dsv.STATUS[st] == "DSV_ERR_SHAPE"

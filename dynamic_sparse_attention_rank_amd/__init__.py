"""Python binding of libdsv.so, the DSV hot path for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the library's HIP kernels.
PyTorch supplies device memory and the current HIP stream. The names mirror the C ABI in
include/dsv.h: `lowrank_topk`, `sparse_attn_fwd`, `sparse_attn_bwd`.

Import fails loudly if the library has not been built (`build()` or
`python -m dynamic_sparse_attention_rank_amd._build`): there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import List, Optional, Sequence, Tuple

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libdsv.so")

DSV_FP32, DSV_BF16 = 0, 1
DSV_GROUP_SUM, DSV_GROUP_MAX = 0, 1
DSV_OP_TOPK, DSV_OP_FWD, DSV_OP_BWD = 0, 1, 2
STATUS = {0: "DSV_OK", 1: "DSV_ERR_NULL", 2: "DSV_ERR_SHAPE", 3: "DSV_ERR_K",
          4: "DSV_ERR_DTYPE", 5: "DSV_ERR_ALIGN", 6: "DSV_ERR_WORKSPACE",
          7: "DSV_ERR_UNSUPPORTED", 8: "DSV_ERR_HIP"}
EXPORTED = ("dsv_workspace_bytes", "dsv_idx_elems", "dsv_idx_row_offset", "dsv_lowrank_topk",
            "dsv_sparse_attn_fwd", "dsv_sparse_attn_bwd", "dsv_bwd_chunks",
            "dsv_sparse_attn_bwd_profiled", "dsv_validate", "dsv_status_string",
            "dsv_last_error", "dsv_version", "dsv_plan_heads", "dsv_default_cost_model",
            "dsv_dispatch_k", "dsv_adaptive_k", "dsv_topk_max_cache_bytes", "dsv_plan_order",
            "dsv_sparse_attn_bwd_noalloc")


class DsvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class CostModel(ctypes.Structure):
    _fields_ = [("topk_ns_per_score", ctypes.c_double), ("attn_ns_per_edge", ctypes.c_double)]


class Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "heads", "frames", "height", "width", "head_dim", "rank",
                 "gt", "gh", "gw", "dtype")]

    @property
    def seq(self) -> int:
        return self.frames * self.height * self.width

    @property
    def group_size(self) -> int:
        return self.gt * self.gh * self.gw

    @property
    def n_groups(self) -> int:
        return self.seq // self.group_size


def problem(batch, heads, frames, height, width, head_dim, rank, group, dtype) -> Problem:
    gt, gh, gw = group
    dt = {"fp32": DSV_FP32, "bf16": DSV_BF16}.get(dtype, dtype)
    return Problem(batch, heads, frames, height, width, head_dim, rank, gt, gh, gw, dt)


def problem_for(cfg) -> Problem:
    """Problem descriptor of a `synth` workload."""
    return problem(cfg.batch, cfg.heads, cfg.frames, cfg.height, cfg.width, cfg.head_dim,
                   cfg.rank, cfg.group, cfg.dtype)


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m dynamic_sparse_attention_rank_amd._build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(Problem)
        i32p = ctypes.POINTER(ctypes.c_int32)
        vp, sz, f = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float
        L.dsv_workspace_bytes.argtypes = [ctypes.c_int, P, i32p]
        L.dsv_workspace_bytes.restype = sz
        L.dsv_topk_max_cache_bytes.argtypes = [P]
        L.dsv_topk_max_cache_bytes.restype = sz
        L.dsv_idx_elems.argtypes = [P, i32p]
        L.dsv_idx_elems.restype = ctypes.c_int64
        L.dsv_idx_row_offset.argtypes = [P, i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
        L.dsv_idx_row_offset.restype = ctypes.c_int64
        L.dsv_lowrank_topk.argtypes = [P, vp, vp, i32p, ctypes.c_int, vp, vp, sz, vp]
        L.dsv_sparse_attn_fwd.argtypes = [P, vp, vp, vp, vp, i32p, f, vp, vp, vp, sz, vp]
        L.dsv_sparse_attn_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, i32p, f, vp, vp, vp,
                                          vp, sz, vp]
        L.dsv_sparse_attn_bwd_profiled.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, i32p, f, vp,
                                                   vp, vp, vp, sz, vp, ctypes.POINTER(vp),
                                                   ctypes.c_int]
        L.dsv_sparse_attn_bwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, i32p, f, vp,
                                                  vp, vp, vp]
        L.dsv_bwd_chunks.argtypes = [P, i32p, sz]
        L.dsv_bwd_chunks.restype = ctypes.c_int
        L.dsv_validate.argtypes = [ctypes.c_int, P, i32p, ctypes.c_int,
                                   ctypes.POINTER(vp), ctypes.c_int, sz]
        dp = ctypes.POINTER(ctypes.c_double)
        L.dsv_plan_heads.argtypes = [i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
                                     ctypes.c_double, i32p, dp, dp]
        L.dsv_plan_order.argtypes = [i32p, ctypes.c_int32, ctypes.c_double, ctypes.c_double,
                                     i32p]
        L.dsv_default_cost_model.argtypes = [P, ctypes.c_int, ctypes.POINTER(CostModel)]
        L.dsv_dispatch_k.argtypes = [P, i32p, ctypes.POINTER(CostModel), i32p, i32p]
        L.dsv_adaptive_k.argtypes = [P, vp, vp, f, ctypes.c_double, vp, vp, vp]
        L.dsv_status_string.restype = ctypes.c_char_p
        L.dsv_status_string.argtypes = [ctypes.c_int]
        L.dsv_last_error.restype = ctypes.c_char_p
        L.dsv_version.restype = ctypes.c_char_p
        for fn in ("dsv_lowrank_topk", "dsv_sparse_attn_fwd", "dsv_sparse_attn_bwd",
                   "dsv_sparse_attn_bwd_profiled", "dsv_validate", "dsv_plan_heads",
                   "dsv_default_cost_model", "dsv_dispatch_k", "dsv_adaptive_k",
                   "dsv_plan_order", "dsv_sparse_attn_bwd_noalloc"):
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def _kph(k_per_head: Sequence[int]):
    arr = (ctypes.c_int32 * len(k_per_head))(*[int(x) for x in k_per_head])
    return arr


def _check(status: int) -> None:
    if status != 0:
        raise DsvError(status, lib().dsv_last_error().decode())


def last_error() -> str:
    return lib().dsv_last_error().decode()


def version() -> str:
    return lib().dsv_version().decode()


def idx_elems(p: Problem, k_per_head: Sequence[int]) -> int:
    return int(lib().dsv_idx_elems(ctypes.byref(p), _kph(k_per_head)))


def idx_row_offset(p: Problem, k_per_head: Sequence[int], b: int, h: int, g: int) -> int:
    return int(lib().dsv_idx_row_offset(ctypes.byref(p), _kph(k_per_head), b, h, g))


def workspace_bytes(op: int, p: Problem, k_per_head: Sequence[int]) -> int:
    return int(lib().dsv_workspace_bytes(op, ctypes.byref(p), _kph(k_per_head)))


def validate(op: int, p: Problem, k_per_head: Sequence[int], ptrs: Sequence[int],
             reduce: int = DSV_GROUP_SUM, ws_bytes: int = 0) -> int:
    """Status the call would return for these arguments (no HIP call is made)."""
    arr = (ctypes.c_void_p * len(ptrs))(*ptrs)
    return int(lib().dsv_validate(op, ctypes.byref(p), _kph(k_per_head), reduce, arr,
                                  len(ptrs), ws_bytes))


def plan_heads(k_per_head: Sequence[int], n_parts: int, fixed_cost: float = 0.0,
               cost_per_k: float = 1.0) -> Tuple[List[int], List[float], float]:
    """(part of each head, load of each part, rho_s) of the longest-processing-time placement
    of heads with cost fixed_cost + cost_per_k * k_h over n_parts devices."""
    H = len(k_per_head)
    part = (ctypes.c_int32 * max(H, 1))()
    load = (ctypes.c_double * max(n_parts, 1))()
    rho = ctypes.c_double()
    _check(lib().dsv_plan_heads(_kph(k_per_head), H, n_parts, float(fixed_cost),
                                float(cost_per_k), part, load, ctypes.byref(rho)))
    return list(part)[:H], list(load)[:n_parts], rho.value


def plan_order(k_per_head: Sequence[int], fixed_cost: float = 0.0,
               cost_per_k: float = 1.0) -> List[int]:
    """Heads in the planner's processing order (decreasing cost, ties to the lower head); with
    the defaults, the order in which the kernels launch the heads of a problem."""
    H = len(k_per_head)
    out = (ctypes.c_int32 * max(H, 1))()
    _check(lib().dsv_plan_order(_kph(k_per_head), H, float(fixed_cost), float(cost_per_k),
                                out))
    return list(out)[:H]


def default_cost_model(p: Problem, with_backward: bool = True) -> CostModel:
    """Measured MI355X per-unit costs of this library's kernels, scaled to the problem."""
    cm = CostModel()
    _check(lib().dsv_default_cost_model(ctypes.byref(p), int(with_backward), ctypes.byref(cm)))
    return cm


def dispatch_k(p: Problem, k_per_head: Sequence[int],
               cost_model: Optional[CostModel] = None) -> Tuple[List[int], int]:
    """(k per head after the dense-versus-sparse choice, number of dense heads)."""
    cm = cost_model if cost_model is not None else default_cost_model(p)
    out = (ctypes.c_int32 * p.heads)()
    nd = ctypes.c_int32()
    _check(lib().dsv_dispatch_k(ctypes.byref(p), _kph(k_per_head), ctypes.byref(cm), out,
                                ctypes.byref(nd)))
    return list(out), nd.value


# ----------------------------------------------------------------------------- torch layer
def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    return stream if stream is not None else torch.cuda.current_stream()


def _stream_ptr(stream) -> int:
    return int(_stream(stream).cuda_stream)


def _dev(t, name, dtype=None, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _storage_dtype(p: Problem):
    torch = _torch()
    return torch.float32 if p.dtype == DSV_FP32 else torch.bfloat16


def lowrank_topk(p: Problem, q_lr, k_lr, k_per_head: Sequence[int], idx=None,
                 reduce: int = DSV_GROUP_SUM, stream=None, ws=None):
    """Critical-KV index lists (packed int32, see include/dsv.h) for Q_lr, K_lr [B,H,S,r].
    `ws` (optional uint8 device tensor): with reduce=MAX, room for c * topk_max_cache_bytes(p)
    bytes keeps the group scores of c (b, h) slots between selection passes."""
    torch = _torch()
    dt = _storage_dtype(p)
    shp = (p.batch, p.heads, p.seq, p.rank)
    qp = _dev(q_lr, "q_lr", dt, shp)
    kp = _dev(k_lr, "k_lr", dt, shp)
    n = idx_elems(p, k_per_head)
    if idx is None:   # allocated on the launch stream: the caching allocator orders its reuse
        with torch.cuda.stream(_stream(stream)):
            idx = torch.empty(max(n, 1), dtype=torch.int32, device=q_lr.device)
    ip = _dev(idx, "idx", torch.int32)
    if idx.numel() < n:
        raise ValueError("idx is too small")
    wp, wb = None, 0
    if ws is not None:
        wp = _dev(ws, "ws", torch.uint8)
        wb = ws.numel()
    _check(lib().dsv_lowrank_topk(ctypes.byref(p), qp, kp, _kph(k_per_head), reduce, ip,
                                  wp, wb, _stream_ptr(stream)))
    return idx


def topk_max_cache_bytes(p: Problem) -> int:
    """Workspace bytes per (b, h) slot for the MAX score cache of lowrank_topk."""
    n = int(lib().dsv_topk_max_cache_bytes(ctypes.byref(p)))
    if n == ctypes.c_size_t(-1).value:
        raise ValueError(last_error())
    return n


def adaptive_k(p: Problem, q_lr, k_lr, mass: float = 0.9, logit_scale: Optional[float] = None,
               k_group=None, stream=None):
    """(k_head [H], k_group [B, H, NG]) int32 device tensors: per group, the keys that carry
    `mass` of the estimated attention (see include/dsv.h); logit_scale defaults to
    1 / (sqrt(d) * G), the mean member logit."""
    torch = _torch()
    dt = _storage_dtype(p)
    shp = (p.batch, p.heads, p.seq, p.rank)
    qp = _dev(q_lr, "q_lr", dt, shp)
    kp = _dev(k_lr, "k_lr", dt, shp)
    if logit_scale is None:
        logit_scale = 1.0 / (math.sqrt(p.head_dim) * p.group_size)
    with torch.cuda.stream(_stream(stream)):   # outputs belong to the launch stream
        if k_group is None:
            k_group = torch.empty((p.batch, p.heads, p.n_groups), dtype=torch.int32,
                                  device=q_lr.device)
        k_head = torch.empty(p.heads, dtype=torch.int32, device=q_lr.device)
    gp = _dev(k_group, "k_group", torch.int32, (p.batch, p.heads, p.n_groups))
    _check(lib().dsv_adaptive_k(ctypes.byref(p), qp, kp, float(logit_scale), float(mass), gp,
                                k_head.data_ptr(), _stream_ptr(stream)))
    return k_head, k_group


def sparse_attn_fwd(p: Problem, q, k, v, idx, k_per_head: Sequence[int],
                    scale: Optional[float] = None, o=None, lse=None, stream=None):
    """(O, LSE) of the query-grouped sparse attention forward."""
    torch = _torch()
    dt = _storage_dtype(p)
    shp = (p.batch, p.heads, p.seq, p.head_dim)
    if scale is None:
        scale = 1.0 / math.sqrt(p.head_dim)
    ptr = [_dev(q, "q", dt, shp), _dev(k, "k", dt, shp), _dev(v, "v", dt, shp),
           _dev(idx, "idx", torch.int32)]
    if idx.numel() < idx_elems(p, k_per_head):
        raise ValueError("idx is too small")
    with torch.cuda.stream(_stream(stream)):   # outputs belong to the launch stream
        if o is None:
            o = torch.empty(shp, dtype=dt, device=q.device)
        if lse is None:
            lse = torch.empty(shp[:3], dtype=torch.float32, device=q.device)
    op = _dev(o, "o", dt, shp)
    lp = _dev(lse, "lse", torch.float32, shp[:3])
    _check(lib().dsv_sparse_attn_fwd(ctypes.byref(p), ptr[0], ptr[1], ptr[2], ptr[3],
                                     _kph(k_per_head), float(scale), op, lp, None, 0,
                                     _stream_ptr(stream)))
    return o, lse


def bwd_chunks(p: Problem, k_per_head: Sequence[int], ws_bytes: int) -> int:
    """Head chunks the backward uses with a workspace of ws_bytes (-1 if invalid/too small)."""
    return int(lib().dsv_bwd_chunks(ctypes.byref(p), _kph(k_per_head), ws_bytes))


def sparse_attn_bwd(p: Problem, q, k, v, o, d_o, lse, idx, k_per_head: Sequence[int],
                    scale: Optional[float] = None, dq=None, dk=None, dv=None, ws=None,
                    stream=None, events: Optional[Sequence[int]] = None):
    """(dQ, dK, dV) in fp32 for the query-grouped sparse attention.

    `ws` is a device uint8 tensor of at least workspace_bytes(DSV_OP_BWD, ...) bytes; one is
    allocated for the call when it is None. `events` (profiling, bf16 only): raw hipEvent_t
    handles, 4 per head chunk, passed to dsv_sparse_attn_bwd_profiled."""
    torch = _torch()
    dt = _storage_dtype(p)
    shp = (p.batch, p.heads, p.seq, p.head_dim)
    if scale is None:
        scale = 1.0 / math.sqrt(p.head_dim)
    ptr = [_dev(q, "q", dt, shp), _dev(k, "k", dt, shp), _dev(v, "v", dt, shp),
           _dev(o, "o", dt, shp), _dev(d_o, "d_o", dt, shp),
           _dev(lse, "lse", torch.float32, shp[:3]), _dev(idx, "idx", torch.int32)]
    if idx.numel() < idx_elems(p, k_per_head):
        raise ValueError("idx is too small")
    outs = []
    need = workspace_bytes(DSV_OP_BWD, p, k_per_head)
    # Outputs and the call's own workspace are allocated on the launch stream: the caching
    # allocator then hands the workspace to nothing else until that stream has passed the
    # call, although it is dropped when this function returns.
    with torch.cuda.stream(_stream(stream)):
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            if t is None:
                t = torch.empty(shp, dtype=torch.float32, device=q.device)
            _dev(t, name, torch.float32, shp)
            outs.append(t)
        if ws is None and need > 0:
            ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    wp = _dev(ws, "ws", torch.uint8) if ws is not None else None
    wn = ws.numel() if ws is not None else 0
    args = (ctypes.byref(p), *ptr[:6], ptr[6], _kph(k_per_head), float(scale),
            outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(), wp, wn,
            _stream_ptr(stream))
    if events is None:
        _check(lib().dsv_sparse_attn_bwd(*args))
    else:
        ev = (ctypes.c_void_p * len(events))(*events)
        _check(lib().dsv_sparse_attn_bwd_profiled(*args, ev, len(events)))
    return tuple(outs)


def idx_rows(idx, p: Problem, k_per_head: Sequence[int], b: int, h: int):
    """View of the (b, h) block of a packed idx tensor as [NG, k_h]."""
    off = idx_row_offset(p, k_per_head, b, h, 0)
    kh = int(k_per_head[h])
    return idx[off:off + p.n_groups * kh].view(p.n_groups, kh)


def build(verbose: bool = False) -> str:
    from . import _build
    return _build.build(verbose=verbose)

"""Python binding of libssa.so, the HIP (gfx950) Spatial Sparse Attention library.

Argument marshalling only: every step of the computation runs in the library's
HIP kernels.  PyTorch supplies device memory (tensors) and the stream.  The
library must have been built (``python spatial_sparse_attention_amd/build.py``);
importing the binding without it raises immediately.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["Plan", "forward", "forward_workspace_size", "backward", "backward_workspace_size",
           "SSAError", "lib", "LIB_PATH", "STAGE_POOL", "STAGE_SELECT", "STAGE_ATTEND", "STAGE_ALL"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libssa.so")
STAGE_POOL, STAGE_SELECT, STAGE_ATTEND, STAGE_ALL = 1, 2, 4, 7
_DTYPES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
_STATUS = {0: "SSA_OK", 1: "SSA_ERR_INVALID_ARG", 2: "SSA_ERR_UNSUPPORTED", 3: "SSA_ERR_WORKSPACE",
           4: "SSA_ERR_COORD_RANGE", 5: "SSA_ERR_HIP", 6: "SSA_ERR_BAD_PLAN"}

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t


class PlanInfo(ctypes.Structure):
    _fields_ = [("n", _i64), ("num_blocks", _i64), ("num_cells", _i64), ("block", _i32),
                ("window", _i32), ("max_block_rows", _i32), ("perm", _vp), ("blk_off", _vp),
                ("blk_key", _vp), ("tok2blk", _vp), ("blk_cell", _vp), ("cell_off", _vp),
                ("cell_blk", _vp), ("lpt", _vp)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python spatial_sparse_attention_amd/build.py`")
    L = ctypes.CDLL(LIB_PATH)
    grid_t = ctypes.POINTER(_i32)
    L.ssa_plan_workspace_size.argtypes = [_i64, grid_t, _i32, _i32]
    L.ssa_plan_workspace_size.restype = _sz
    L.ssa_plan_create.argtypes = [_vp, _i64, grid_t, _i32, _i32, _vp, _sz, _vp, ctypes.POINTER(_vp)]
    L.ssa_plan_create.restype = ctypes.c_int
    L.ssa_plan_get_info.argtypes = [_vp, ctypes.POINTER(PlanInfo)]
    L.ssa_plan_get_info.restype = ctypes.c_int
    L.ssa_plan_destroy.argtypes = [_vp]
    L.ssa_plan_destroy.restype = None
    L.ssa_forward_workspace_size.argtypes = [_vp, ctypes.c_int, _i32, _i32, _i32, ctypes.c_int]
    L.ssa_forward_workspace_size.restype = _sz
    fwd = [_vp, ctypes.c_int, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, ctypes.c_float,
           _vp, _vp, _vp, _sz, ctypes.c_int, _vp]
    L.ssa_forward.argtypes = fwd
    L.ssa_forward.restype = ctypes.c_int
    L.ssa_forward_stages.argtypes = fwd + [ctypes.c_uint32]
    L.ssa_forward_stages.restype = ctypes.c_int
    L.ssa_backward_workspace_size.argtypes = [_vp, ctypes.c_int, _i32, _i32, _i32]
    L.ssa_backward_workspace_size.restype = _sz
    L.ssa_backward.argtypes = [_vp, ctypes.c_int, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                               ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _sz, _vp]
    L.ssa_backward.restype = ctypes.c_int
    L.ssa_status_string.argtypes = [ctypes.c_int]
    L.ssa_status_string.restype = ctypes.c_char_p
    return L


lib = _load()


class SSAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_STATUS.get(status, status)} "
                         f"({lib.ssa_status_string(status).decode()})")


def _check(status: int, where: str):
    if status != 0:
        raise SSAError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Plan:
    """Block partition of int32 coordinates [N,3] on the GPU (ssa_plan_create)."""

    def __init__(self, coords: torch.Tensor, grid, block: int, window: int, stream=None):
        if coords.dtype != torch.int32 or coords.dim() != 2 or coords.shape[1] != 3:
            raise ValueError("coords must be an int32 tensor of shape [N,3]")
        if not coords.is_contiguous():
            raise ValueError("coords must be contiguous")
        grid = [int(grid)] * 3 if isinstance(grid, int) else [int(x) for x in grid]
        self.grid = (_i32 * 3)(*grid)
        self.n = int(coords.shape[0])
        self.block, self.window = int(block), int(window)
        size = lib.ssa_plan_workspace_size(self.n, self.grid, self.block, self.window)
        if size == 0:
            raise SSAError(1, "ssa_plan_workspace_size")
        self.ws = torch.empty(size, dtype=torch.uint8, device=coords.device)
        self.coords = coords
        h = _vp()
        st = lib.ssa_plan_create(_ptr(coords), self.n, self.grid, self.block, self.window,
                                 _ptr(self.ws), size, _stream(stream), ctypes.byref(h))
        _check(st, "ssa_plan_create")
        self.handle = h
        info = PlanInfo()
        _check(lib.ssa_plan_get_info(h, ctypes.byref(info)), "ssa_plan_get_info")
        self.info = info
        self.num_blocks = int(info.num_blocks)
        self.num_cells = int(info.num_cells)
        self.max_block_rows = int(info.max_block_rows)

    def _view(self, ptr, count):
        off = int(ptr) - self.ws.data_ptr()
        return self.ws[off:off + 4 * count].view(torch.int32)

    def arrays(self) -> dict:
        """Views of the plan's device arrays (int32 tensors inside the plan workspace)."""
        n, M, C = self.n, self.num_blocks, self.num_cells
        if n == 0:
            return {}
        i = self.info
        return {"perm": self._view(i.perm, n), "blk_off": self._view(i.blk_off, M + 1),
                "blk_key": self._view(i.blk_key, M), "tok2blk": self._view(i.tok2blk, n),
                "blk_cell": self._view(i.blk_cell, M), "cell_off": self._view(i.cell_off, C + 1),
                "cell_blk": self._view(i.cell_blk, M), "lpt": self._view(i.lpt, M)}

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            lib.ssa_plan_destroy(h)
            self.handle = None


def forward_workspace_size(plan: Plan, dtype, heads: int, dim: int, topk: int,
                           save_for_bwd: bool = False) -> int:
    return int(lib.ssa_forward_workspace_size(plan.handle, _DTYPES[dtype], heads, dim, topk,
                                              int(save_for_bwd)))


def _check_qkv(plan, q, k, v, wk, wv, gates):
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for t in (q, k, v, wk, wv, gates):
        if t.dtype != q.dtype or not t.is_contiguous() or t.device != q.device:
            raise ValueError("all tensors must be contiguous, on one device, with one dtype")
    N, H, d = q.shape
    if N != plan.n or k.shape != q.shape or v.shape != q.shape or gates.shape != (N, H, 3) \
            or wk.shape != (d, d) or wv.shape != (d, d):
        raise ValueError("shape mismatch")
    return N, H, d


def forward(plan: Plan, q, k, v, wk, wv, gates, topk: int, scale: float = 0.0, out=None,
            sel_out=None, ws=None, stream=None, stages: int = STAGE_ALL, want_sel: bool = True,
            save_for_bwd: bool = False):
    """SSA forward (ssa_forward_stages).  q,k,v [N,H,d], gates [N,H,3], wk,wv [d,d], one dtype.
    Returns (out [N,H,d], sel [H,M,topk] int32 or None).  With save_for_bwd, `ws` must be
    kept and passed to backward()."""
    N, H, d = _check_qkv(plan, q, k, v, wk, wv, gates)
    dt = _DTYPES[q.dtype]
    if out is None:
        out = torch.empty_like(q)
    if sel_out is None and want_sel:
        sel_out = torch.empty((H, max(plan.num_blocks, 1), topk), dtype=torch.int32, device=q.device)
    size = lib.ssa_forward_workspace_size(plan.handle, dt, H, d, topk, int(save_for_bwd))
    if size == 0:
        raise SSAError(2, "ssa_forward_workspace_size")
    if ws is None or ws.numel() < size:
        ws = torch.empty(size, dtype=torch.uint8, device=q.device)
    st = lib.ssa_forward_stages(plan.handle, dt, H, d, _ptr(q), _ptr(k), _ptr(v), _ptr(wk),
                                _ptr(wv), _ptr(gates), int(topk), float(scale), _ptr(out),
                                _ptr(sel_out), _ptr(ws), ws.numel(), int(save_for_bwd),
                                _stream(stream), int(stages))
    _check(st, "ssa_forward")
    return out, sel_out


def backward_workspace_size(plan: Plan, dtype, heads: int, dim: int, topk: int) -> int:
    return int(lib.ssa_backward_workspace_size(plan.handle, _DTYPES[dtype], heads, dim, topk))


def backward(plan: Plan, q, k, v, wk, wv, gates, topk: int, sel, dout, fwd_ws, scale: float = 0.0,
             ws=None, stream=None):
    """SSA backward (ssa_backward) with the selection `sel` held fixed.  fwd_ws: the workspace
    of a forward run with save_for_bwd=True on the same inputs.  Returns fp32
    (dq, dk, dv, dgates)."""
    N, H, d = _check_qkv(plan, q, k, v, wk, wv, gates)
    if dout.shape != q.shape or dout.dtype != q.dtype or not dout.is_contiguous():
        raise ValueError("dout must match q")
    if sel.dtype != torch.int32 or not sel.is_contiguous():
        raise ValueError("sel must be a contiguous int32 tensor [H, M, topk]")
    dt = _DTYPES[q.dtype]
    f32 = dict(dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty(q.shape, **f32), torch.empty(q.shape, **f32), torch.empty(q.shape, **f32)
    dg = torch.empty((N, H, 3), **f32)
    size = lib.ssa_backward_workspace_size(plan.handle, dt, H, d, topk)
    if size == 0:
        raise SSAError(2, "ssa_backward_workspace_size")
    if ws is None or ws.numel() < size:
        ws = torch.empty(size, dtype=torch.uint8, device=q.device)
    st = lib.ssa_backward(plan.handle, dt, H, d, _ptr(q), _ptr(k), _ptr(v), _ptr(wk), _ptr(wv),
                          _ptr(gates), int(topk), float(scale), _ptr(sel), _ptr(dout), _ptr(dq),
                          _ptr(dk), _ptr(dv), _ptr(dg), _ptr(fwd_ws), fwd_ws.numel(), _ptr(ws),
                          ws.numel(), _stream(stream))
    _check(st, "ssa_backward")
    return dq, dk, dv, dg

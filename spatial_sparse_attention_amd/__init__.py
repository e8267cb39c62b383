"""Python binding of libssa.so, the HIP (gfx950) Spatial Sparse Attention library.

Argument marshalling only: every step of the computation runs in the library's
HIP kernels.  PyTorch supplies device memory (tensors) and the stream.  The
library must have been built (``python spatial_sparse_attention_amd/build.py``);
importing the binding without it raises immediately.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

__all__ = ["Plan", "Window", "qkv_gates", "forward", "forward_batch", "forward_batch_workspace_size", "forward_max_blocks", "forward_workspace_size", "forward_noalloc", "backward",
           "backward_workspace_size", "NOALLOC_SCRATCH_BYTES",
           "SSAError", "lib", "LIB_PATH", "STAGE_POOL", "STAGE_SELECT", "STAGE_ATTEND", "STAGE_ALL"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libssa.so")
STAGE_POOL, STAGE_SELECT, STAGE_ATTEND, STAGE_ALL = 1, 2, 4, 7
_DTYPES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
_STATUS = {0: "SSA_OK", 1: "SSA_ERR_INVALID_ARG", 2: "SSA_ERR_UNSUPPORTED", 3: "SSA_ERR_WORKSPACE",
           4: "SSA_ERR_COORD_RANGE", 5: "SSA_ERR_HIP", 6: "SSA_ERR_BAD_PLAN", 7: "SSA_ERR_TOO_LARGE"}
NOALLOC_SCRATCH_BYTES = 64 << 20

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t


class PlanInfo(ctypes.Structure):
    _fields_ = [("n", _i64), ("num_blocks", _i64), ("num_cells", _i64), ("block", _i32),
                ("window", _i32), ("max_block_rows", _i32), ("perm", _vp), ("blk_off", _vp),
                ("blk_key", _vp), ("tok2blk", _vp), ("blk_cell", _vp), ("cell_off", _vp),
                ("cell_blk", _vp), ("lpt", _vp), ("window_kind", _i32), ("window_shift", _i32 * 3),
                ("window_tokens", _i32), ("cells_are_block_unions", _i32), ("num_wcells", _i64),
                ("max_wcell_rows", _i32), ("wperm", _vp), ("wcell_off", _vp), ("wlpt", _vp)]


class Window(ctypes.Structure):
    """ssa_window_t: kind 0 = cubic cells floor((c + shift) / edge), 1 = Morton-order runs."""
    _fields_ = [("kind", _i32), ("edge", _i32), ("shift", _i32 * 3), ("tokens", _i32)]


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
    L.ssa_plan_workspace_size_ex.argtypes = [_i64, grid_t, _i32, ctypes.POINTER(Window)]
    L.ssa_plan_workspace_size_ex.restype = _sz
    L.ssa_plan_create_ex.argtypes = [_vp, _i64, grid_t, _i32, ctypes.POINTER(Window), _vp, _sz, _vp,
                                     ctypes.POINTER(_vp)]
    L.ssa_plan_create_ex.restype = ctypes.c_int
    L.ssa_plan_get_info.argtypes = [_vp, ctypes.POINTER(PlanInfo)]
    L.ssa_plan_get_info.restype = ctypes.c_int
    L.ssa_plan_destroy.argtypes = [_vp]
    L.ssa_plan_destroy.restype = None
    L.ssa_forward_max_blocks.argtypes = [ctypes.c_int, _i32]
    L.ssa_forward_max_blocks.restype = _i64
    L.ssa_forward_workspace_size.argtypes = [_vp, ctypes.c_int, _i32, _i32, _i32, ctypes.c_int]
    L.ssa_forward_workspace_size.restype = _sz
    fwd = [_vp, ctypes.c_int, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, ctypes.c_float,
           _vp, _vp, _vp, _sz, ctypes.c_int, _vp]
    L.ssa_forward.argtypes = fwd
    L.ssa_forward.restype = ctypes.c_int
    L.ssa_forward_stages.argtypes = fwd + [ctypes.c_uint32]
    L.ssa_forward_stages.restype = ctypes.c_int
    L.ssa_forward_conv.argtypes = fwd
    L.ssa_forward_conv.restype = ctypes.c_int
    L.ssa_forward_noalloc.argtypes = [_vp, ctypes.c_int, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _i32, ctypes.c_float, _vp, _vp, _vp]
    L.ssa_forward_noalloc.restype = ctypes.c_int
    L.ssa_forward_batch_workspace_size.argtypes = [_vp, _i32, ctypes.c_int, _i32, _i32, _i32]
    L.ssa_forward_batch_workspace_size.restype = _sz
    L.ssa_forward_batch.argtypes = [_vp, _i32, _vp, ctypes.c_int, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                                    _vp, _i32, ctypes.c_float, _vp, _vp, _sz, _vp]
    L.ssa_forward_batch.restype = ctypes.c_int
    L.ssa_backward_workspace_size.argtypes = [_vp, ctypes.c_int, _i32, _i32, _i32]
    L.ssa_backward_workspace_size.restype = _sz
    L.ssa_backward.argtypes = [_vp, ctypes.c_int, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                               ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _sz, _vp]
    L.ssa_backward.restype = ctypes.c_int
    L.ssa_backward_conv.argtypes = L.ssa_backward.argtypes
    L.ssa_backward_conv.restype = ctypes.c_int
    L.ssa_qkv_gates.argtypes = [ctypes.c_int, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                ctypes.c_float, ctypes.c_float, _vp, _vp, _vp, _vp, _vp]
    L.ssa_qkv_gates.restype = ctypes.c_int
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


def _alloc_on(stream):
    """Context for the binding's own allocations: torch's caching allocator ties a block to
    the stream current at allocation, so tensors that the library's kernels use on
    `stream` are allocated with `stream` current (their memory is then reused only in that
    stream's order)."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _uses(stream, *tensors):
    """Tell the caching allocator that `stream` uses caller-held tensors allocated on another
    stream (so their memory is not reused while its kernels may still read or write them)."""
    if stream is None or stream == torch.cuda.current_stream():
        return
    for t in tensors:
        if t is not None and t.is_cuda:
            t.record_stream(stream)


class Plan:
    """Block partition of int32 coordinates [N,3] on the GPU (ssa_plan_create_ex).  The window
    branch uses cubic cells of edge `window` shifted by `shift`, or, with sfc_tokens > 0,
    runs of sfc_tokens tokens along the Morton order of the voxels.  `ws`: an optional uint8
    device buffer for the plan's arrays (allocated here when absent or too small)."""

    def __init__(self, coords: torch.Tensor, grid, block: int, window: int, stream=None,
                 shift=(0, 0, 0), sfc_tokens: int = 0, ws=None):
        if coords.dtype != torch.int32 or coords.dim() != 2 or coords.shape[1] != 3:
            raise ValueError("coords must be an int32 tensor of shape [N,3]")
        if not coords.is_contiguous():
            raise ValueError("coords must be contiguous")
        grid = [int(grid)] * 3 if isinstance(grid, int) else [int(x) for x in grid]
        self.grid = (_i32 * 3)(*grid)
        self.n = int(coords.shape[0])
        self.block, self.window = int(block), int(window)
        self.win = Window(1 if sfc_tokens else 0, int(window), (_i32 * 3)(*[int(x) for x in shift]),
                          int(sfc_tokens))
        size = lib.ssa_plan_workspace_size_ex(self.n, self.grid, self.block, ctypes.byref(self.win))
        if size == 0:
            raise SSAError(1, "ssa_plan_workspace_size")
        if ws is None or ws.numel() < size:
            with _alloc_on(stream):
                ws = torch.empty(size, dtype=torch.uint8, device=coords.device)
        self.ws = ws
        _uses(stream, coords, ws)
        self.coords = coords
        h = _vp()
        st = lib.ssa_plan_create_ex(_ptr(coords), self.n, self.grid, self.block, ctypes.byref(self.win),
                                    _ptr(self.ws), self.ws.numel(), _stream(stream), ctypes.byref(h))
        _check(st, "ssa_plan_create")
        self.handle = h
        info = PlanInfo()
        _check(lib.ssa_plan_get_info(h, ctypes.byref(info)), "ssa_plan_get_info")
        self.info = info
        self.num_blocks = int(info.num_blocks)
        self.num_cells = int(info.num_cells)
        self.max_block_rows = int(info.max_block_rows)
        self.cells_are_block_unions = bool(info.cells_are_block_unions)
        self.num_wcells = int(info.num_wcells)

    def _view(self, ptr, count):
        off = int(ptr) - self.ws.data_ptr()
        return self.ws[off:off + 4 * count].view(torch.int32)

    def arrays(self) -> dict:
        """Views of the plan's device arrays (int32 tensors inside the plan workspace)."""
        n, M, C = self.n, self.num_blocks, self.num_cells
        if n == 0:
            return {}
        i = self.info
        a = {"perm": self._view(i.perm, n), "blk_off": self._view(i.blk_off, M + 1),
             "blk_key": self._view(i.blk_key, M), "tok2blk": self._view(i.tok2blk, n),
             "lpt": self._view(i.lpt, M)}
        if self.cells_are_block_unions:
            a.update(blk_cell=self._view(i.blk_cell, M), cell_off=self._view(i.cell_off, C + 1),
                     cell_blk=self._view(i.cell_blk, M))
        else:
            Cw = self.num_wcells
            a.update(wperm=self._view(i.wperm, n), wcell_off=self._view(i.wcell_off, Cw + 1),
                     wlpt=self._view(i.wlpt, Cw))
        return a

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            lib.ssa_plan_destroy(h)
            self.handle = None


def forward_max_blocks(dtype, dim: int) -> int:
    """Largest number of occupied blocks the forward accepts for dtype and dim (0: unknown)."""
    return int(lib.ssa_forward_max_blocks(_DTYPES[dtype], dim))


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
    # W [d,d] (mean pool + linear map), or [B^3,d,d] position weights (sparse convolution)
    wshape = (d, d) if wk.dim() == 2 else (plan.block ** 3, d, d)
    if N != plan.n or k.shape != q.shape or v.shape != q.shape or gates.shape != (N, H, 3) \
            or wk.shape != wshape or wv.shape != wshape:
        raise ValueError("shape mismatch")
    return N, H, d


def forward(plan: Plan, q, k, v, wk, wv, gates, topk: int, scale: float = 0.0, out=None,
            sel_out=None, ws=None, stream=None, stages: int = STAGE_ALL, want_sel: bool = True,
            save_for_bwd: bool = False):
    """SSA forward (ssa_forward_stages).  q,k,v [N,H,d], gates [N,H,3], wk,wv [d,d], one dtype;
    wk, wv of shape [B^3,d,d] select the sparse-convolution compressor (ssa_forward_conv).
    Returns (out [N,H,d], sel [H,M,topk] int32 or None).  With save_for_bwd, `ws` must be
    kept and passed to backward()."""
    N, H, d = _check_qkv(plan, q, k, v, wk, wv, gates)
    dt = _DTYPES[q.dtype]
    size = lib.ssa_forward_workspace_size(plan.handle, dt, H, d, topk, int(save_for_bwd))
    if size == 0:
        raise SSAError(2, "ssa_forward_workspace_size")
    _uses(stream, q, k, v, wk, wv, gates, out, sel_out, ws, plan.ws)
    with _alloc_on(stream):
        if out is None:
            out = torch.empty_like(q)
        if sel_out is None and want_sel:
            sel_out = torch.empty((H, max(plan.num_blocks, 1), topk), dtype=torch.int32,
                                  device=q.device)
        if ws is None or ws.numel() < size:
            ws = torch.empty(size, dtype=torch.uint8, device=q.device)
    args = (plan.handle, dt, H, d, _ptr(q), _ptr(k), _ptr(v), _ptr(wk), _ptr(wv), _ptr(gates), int(topk),
            float(scale), _ptr(out), _ptr(sel_out), _ptr(ws), ws.numel(), int(save_for_bwd), _stream(stream))
    if wk.dim() == 3:       # the sparse-convolution compressor (all stages)
        if stages != STAGE_ALL:
            raise ValueError("the sparse-convolution forward runs all stages")
        st = lib.ssa_forward_conv(*args)
    else:
        st = lib.ssa_forward_stages(*args, int(stages))
    _check(st, "ssa_forward")
    return out, sel_out


def forward_noalloc(plan: Plan, q, k, v, wk, wv, gates, topk: int, out, sel_out=None,
                    scale: float = 0.0, stream=None):
    """SSA forward through ssa_forward_noalloc: no workspace; `out` [N,H,d] (and `sel_out`
    [H,M,topk] int32, optional) are the caller's.  Allocates nothing."""
    N, H, d = _check_qkv(plan, q, k, v, wk, wv, gates)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must match q")
    if sel_out is not None and (sel_out.dtype != torch.int32 or not sel_out.is_contiguous()
                                or sel_out.numel() < H * max(plan.num_blocks, 1) * topk):
        raise ValueError("sel_out must be a contiguous int32 tensor [H, M, topk]")
    _uses(stream, q, k, v, wk, wv, gates, out, sel_out, plan.ws)
    st = lib.ssa_forward_noalloc(plan.handle, _DTYPES[q.dtype], H, d, _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(wk), _ptr(wv), _ptr(gates), int(topk), float(scale),
                                 _ptr(out), _ptr(sel_out), _stream(stream))
    _check(st, "ssa_forward_noalloc")
    return out, sel_out


def forward_batch_workspace_size(plans, dtype, heads: int, dim: int, topk: int) -> int:
    handles = (_vp * len(plans))(*[p.handle.value for p in plans])
    return int(lib.ssa_forward_batch_workspace_size(handles, len(plans), _DTYPES[dtype], heads, dim, topk))


def forward_batch(plans, tok_off, q, k, v, wk, wv, gates, topk: int, scale: float = 0.0, out=None,
                  ws=None, stream=None):
    """SSA forward of several samples (ssa_forward_batch): sample i owns tokens
    [tok_off[i], tok_off[i+1]) of the concatenated q, k, v, gates [N_total,H,d|3] and has its
    own plan plans[i].  Returns out [N_total,H,d]."""
    N, H, d = q.shape
    for t in (q, k, v, wk, wv, gates):
        if t.dtype != q.dtype or not t.is_contiguous() or t.device != q.device:
            raise ValueError("all tensors must be contiguous, on one device, with one dtype")
    if k.shape != q.shape or v.shape != q.shape or gates.shape != (N, H, 3) or wk.shape != (d, d) \
            or wv.shape != (d, d) or int(tok_off[-1]) != N or len(tok_off) != len(plans) + 1:
        raise ValueError("shape mismatch")
    dt = _DTYPES[q.dtype]
    handles = (_vp * len(plans))(*[p.handle.value for p in plans])
    offs = (_i64 * len(tok_off))(*[int(x) for x in tok_off])
    size = lib.ssa_forward_batch_workspace_size(handles, len(plans), dt, H, d, topk)
    if size == 0:
        raise SSAError(2, "ssa_forward_batch_workspace_size")
    _uses(stream, q, k, v, wk, wv, gates, out, ws, *[p.ws for p in plans])
    with _alloc_on(stream):
        if out is None:
            out = torch.empty_like(q)
        if ws is None or ws.numel() < size:
            ws = torch.empty(size, dtype=torch.uint8, device=q.device)
    st = lib.ssa_forward_batch(handles, len(plans), offs, dt, H, d, _ptr(q), _ptr(k), _ptr(v), _ptr(wk),
                               _ptr(wv), _ptr(gates), int(topk), float(scale), _ptr(out), _ptr(ws),
                               ws.numel(), _stream(stream))
    _check(st, "ssa_forward_batch")
    return out


def qkv_gates(x, w_qkv, w_gate, b_gate, gamma_q, gamma_k, coords, heads: int, dim: int,
              rope_base: float = 0.0, eps: float = 0.0, out=None, stream=None):
    """ssa_qkv_gates: q, k, v [N,H,d] and gates [N,H,3] from token features x [N,C] (one dtype,
    f16 or bf16; W in linear-layer layout [out, C]; b_gate may be None).  Returns (q, k, v, gates)."""
    N, C = x.shape
    H, d = heads, dim
    for t in (x, w_qkv, w_gate, gamma_q, gamma_k) + ((b_gate,) if b_gate is not None else ()):
        if t.dtype != x.dtype or not t.is_contiguous() or t.device != x.device:
            raise ValueError("all tensors must be contiguous, on one device, with one dtype")
    if w_qkv.shape != (3 * H * d, C) or w_gate.shape != (3 * H, C) or gamma_q.shape != (d,) \
            or gamma_k.shape != (d,) or coords.shape != (N, 3) or coords.dtype != torch.int32 \
            or (b_gate is not None and b_gate.shape != (3 * H,)):
        raise ValueError("shape mismatch")
    _uses(stream, x, w_qkv, w_gate, b_gate, gamma_q, gamma_k, coords)
    with _alloc_on(stream):
        if out is None:
            out = (torch.empty((N, H, d), dtype=x.dtype, device=x.device),
                   torch.empty((N, H, d), dtype=x.dtype, device=x.device),
                   torch.empty((N, H, d), dtype=x.dtype, device=x.device),
                   torch.empty((N, H, 3), dtype=x.dtype, device=x.device))
    q, k, v, g = out
    st = lib.ssa_qkv_gates(_DTYPES[x.dtype], N, C, H, d, _ptr(x), _ptr(w_qkv), _ptr(w_gate), _ptr(b_gate),
                           _ptr(gamma_q), _ptr(gamma_k), _ptr(coords), float(rope_base), float(eps),
                           _ptr(q), _ptr(k), _ptr(v), _ptr(g), _stream(stream))
    _check(st, "ssa_qkv_gates")
    return q, k, v, g


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
    size = lib.ssa_backward_workspace_size(plan.handle, dt, H, d, topk)
    if size == 0:
        raise SSAError(2, "ssa_backward_workspace_size")
    _uses(stream, q, k, v, wk, wv, gates, sel, dout, fwd_ws, ws, plan.ws)
    with _alloc_on(stream):
        dq, dk, dv = (torch.empty(q.shape, **f32), torch.empty(q.shape, **f32),
                      torch.empty(q.shape, **f32))
        dg = torch.empty((N, H, 3), **f32)
        if ws is None or ws.numel() < size:
            ws = torch.empty(size, dtype=torch.uint8, device=q.device)
    fn = lib.ssa_backward_conv if wk.dim() == 3 else lib.ssa_backward
    st = fn(plan.handle, dt, H, d, _ptr(q), _ptr(k), _ptr(v), _ptr(wk), _ptr(wv),
                          _ptr(gates), int(topk), float(scale), _ptr(sel), _ptr(dout), _ptr(dq),
                          _ptr(dk), _ptr(dv), _ptr(dg), _ptr(fwd_ws), fwd_ws.numel(), _ptr(ws),
                          ws.numel(), _stream(stream))
    _check(st, "ssa_backward")
    return dq, dk, dv, dg

"""The C ABI on the CPU: the library loads, exports every function ssa.h declares, and
its host-side argument checks return the documented status codes (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssa.h")


@pytest.fixture(scope="module")
def ssa():
    import spatial_sparse_attention_amd as m
    return m


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssa_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported(ssa):
    names = _declared()
    assert "ssa_forward" in names and "ssa_plan_create" in names
    out = subprocess.run(["nm", "-D", "--defined-only", ssa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (ssa_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(ssa.lib, n)


def test_status_strings(ssa):
    for code in range(8):
        assert ssa.lib.ssa_status_string(code)
    assert ssa.lib.ssa_status_string(99) == b"unknown status"


def _grid(g=(8, 8, 8)):
    return (ctypes.c_int32 * 3)(*g)


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: checks fail before any access


def test_plan_argument_errors(ssa):
    L = ssa.lib
    h = ctypes.c_void_p()
    ws = ctypes.create_string_buffer(1 << 16)
    size = L.ssa_plan_workspace_size(10, _grid(), 2, 2)
    assert size > 0
    assert L.ssa_plan_create(FAKE, 10, _grid(), 2, 2, ws, size, None, None) == 1
    assert L.ssa_plan_create(FAKE, -1, _grid(), 2, 2, ws, size, None, ctypes.byref(h)) == 1
    assert L.ssa_plan_create(FAKE, 10, _grid(), 0, 2, ws, size, None, ctypes.byref(h)) == 1
    assert L.ssa_plan_create(FAKE, 10, _grid(), 2, 0, ws, size, None, ctypes.byref(h)) == 1
    assert L.ssa_plan_create(FAKE, 10, _grid((8, 0, 8)), 2, 2, ws, size, None, ctypes.byref(h)) == 1
    assert L.ssa_plan_create(None, 10, _grid(), 2, 2, ws, size, None, ctypes.byref(h)) == 1
    # window descriptions (ssa_plan_create_ex): checked before any launch
    W = ssa.Window
    ex = lambda win, g=_grid(): L.ssa_plan_create_ex(FAKE, 10, g, 2, ctypes.byref(win), ws, size, None,
                                                    ctypes.byref(h))
    assert ex(W(7, 2, (ctypes.c_int32 * 3)(0, 0, 0), 0)) == 1          # unknown kind
    assert ex(W(0, 0, (ctypes.c_int32 * 3)(0, 0, 0), 0)) == 1          # zero edge
    assert ex(W(0, 4, (ctypes.c_int32 * 3)(0, -1, 0), 0)) == 1         # negative shift
    assert ex(W(0, 4, (ctypes.c_int32 * 3)(0, 4, 0), 0)) == 1          # shift >= edge
    assert ex(W(1, 0, (ctypes.c_int32 * 3)(0, 0, 0), 0)) == 1          # SFC without a window size
    assert ex(W(1, 0, (ctypes.c_int32 * 3)(0, 0, 0), 8), _grid((2048, 8, 8))) == 2  # Morton codes > 30 bits
    assert L.ssa_plan_create_ex(FAKE, 10, _grid(), 2, None, ws, size, None, ctypes.byref(h)) == 1
    # workspace missing / too small
    assert L.ssa_plan_create(FAKE, 10, _grid(), 2, 2, None, size, None, ctypes.byref(h)) == 3
    assert L.ssa_plan_create(FAKE, 10, _grid(), 2, 2, ws, size - 1, None, ctypes.byref(h)) == 3
    assert h.value is None


def test_empty_plan_and_forward_checks(ssa):
    L = ssa.lib
    h = ctypes.c_void_p()
    size = L.ssa_plan_workspace_size(0, _grid(), 2, 4)
    ws = ctypes.create_string_buffer(size)
    assert L.ssa_plan_create(None, 0, _grid(), 2, 4, ws, size, None, ctypes.byref(h)) == 0
    info = ssa.PlanInfo()
    assert L.ssa_plan_get_info(h, ctypes.byref(info)) == 0
    assert info.n == 0 and info.num_blocks == 0
    wsz = L.ssa_forward_workspace_size(h, 1, 2, 64, 4, 0)
    assert wsz > 0
    assert L.ssa_forward_workspace_size(h, 1, 2, 64, 4, 1) > wsz   # saved state for backward
    fws = ctypes.create_string_buffer(wsz)
    args = lambda dt=1, H=2, d=64, k=4, sc=0.0: (h, dt, H, d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, k,
                                                 ctypes.c_float(sc), FAKE, None, fws, wsz, 0, None)
    assert L.ssa_forward(*args()) == 0                 # N = 0: nothing to do
    assert L.ssa_forward(*args(dt=3)) == 1
    assert L.ssa_forward(*args(dt=-1)) == 1
    assert L.ssa_forward(*args(H=0)) == 1
    assert L.ssa_forward(*args(d=48)) == 2
    assert L.ssa_forward(*args(k=0)) == 1
    assert L.ssa_forward(*args(k=300)) == 2
    assert L.ssa_forward(*args(sc=-1.0)) == 1
    assert L.ssa_forward(*args(sc=float("nan"))) == 1
    assert L.ssa_forward(*args(sc=float("inf"))) == 1
    assert L.ssa_forward_stages(*(args() + (0,))) == 1
    assert L.ssa_forward_stages(*(args() + (8,))) == 1
    assert L.ssa_plan_get_info(h, None) == 1
    assert L.ssa_plan_get_info(None, ctypes.byref(info)) == 6
    assert L.ssa_forward(None, 1, 2, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, ctypes.c_float(0),
                         FAKE, None, fws, wsz, 0, None) == 6
    # backward
    bsz = L.ssa_backward_workspace_size(h, 1, 2, 64, 4)
    assert bsz > 0
    bws = ctypes.create_string_buffer(bsz)
    bargs = lambda dt=1, d=64, k=4, sc=0.0: (h, dt, 2, d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, k,
                                             ctypes.c_float(sc), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                             fws, wsz, bws, bsz, None)
    assert L.ssa_backward(*bargs()) == 0              # N = 0
    assert L.ssa_backward(*bargs(dt=5)) == 1
    assert L.ssa_backward(*bargs(d=80)) == 2
    assert L.ssa_backward(*bargs(k=0)) == 1
    assert L.ssa_backward(*bargs(sc=-2.0)) == 1
    assert L.ssa_backward(*((None,) + bargs()[1:])) == 6
    # several samples: argument checks before any launch
    plans = (ctypes.c_void_p * 1)(h.value)
    offs = (ctypes.c_int64 * 2)(0, 0)
    assert L.ssa_forward_batch_workspace_size(plans, 1, 1, 2, 64, 4) > 0
    assert L.ssa_forward_batch(None, 1, offs, 1, 2, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4,
                               ctypes.c_float(0), FAKE, fws, wsz, None) == 1
    bad = (ctypes.c_int64 * 2)(0, 5)                       # the plan holds 0 tokens
    assert L.ssa_forward_batch(plans, 1, bad, 1, 2, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4,
                               ctypes.c_float(0), FAKE, fws, wsz, None) == 1
    assert L.ssa_forward_batch(plans, 1, offs, 1, 2, 48, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4,
                               ctypes.c_float(0), FAKE, fws, wsz, None) == 2
    assert L.ssa_forward_batch(plans, 1, offs, 1, 2, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4,
                               ctypes.c_float(0), FAKE, fws, wsz, None) == 0
    L.ssa_plan_destroy(h)
    L.ssa_plan_destroy(None)


def test_qkv_gates_argument_errors(ssa):
    L = ssa.lib
    f = ctypes.c_float
    args = lambda dt=1, n=10, C=64, d=96: (dt, n, C, 2, d, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, f(0), f(0),
                                           FAKE, FAKE, FAKE, FAKE, None)
    assert L.ssa_qkv_gates(*args(n=0)) == 0           # nothing to do
    assert L.ssa_qkv_gates(*args(dt=0)) == 2          # f32
    assert L.ssa_qkv_gates(*args(dt=5)) == 1
    assert L.ssa_qkv_gates(*args(d=48)) == 2
    assert L.ssa_qkv_gates(*args(C=60)) == 2          # rows not 16-byte aligned
    assert L.ssa_qkv_gates(*args(C=0)) == 1
    bad = list(args())
    bad[5] = None
    assert L.ssa_qkv_gates(*bad) == 1                 # no features
    bad = list(args())
    bad[12] = f(-1.0)
    assert L.ssa_qkv_gates(*bad) == 1                 # negative rotary base


def test_max_blocks_argument_errors(ssa):
    L = ssa.lib
    assert L.ssa_forward_max_blocks(5, 64) == 0
    assert L.ssa_forward_max_blocks(-1, 64) == 0
    assert L.ssa_forward_max_blocks(1, 48) == 0
    assert L.ssa_forward_max_blocks(1, 96) >= 0      # 0 without a device


def test_workspace_sizes_monotone(ssa):
    L = ssa.lib
    a = L.ssa_plan_workspace_size(1000, _grid(), 2, 2)
    b = L.ssa_plan_workspace_size(100000, _grid(), 2, 2)
    assert 0 < a < b
    assert L.ssa_plan_workspace_size(-5, _grid(), 2, 2) == 0

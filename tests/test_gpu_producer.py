"""GPU parity of ssa_qkv_gates (the step that produces SSA's inputs: projections, RMS norm and
3D rotary embedding of q and k, sigmoid gates) against the oracle's float64 qkv_gates."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity import TOL, check_selection, compare, torch_dtype

pytestmark = pytest.mark.gpu


def _run(pin, coords, H, d, dt):
    import torch
    import spatial_sparse_attention_amd as ssa
    tdt = torch_dtype(dt)
    dev = {k: (torch.from_numpy(np.ascontiguousarray(v)).cuda().to(tdt) if v is not None else None)
           for k, v in pin.items()}
    c = torch.from_numpy(np.ascontiguousarray(coords, dtype=np.int32)).cuda()
    out = ssa.qkv_gates(dev["x"], dev["w_qkv"], dev["w_gate"], dev["b_gate"], dev["gamma_q"], dev["gamma_k"],
                        c, H, d)
    torch.cuda.synchronize()
    return [t.double().cpu().numpy() for t in out]


def _ref(pin, coords, H, d, rows=None):
    x = pin["x"] if rows is None else pin["x"][rows]
    c = coords if rows is None else coords[rows]
    return oracle.qkv_gates(x, pin["w_qkv"], pin["w_gate"], pin["b_gate"], pin["gamma_q"], pin["gamma_k"],
                            c, H, d)


CASES = [  # (N, C, H, d, dtype, bias, grid)
    (500, 64, 2, 32, "f16", True, 16),
    (1000, 200, 3, 96, "bf16", True, 64),      # C not a multiple of the 64-wide chunk
    (300, 128, 4, 128, "f16", False, 200),
    (700, 96, 2, 64, "bf16", True, 1000),      # large coordinates: large rotary angles
    (130, 24, 5, 96, "f16", True, 8),          # 3 H > d: two gate tiles; a ragged token tile
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[4]}_N{c[0]}_C{c[1]}_H{c[2]}_d{c[3]}" for c in CASES])
def test_qkv_gates_small(case):
    N, C, H, d, dt, bias, G = case
    rng = np.random.default_rng(N + C)
    coords = rng.integers(0, G, (N, 3)).astype(np.int32)
    pin = W.producer_inputs(N, C, H, d, dt, seed=N, bias=bias)
    got = _run(pin, coords, H, d, dt)
    ref = _ref(pin, coords, H, d)
    for name, a, b in zip(("q", "k", "v", "gates"), got, ref):
        compare(a, b, dt, name)


@pytest.mark.timeout(600)
def test_qkv_gates_full_shape_sampled():
    """The 80k-voxel block's producer (width 2,112, 22 heads x 96, fp16) in full on the GPU;
    4,096 tokens against the oracle (tokens are independent, so the oracle on those rows is
    exact)."""
    wl, base = W.make_inputs("shells80k")
    coords = base["coords"]
    N, C, H, d = len(coords), 2112, 22, 96
    pin = W.producer_inputs(N, C, H, d, "f16", seed=3)
    got = _run(pin, coords, H, d, "f16")
    rows = np.random.default_rng(0).choice(N, 4096, replace=False)
    ref = _ref(pin, coords, H, d, rows)
    for name, a, b in zip(("q", "k", "v", "gates"), got, ref):
        compare(a[rows], b, "f16", name)
        assert np.isfinite(a).all()


def test_producer_then_ssa():
    """Features -> q, k, v, gates -> SSA, on the GPU, against the oracle of both steps."""
    import torch
    import spatial_sparse_attention_amd as ssa
    N, G, C, H, d, dt = 1200, 16, 128, 2, 96, "f16"
    rng = np.random.default_rng(9)
    flat = rng.choice(G ** 3, N, replace=False)
    coords = np.stack(np.unravel_index(flat, (G,) * 3), -1).astype(np.int32)
    pin = W.producer_inputs(N, C, H, d, dt, seed=9)
    q, k, v, g = _run(pin, coords, H, d, dt)
    w = W.random_inputs(coords, H, d, dt, seed=9, grid=G)
    inp = {"coords": coords, "grid": G, "block": 4, "window": 4, "topk": 4, "dtype": dt,
           "q": q.astype(np.float32), "k": k.astype(np.float32), "v": v.astype(np.float32),
           "gates": g.astype(np.float32), "wk": w["wk"], "wv": w["wv"]}
    from parity import gpu_forward
    out, sel, plan = gpu_forward(inp)
    # the oracle of both steps; the GPU's fp16 q, k, v, gates feed the oracle's SSA so that
    # the selection rule compares like with like
    rq, rk, rv, rg = _ref(pin, coords, H, d)
    for name, a, b in zip(("q", "k", "v", "gates"), (q, k, v, g), (rq, rk, rv, rg)):
        compare(a, b, dt, name)
    ref = oracle.forward(inp)
    near = {}
    for h in range(H):
        for b in range(ref["part"].M):
            if check_selection(ref["sigma"][h, b], 4, sel[h, b]) == "near":
                near[(h, b)] = sel[h, b]
    if near:
        ref = oracle.forward(inp, sel_override=near)
    compare(out, ref["out"], dt, "ssa output")

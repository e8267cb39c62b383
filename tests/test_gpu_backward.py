"""GPU backward parity: dQ, dK, dV and gate gradients against the oracle's float64 analytic
backward, with the selection the GPU forward chose held fixed."""
import numpy as np
import pytest

import oracle
import workloads as W
from brute import tiny_case
from parity import check_backward_all, check_forward_all, compare_grad, gpu_backward

pytestmark = pytest.mark.gpu

CASES = [  # (N, G, H, d, B, w, k, dtype)
    (300, 12, 2, 32, 2, 2, 3, "f32"),
    (600, 12, 2, 64, 2, 4, 3, "f32"),
    (600, 12, 2, 96, 3, 3, 4, "f32"),
    (500, 12, 1, 128, 2, 2, 4, "f32"),
    (1500, 20, 2, 32, 4, 4, 4, "f16"),
    (1500, 20, 2, 64, 4, 4, 4, "f16"),
    (1500, 20, 2, 96, 4, 4, 4, "f16"),
    (1500, 20, 2, 32, 4, 8, 4, "bf16"),
    (1200, 16, 2, 128, 4, 8, 2, "bf16"),
    (2000, 24, 1, 96, 3, 6, 5, "f16"),
    (800, 10, 2, 64, 2, 100, 100, "bf16"),
    (700, 9, 1, 32, 1, 1, 6, "f32"),
    (400, 8, 2, 96, 8, 8, 3, "f16"),
    (3000, 40, 2, 64, 2, 2, 4, "f16"),      # ~2,500 blocks
    (7000, 40, 1, 32, 1, 1, 8, "f32"),      # 7,000 single-token blocks
]


def _inputs(case, distinct=True, scale=None):
    N, G, H, d, B, w, k, dt = case
    rng = np.random.default_rng(N * 11 + d)
    c = tiny_case(rng, N, G, H, d, distinct=distinct)
    inp = W.random_inputs(c["coords"], H, d, dt, seed=N + 7 * d, grid=G, backward=True)
    inp.update(block=B, window=w, topk=k)
    if scale is not None:
        inp["scale"] = scale
    return inp


def _check(inp):
    out, sel, dq, dk, dv, dg = gpu_backward(inp, inp["do"])
    rq, rk, rv, rg = oracle.backward(inp, sel, inp["do"], scale=inp.get("scale"))
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv), ("dgates", dg, rg)):
        compare_grad(got, ref, inp["dtype"], name)


@pytest.mark.parametrize("case", CASES, ids=[f"{c[7]}_d{c[3]}_B{c[4]}_w{c[5]}_k{c[6]}_N{c[0]}" for c in CASES])
def test_backward_small(case):
    _check(_inputs(case))


@pytest.mark.parametrize("case,scale", [((1500, 20, 2, 64, 4, 4, 4, "f16"), 0.05),
                                        ((600, 12, 2, 32, 2, 4, 3, "f32"), 0.3)])
def test_backward_explicit_scale(case, scale):
    _check(_inputs(case, scale=scale))


def test_backward_duplicate_coordinates():
    inp = _inputs((1500, 12, 2, 64, 4, 4, 4, "f16"), distinct=False)
    assert len(np.unique(inp["coords"], axis=0)) < len(inp["coords"])
    _check(inp)


def test_backward_rejects_other_scale():
    """The saved log-sum-exp values hold the forward's scale: a backward with another one
    is refused."""
    import torch
    import spatial_sparse_attention_amd as ssa
    from parity import to_dev
    inp = _inputs((600, 12, 2, 64, 2, 4, 3, "f16"))
    dev = to_dev(inp)
    plan = ssa.Plan(dev["coords"], inp["grid"], inp["block"], inp["window"])
    N, H, d = dev["q"].shape
    fws = torch.empty(ssa.forward_workspace_size(plan, dev["q"].dtype, H, d, 3, True),
                      dtype=torch.uint8, device="cuda")
    args = (dev["q"], dev["k"], dev["v"], dev["wk"], dev["wv"], dev["gates"], 3)
    out, sel = ssa.forward(plan, *args, 0.2, ws=fws, save_for_bwd=True)
    do = torch.ones_like(dev["q"])
    with pytest.raises(ssa.SSAError) as e:
        ssa.backward(plan, *args, sel, do, fws, scale=0.0)
    assert e.value.status == 1
    ssa.backward(plan, *args, sel, do, fws, scale=0.2)
    torch.cuda.synchronize()


@pytest.mark.timeout(900)
def test_backward_shells80k_all_heads():
    """The 80k-voxel backward workload (22 heads x 96, fp16, W_v != W_k) in full on the GPU:
    its forward output and selection, and dq, dk, dv, dgates of all 22 heads, against the
    oracle (run per head in a process pool)."""
    wl, inp = W.make_inputs("shells80k_bwd", distinct_w=True)
    out, sel, dq, dk, dv, dg = gpu_backward(inp, inp["do"])
    counts, mx, rel = check_forward_all(inp, out, sel)
    print(f"forward: rows exact {counts['exact']} near {counts['near']}; max-abs {mx:.3g} rel {rel:.3g}")
    res = check_backward_all(inp, sel, (dq, dk, dv, dg))
    print("backward:", res)


def test_backward_deterministic():
    rng = np.random.default_rng(5)
    c = tiny_case(rng, 1500, 20, 2, 64)
    inp = W.random_inputs(c["coords"], 2, 64, "f16", seed=3, grid=20, backward=True)
    inp.update(block=4, window=4, topk=4)
    a = gpu_backward(inp, inp["do"])
    b = gpu_backward(inp, inp["do"])
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)

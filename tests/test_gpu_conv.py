"""GPU parity of the sparse-convolution compressor (ssa_forward_conv, ssa_backward_conv)
against the oracle's pool_conv path, forward and backward."""
import numpy as np
import pytest

import oracle
import workloads as W
from brute import tiny_case
from parity import check_forward_all, check_selection, compare, compare_grad, to_dev

pytestmark = pytest.mark.gpu

CASES = [  # (N, G, H, d, B, w, k, dtype)
    (1500, 20, 2, 64, 4, 4, 4, "f16"),
    (900, 16, 2, 96, 2, 4, 5, "bf16"),
    (400, 10, 1, 32, 2, 2, 3, "f32"),
    (1200, 16, 2, 128, 4, 8, 3, "f16"),
]


def _inputs(case, seed=0):
    N, G, H, d, B, w, k, dt = case
    rng = np.random.default_rng(N + d + seed)
    c = tiny_case(rng, N, G, H, d)
    inp = W.random_inputs(c["coords"], H, d, dt, seed=N + seed, grid=G, backward=True)
    inp.update(block=B, window=w, topk=k)
    inp["wk_conv"], inp["wv_conv"] = W.conv_weights(B, d, dt, seed=N)
    return inp


def _dev_conv(inp, tdt):
    import torch
    return (torch.from_numpy(inp["wk_conv"]).cuda().to(tdt), torch.from_numpy(inp["wv_conv"]).cuda().to(tdt))


def _gpu(inp, save=False):
    import torch
    import spatial_sparse_attention_amd as ssa
    dev = to_dev(inp)
    wkc, wvc = _dev_conv(inp, dev["q"].dtype)
    plan = ssa.Plan(dev["coords"], inp["grid"], inp["block"], inp["window"])
    N, H, d = dev["q"].shape
    ws = torch.empty(ssa.forward_workspace_size(plan, dev["q"].dtype, H, d, inp["topk"], save),
                     dtype=torch.uint8, device="cuda")
    out, sel = ssa.forward(plan, dev["q"], dev["k"], dev["v"], wkc, wvc, dev["gates"], inp["topk"], ws=ws,
                           save_for_bwd=save)
    return dev, plan, (wkc, wvc), ws, out, sel


def _check_forward(inp, out, sel):
    H, k = inp["q"].shape[1], inp["topk"]
    ref = oracle.forward(inp)
    near = {}
    for h in range(H):
        for b in range(ref["part"].M):
            if check_selection(ref["sigma"][h, b], k, sel[h, b]) == "near":
                near[(h, b)] = sel[h, b]
    if near:
        ref = oracle.forward(inp, sel_override=near)
    compare(out, ref["out"], inp["dtype"], "conv forward")


@pytest.mark.parametrize("case", CASES, ids=[f"{c[7]}_d{c[3]}_B{c[4]}" for c in CASES])
def test_forward_conv_small(case):
    import torch
    inp = _inputs(case)
    dev, plan, wc, ws, out, sel = _gpu(inp)
    torch.cuda.synchronize()
    _check_forward(inp, out.double().cpu().numpy(), sel.cpu().numpy())


def test_uniform_position_weights_equal_mean_pool():
    """Wc[o] = W^T at every position: the same selection and (to rounding) the same output as
    the mean pool + linear map forward."""
    import torch
    import spatial_sparse_attention_amd as ssa
    inp = _inputs(CASES[0])
    B, d = inp["block"], inp["q"].shape[2]
    inp["wk_conv"] = np.broadcast_to(inp["wk"].T, (B ** 3, d, d)).copy()
    inp["wv_conv"] = np.broadcast_to(inp["wv"].T, (B ** 3, d, d)).copy()
    dev, plan, wc, ws, out, sel = _gpu(inp)
    out2, sel2 = ssa.forward(plan, dev["q"], dev["k"], dev["v"], dev["wk"], dev["wv"], dev["gates"], inp["topk"])
    torch.cuda.synchronize()
    np.testing.assert_allclose(out.double().cpu().numpy(), out2.double().cpu().numpy(), atol=2e-3)


@pytest.mark.parametrize("case", CASES[:3], ids=[f"{c[7]}_d{c[3]}_B{c[4]}" for c in CASES[:3]])
def test_backward_conv_small(case):
    import torch
    import spatial_sparse_attention_amd as ssa
    inp = _inputs(case, seed=1)
    dev, plan, (wkc, wvc), ws, out, sel = _gpu(inp, save=True)
    do = torch.from_numpy(inp["do"]).cuda().to(dev["q"].dtype)
    dq, dk, dv, dg = ssa.backward(plan, dev["q"], dev["k"], dev["v"], wkc, wvc, dev["gates"], inp["topk"], sel,
                                  do, ws)
    with pytest.raises(ssa.SSAError) as e:   # a mean-pool backward on a convolution forward's state
        ssa.backward(plan, dev["q"], dev["k"], dev["v"], dev["wk"], dev["wv"], dev["gates"], inp["topk"], sel,
                     do, ws)
    assert e.value.status == 1
    torch.cuda.synchronize()
    rq, rk, rv, rg = oracle.backward(inp, sel.cpu().numpy().astype(np.int64), inp["do"])
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv), ("dgates", dg, rg)):
        compare_grad(got.double().cpu().numpy(), ref, inp["dtype"], name)


@pytest.mark.timeout(900)
def test_forward_conv_full_shape():
    """The 80k-voxel workload (22 x 96 fp16) with the sparse-convolution compressor (8^3
    position weights): every output element and selection row."""
    import torch
    wl, base = W.make_inputs("shells80k", distinct_w=True)
    inp = dict(base)
    inp["wk_conv"], inp["wv_conv"] = W.conv_weights(8, 96, "f16", seed=3)
    dev, plan, wc, ws, out, sel = _gpu(inp)
    torch.cuda.synchronize()
    counts, mx, rel = check_forward_all(inp, out.double().cpu().numpy(), sel.cpu().numpy().astype(np.int64))
    print(f"rows exact {counts['exact']} near {counts['near']}; max-abs {mx:.3g} rel-L2 {rel:.3g}")

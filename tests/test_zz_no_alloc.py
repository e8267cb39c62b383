"""ssa_forward_noalloc (the forward for callers that cannot allocate: its workspace is a
fixed device array of the library) against ssa_forward with a caller workspace, through
the C ABI: two calls in a row, the second on a smaller problem, plus the size limit."""
import numpy as np
import pytest

import oracle
import workloads as W
from brute import tiny_case
from parity import compare, to_dev

pytestmark = pytest.mark.gpu


def _problem(N, G, H, d, B, w, k, dt, seed):
    rng = np.random.default_rng(seed)
    c = tiny_case(rng, N, G, H, d)
    inp = W.random_inputs(c["coords"], H, d, dt, seed=seed, grid=G)
    inp.update(block=B, window=w, topk=k)
    return inp


def _both(inp):
    import torch
    import spatial_sparse_attention_amd as ssa
    dev = to_dev(inp)
    plan = ssa.Plan(dev["coords"], inp["grid"], inp["block"], inp["window"])
    args = (dev["q"], dev["k"], dev["v"], dev["wk"], dev["wv"], dev["gates"], inp["topk"])
    ref_out, ref_sel = ssa.forward(plan, *args)
    out = torch.full_like(dev["q"], float("nan"))
    sel = torch.full_like(ref_sel, -7)
    ssa.forward_noalloc(plan, *args, out, sel)
    torch.cuda.synchronize()
    return (out.double().cpu().numpy(), sel.cpu().numpy(), ref_out.double().cpu().numpy(),
            ref_sel.cpu().numpy())


def test_noalloc_matches_forward_twice():
    # first call: ~2,000 blocks (both selection paths' code shared), then a smaller problem
    # that reuses the array holding the first call's contents
    for N, G, H, d, B, w, k, dt, seed in ((3000, 30, 3, 64, 2, 4, 5, "f16", 1),
                                          (700, 12, 2, 64, 2, 2, 3, "f16", 2)):
        inp = _problem(N, G, H, d, B, w, k, dt, seed)
        out, sel, ref_out, ref_sel = _both(inp)
        np.testing.assert_array_equal(sel, ref_sel)
        np.testing.assert_array_equal(out, ref_out)
        # and to the oracle's bar, with the same selection
        ref = oracle.forward(inp, sel_override={(h, b): sel[h, b] for h in range(H)
                                                for b in range(sel.shape[1])})
        compare(out, ref["out"], dt, "noalloc vs oracle")


def test_noalloc_rejects_too_large():
    import torch
    import spatial_sparse_attention_amd as ssa
    rng = np.random.default_rng(3)
    N, G, H, d = 40000, 64, 22, 96
    flat = rng.choice(G ** 3, N, replace=False)
    coords = torch.from_numpy(np.stack(np.unravel_index(flat, (G,) * 3), -1).astype(np.int32)).cuda()
    plan = ssa.Plan(coords, G, 8, 8)
    need = ssa.forward_workspace_size(plan, torch.float16, H, d, 8) - 256
    assert need > ssa.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((N, H, d), dtype=torch.float16, device="cuda")
    wm = torch.zeros((d, d), dtype=torch.float16, device="cuda")
    g = torch.zeros((N, H, 3), dtype=torch.float16, device="cuda")
    out = torch.empty_like(x)
    with pytest.raises(ssa.SSAError) as e:
        ssa.forward_noalloc(plan, x, x, x, wm, wm, g, 8, out)
    assert e.value.status == 7

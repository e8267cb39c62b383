"""Workspaces and outputs filled with NaN bit patterns (all bytes 0xFF: NaN in f32, f16 and
bf16, -1 in int32) before a call give the same bits as zero-filled ones: no kernel reads a
word of its workspace that the same call (or, for the backward, its forward) did not write.
Plan, forward (every window kind, both compressors, the in-kernel radix top-k), several
samples and the backward."""
import numpy as np
import pytest

import workloads as W
from brute import tiny_case

pytestmark = pytest.mark.gpu

FWD = [  # (N, G, H, d, B, w, k, dtype, window options)
    (1500, 20, 2, 64, 4, 4, 4, "f16", {}),
    (900, 12, 2, 96, 2, 4, 5, "bf16", {}),
    (600, 12, 2, 32, 2, 2, 3, "f32", {}),
    (3000, 40, 1, 64, 2, 2, 4, "f16", {}),                                # M > 1024
    (1200, 16, 2, 64, 4, 8, 3, "bf16", dict(window_shift=(4, 4, 4))),     # shifted cells
    (1500, 20, 2, 64, 4, 4, 4, "f16", dict(sfc_tokens=64)),               # Morton windows
    (1500, 20, 2, 64, 4, 2, 4, "f16", {}),                                # cells smaller than blocks
]


def _inputs(case, backward=False):
    N, G, H, d, B, w, k, dt, win = case
    rng = np.random.default_rng(N + d + B)
    c = tiny_case(rng, N, G, H, d)
    inp = W.random_inputs(c["coords"], H, d, dt, seed=N + 5 * d, grid=G, backward=backward)
    inp.update(block=B, window=w, topk=k, **win)
    return inp


def _filled(nbytes, fill):
    import torch
    return torch.full((max(int(nbytes), 1),), fill, dtype=torch.uint8, device="cuda")


def _like(t, fill):
    """A tensor of t's shape and dtype whose bytes are all `fill`."""
    return _filled(t.numel() * t.element_size(), fill)[: t.numel() * t.element_size()].view(t.dtype).view(t.shape)


def _plan(ssa, dev, inp, fill):
    import torch
    probe = ssa.Plan(dev["coords"], inp["grid"], inp["block"], inp["window"],
                     shift=inp.get("window_shift", (0, 0, 0)), sfc_tokens=inp.get("sfc_tokens", 0))
    ws = _filled(probe.ws.numel(), fill)
    del probe
    return ssa.Plan(dev["coords"], inp["grid"], inp["block"], inp["window"],
                    shift=inp.get("window_shift", (0, 0, 0)), sfc_tokens=inp.get("sfc_tokens", 0), ws=ws)


def _forward(inp, fill, conv=None):
    import torch
    import spatial_sparse_attention_amd as ssa
    from parity import to_dev
    dev = to_dev(inp)
    plan = _plan(ssa, dev, inp, fill)
    N, H, d = dev["q"].shape
    wk, wv = conv if conv is not None else (dev["wk"], dev["wv"])
    ws = _filled(ssa.forward_workspace_size(plan, dev["q"].dtype, H, d, inp["topk"]), fill)
    out = _like(dev["q"], fill)
    sel = _like(torch.empty((H, max(plan.num_blocks, 1), inp["topk"]), dtype=torch.int32, device="cuda"), fill)
    ssa.forward(plan, dev["q"], dev["k"], dev["v"], wk, wv, dev["gates"], inp["topk"], out=out, sel_out=sel, ws=ws)
    torch.cuda.synchronize()
    arrays = {k: v.clone() for k, v in plan.arrays().items()}
    return out.cpu(), sel.cpu(), arrays


def _same(a, b, what):
    import torch
    assert a.dtype == b.dtype and a.shape == b.shape, what
    assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), what


@pytest.mark.parametrize("case", FWD, ids=[f"{c[7]}_d{c[3]}_B{c[4]}_w{c[5]}" + ''.join('_' + o for o in c[8]) for c in FWD])
def test_forward_poisoned_workspaces(case):
    inp = _inputs(case)
    o0, s0, a0 = _forward(inp, 0)
    o1, s1, a1 = _forward(inp, 0xFF)
    _same(o0, o1, "out")
    _same(s0, s1, "sel")
    assert a0.keys() == a1.keys()
    for k in a0:
        _same(a0[k].cpu(), a1[k].cpu(), k)
    assert not o1.float().isnan().any()


def test_forward_conv_poisoned_workspaces():
    import torch
    inp = _inputs((1200, 16, 2, 64, 4, 4, 3, "f16", {}))
    wkc, wvc = W.conv_weights(4, 64, "f16", seed=3)
    conv = (torch.from_numpy(wkc).cuda().half(), torch.from_numpy(wvc).cuda().half())
    o0, s0, _ = _forward(inp, 0, conv)
    o1, s1, _ = _forward(inp, 0xFF, conv)
    _same(o0, o1, "out")
    _same(s0, s1, "sel")


def test_forward_batch_poisoned_workspace():
    import torch
    import spatial_sparse_attention_amd as ssa
    from parity import to_dev
    inps = [_inputs((n, 16, 2, 64, 4, 4, 3, "f16", {})) for n in (700, 1100)]
    devs = [to_dev(i) for i in inps]
    cat = {k: torch.cat([d[k] for d in devs]) for k in ("q", "k", "v", "gates")}
    outs = []
    for fill in (0, 0xFF):
        plans = [_plan(ssa, d, i, fill) for d, i in zip(devs, inps)]
        H, d = 2, 64
        ws = _filled(ssa.forward_batch_workspace_size(plans, torch.float16, H, d, 3), fill)
        out = _like(cat["q"], fill)
        tok_off = [0, 700, 1800]
        ssa.forward_batch(plans, tok_off, cat["q"], cat["k"], cat["v"], devs[0]["wk"], devs[0]["wv"],
                          cat["gates"], 3, out=out, ws=ws)
        torch.cuda.synchronize()
        outs.append(out.cpu())
    _same(outs[0], outs[1], "batch out")


@pytest.mark.parametrize("case", [(1500, 20, 2, 64, 4, 4, 4, "f16", {}), (900, 12, 2, 96, 2, 4, 5, "bf16", {}),
                                  (600, 12, 2, 32, 2, 2, 3, "f32", {}), (3000, 40, 1, 64, 2, 2, 4, "f16", {})],
                         ids=["f16_d64", "bf16_d96", "f32_d32", "f16_radix"])
@pytest.mark.parametrize("conv", [False, True], ids=["pool", "conv"])
def test_backward_poisoned_workspaces(case, conv):
    import torch
    import spatial_sparse_attention_amd as ssa
    from parity import to_dev
    inp = _inputs(case, backward=True)
    dev = to_dev(inp)
    N, H, d = dev["q"].shape
    tdt = dev["q"].dtype
    if conv:
        wkc, wvc = W.conv_weights(inp["block"], d, inp["dtype"], seed=5)
        wk, wv = torch.from_numpy(wkc).cuda().to(tdt), torch.from_numpy(wvc).cuda().to(tdt)
    else:
        wk, wv = dev["wk"], dev["wv"]
    dout = torch.from_numpy(np.ascontiguousarray(inp["do"])).cuda().to(tdt)
    res = []
    for fill in (0, 0xFF):
        plan = _plan(ssa, dev, inp, fill)
        k = inp["topk"]
        fws = _filled(ssa.forward_workspace_size(plan, tdt, H, d, k, True), fill)
        _, sel = ssa.forward(plan, dev["q"], dev["k"], dev["v"], wk, wv, dev["gates"], k, ws=fws,
                             save_for_bwd=True)
        bws = _filled(ssa.backward_workspace_size(plan, tdt, H, d, k), fill)
        grads = ssa.backward(plan, dev["q"], dev["k"], dev["v"], wk, wv, dev["gates"], k, sel, dout, fws, ws=bws)
        torch.cuda.synchronize()
        res.append([g.cpu() for g in grads])
    for name, a, b in zip(("dq", "dk", "dv", "dgates"), res[0], res[1]):
        _same(a, b, name)
        assert not b.isnan().any(), name

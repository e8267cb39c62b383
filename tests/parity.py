"""Helpers for GPU-vs-oracle parity: device upload, the selection rule for near ties,
and output tolerances (fp32: max-abs 1e-4; fp16/bf16: max-abs 2e-2 and rel-L2 5e-3)."""
import numpy as np

import oracle

TOL = {"f32": {"abs": 1e-4, "rel_l2": None}, "f16": {"abs": 2e-2, "rel_l2": 5e-3},
       "bf16": {"abs": 2e-2, "rel_l2": 5e-3}}
GAP = 1e-4


def torch_dtype(dt):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dt]


def to_dev(inp, dt=None):
    import torch
    dt = dt or inp["dtype"]
    tdt = torch_dtype(dt)
    dev = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to("cuda").to(tdt)
           for k in ("q", "k", "v", "wk", "wv", "gates")}
    dev["coords"] = torch.from_numpy(np.ascontiguousarray(inp["coords"], dtype=np.int32)).to("cuda")
    return dev


def gpu_forward(inp, dt=None, plan=None, stream=None):
    import torch
    import spatial_sparse_attention_amd as ssa
    dev = to_dev(inp, dt)
    if plan is None:
        plan = ssa.Plan(dev["coords"], inp["grid"], inp["block"], inp["window"])
    out, sel = ssa.forward(plan, dev["q"], dev["k"], dev["v"], dev["wk"], dev["wv"], dev["gates"],
                           inp["topk"], inp.get("scale", 0.0) or 0.0, stream=stream)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), sel.cpu().numpy().astype(np.int64), plan


def check_selection(sigma, k, row):
    """R18: exact set when the oracle's k-th/(k+1)-th relative gap is >= 1e-4; otherwise
    every clearly-better block must be chosen and only near-tied ones may differ.
    Returns 'exact' or 'near'."""
    M = len(sigma)
    kk = min(k, M)
    row = np.asarray(row)
    chosen = row[row >= 0]
    assert len(chosen) == kk, (row, kk)
    assert (row[kk:] == -1).all()
    assert np.all(np.diff(chosen) > 0), row
    assert chosen.min() >= 0 and chosen.max() < M
    order = np.lexsort((np.arange(M), -sigma))
    if kk == M:
        return "exact"
    sk, sk1 = sigma[order[kk - 1]], sigma[order[kk]]
    gap = (sk - sk1) / sk if sk > 0 else 0.0
    if gap >= GAP:
        assert set(chosen.tolist()) == set(order[:kk].tolist()), (sorted(chosen), sorted(order[:kk]), gap)
        return "exact"
    must = np.nonzero(sigma > sk * (1 + GAP))[0]
    assert set(must.tolist()) <= set(chosen.tolist())
    assert np.all(sigma[chosen] >= sk * (1 - GAP))
    return "near"


def compare(got, ref, dt, what=""):
    err = np.abs(got - ref)
    tol = TOL[dt]
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert err.max() <= tol["abs"], f"{what}: max-abs {err.max():.3g} > {tol['abs']}"
    if tol["rel_l2"] is not None:
        rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
        assert rel <= tol["rel_l2"], f"{what}: rel-L2 {rel:.3g} > {tol['rel_l2']}"
    return float(err.max())


def check_items(inp, out_gpu, sel_gpu, items, dt=None):
    """Oracle outputs for (head, block) items vs the GPU; near ties re-run with the GPU's
    selection.  Returns counts of exact and near-tie selections."""
    dt = dt or inp["dtype"]
    res = oracle.forward_items(inp, items)
    counts = {"exact": 0, "near": 0}
    forced = {}
    for it in items:
        h, b = it
        kind = check_selection(res[it]["sigma"], inp["topk"], sel_gpu[h, b])
        counts[kind] += 1
        if kind == "near":
            forced[it] = sel_gpu[h, b]
    if forced:
        res2 = oracle.forward_items(inp, list(forced), sel_override=forced,
                                    ktv=(res["ktil"], res["vtil"]))
        for it in forced:
            res[it] = res2[it]
    got = np.concatenate([out_gpu[res[it]["rows"], it[0]] for it in items])
    ref = np.concatenate([res[it]["out"] for it in items])
    compare(got, ref, dt, f"{len(items)} items")
    return counts


def gpu_backward(inp, dout, dt=None, plan=None):
    """GPU forward (saving state) + backward.  Returns numpy float64 (out, sel, dq, dk, dv, dg)."""
    import torch
    import spatial_sparse_attention_amd as ssa
    dev = to_dev(inp, dt)
    do = torch.from_numpy(np.ascontiguousarray(dout)).to("cuda").to(dev["q"].dtype)
    if plan is None:
        plan = ssa.Plan(dev["coords"], inp["grid"], inp["block"], inp["window"])
    N, H, d = dev["q"].shape
    fws = torch.empty(ssa.forward_workspace_size(plan, dev["q"].dtype, H, d, inp["topk"], True),
                      dtype=torch.uint8, device="cuda")
    out, sel = ssa.forward(plan, dev["q"], dev["k"], dev["v"], dev["wk"], dev["wv"], dev["gates"],
                           inp["topk"], 0.0, ws=fws, save_for_bwd=True)
    dq, dk, dv, dg = ssa.backward(plan, dev["q"], dev["k"], dev["v"], dev["wk"], dev["wv"],
                                  dev["gates"], inp["topk"], sel, do, fws)
    torch.cuda.synchronize()
    f = lambda t: t.double().cpu().numpy()
    return f(out), sel.cpu().numpy().astype(np.int64), f(dq), f(dk), f(dv), f(dg)


GRAD_TOL = {"f32": {"abs": 1e-3, "rel_l2": 1e-5}, "f16": {"abs": 2e-2, "rel_l2": 5e-3},
            "bf16": {"abs": 2e-2, "rel_l2": 5e-3}}


def compare_grad(got, ref, dt, what=""):
    tol = GRAD_TOL[dt]
    assert np.isfinite(got).all(), f"{what}: non-finite"
    err = np.abs(got - ref).max()
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert err <= tol["abs"], f"{what}: max-abs {err:.3g} > {tol['abs']} (rel-L2 {rel:.3g})"
    assert rel <= tol["rel_l2"], f"{what}: rel-L2 {rel:.3g} > {tol['rel_l2']}"
    return float(err), float(rel)

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
        plan = make_plan(inp, dev["coords"])
    out, sel = ssa.forward(plan, dev["q"], dev["k"], dev["v"], dev["wk"], dev["wv"], dev["gates"],
                           inp["topk"], inp.get("scale", 0.0) or 0.0, stream=stream)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), sel.cpu().numpy().astype(np.int64), plan


def make_plan(inp, coords_dev):
    """The GPU plan of an input dict, its window partition included."""
    import spatial_sparse_attention_amd as ssa
    return ssa.Plan(coords_dev, inp["grid"], inp["block"], inp["window"],
                    shift=inp.get("window_shift", (0, 0, 0)), sfc_tokens=inp.get("sfc_tokens", 0))


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
    """GPU forward (saving state) + backward.  Returns numpy float64 (out, sel, dq, dk, dv, dg).
    inp["scale"] (0 or missing: 1/sqrt(d)) is passed to both calls."""
    import torch
    import spatial_sparse_attention_amd as ssa
    dev = to_dev(inp, dt)
    do = torch.from_numpy(np.ascontiguousarray(dout)).to("cuda").to(dev["q"].dtype)
    if plan is None:
        plan = ssa.Plan(dev["coords"], inp["grid"], inp["block"], inp["window"])
    N, H, d = dev["q"].shape
    fws = torch.empty(ssa.forward_workspace_size(plan, dev["q"].dtype, H, d, inp["topk"], True),
                      dtype=torch.uint8, device="cuda")
    scale = inp.get("scale", 0.0) or 0.0
    out, sel = ssa.forward(plan, dev["q"], dev["k"], dev["v"], dev["wk"], dev["wv"], dev["gates"],
                           inp["topk"], scale, ws=fws, save_for_bwd=True)
    dq, dk, dv, dg = ssa.backward(plan, dev["q"], dev["k"], dev["v"], dev["wk"], dev["wv"],
                                  dev["gates"], inp["topk"], sel, do, fws, scale=scale)
    torch.cuda.synchronize()
    f = lambda t: t.double().cpu().numpy()
    return f(out), sel.cpu().numpy().astype(np.int64), f(dq), f(dk), f(dv), f(dg)


GRAD_TOL = {"f32": {"abs": 1e-4, "rel_l2": 1e-5}, "f16": {"abs": 2e-2, "rel_l2": 5e-3},
            "bf16": {"abs": 2e-2, "rel_l2": 5e-3}}


def compare_grad(got, ref, dt, what=""):
    """Gradients (fp32 outputs) against the oracle.  For bf16 inputs the max-abs bound grows with
    the gradient's magnitude past 8: the GPU's probabilities and pooled values enter the
    products in bf16 (unit roundoff 2^-9), so a gradient of size G carries errors of order
    G * 2^-9 -- at |G| = 8 that is bf16's own half-ulp, above 2e-2 (the rel-L2 bound stays)."""
    tol = GRAD_TOL[dt]
    assert np.isfinite(got).all(), f"{what}: non-finite"
    err = np.abs(got - ref).max()
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    bound = tol["abs"] * (max(1.0, float(np.abs(ref).max()) / 8.0) if dt == "bf16" else 1.0)
    assert err <= bound, f"{what}: max-abs {err:.3g} > {bound:.3g} (rel-L2 {rel:.3g}, max |ref| {np.abs(ref).max():.3g})"
    assert rel <= tol["rel_l2"], f"{what}: rel-L2 {rel:.3g} > {tol['rel_l2']}"
    return float(err), float(rel)


# ---------------------------------------------------------------- full-size parity in a process pool
class Stats:
    """Streaming max-abs and rel-L2 over many slices of one output tensor."""

    def __init__(self):
        self.max_abs, self.err2, self.ref2, self.n = 0.0, 0.0, 0.0, 0

    def add(self, got, ref):
        got = np.asarray(got, np.float64)
        ref = np.asarray(ref, np.float64)
        assert np.isfinite(got).all(), "non-finite output"
        e = got - ref
        if e.size:
            self.max_abs = max(self.max_abs, float(np.abs(e).max()))
        self.err2 += float((e * e).sum())
        self.ref2 += float((ref * ref).sum())
        self.n += e.size

    def rel_l2(self):
        return (self.err2 ** 0.5) / max(self.ref2 ** 0.5, 1e-30)

    def check(self, tol, what):
        assert self.max_abs <= tol["abs"], f"{what}: max-abs {self.max_abs:.3g} > {tol['abs']}"
        if tol.get("rel_l2") is not None:
            assert self.rel_l2() <= tol["rel_l2"], f"{what}: rel-L2 {self.rel_l2():.3g} > {tol['rel_l2']}"
        return self.max_abs, self.rel_l2()


def pool_forward_task(inp_h, h, payload, shared):
    """Worker (oracle.parallel): the oracle forward for `blocks` of head h, each selection row
    checked against the GPU's by the R18 rule; near ties re-run with the GPU's selection.
    Returns (list of (rows, out), counts)."""
    blocks, gpu_rows = payload
    ktv = (np.asarray(shared["ktil"][h:h + 1]), np.asarray(shared["vtil"][h:h + 1]))
    items = [(0, int(b)) for b in blocks]
    scale = inp_h.get("scale") or None
    res = oracle.forward_items(inp_h, items, ktv=ktv, scale=scale)
    counts = {"exact": 0, "near": 0}
    forced = {}
    for i, it in enumerate(items):
        try:
            kind = check_selection(res[it]["sigma"], inp_h["topk"], gpu_rows[i])
        except AssertionError as e:
            raise AssertionError(f"selection of head {h}, block {it[1]}: {e}") from None
        counts[kind] += 1
        if kind == "near":
            forced[it] = gpu_rows[i]
    if forced:
        res2 = oracle.forward_items(inp_h, list(forced), sel_override=forced, ktv=ktv, scale=scale)
        for it in forced:
            res[it] = res2[it]
    return [(res[it]["rows"], res[it]["out"]) for it in items], counts


def check_forward_all(inp, out_gpu, sel_gpu, heads=None, workers=None):
    """Every output element and every selection row of a forward, against the oracle run
    in a process pool (one task per (head, run of blocks)).  Returns (counts, max_abs, rel)."""
    from oracle.parallel import HeadPool, workers_available
    part = oracle.partition(inp["coords"], inp["block"], inp["grid"])
    ktil, vtil = oracle.compress(inp, inp["k"], inp["v"], part)
    N, H, d = inp["q"].shape
    heads = list(range(H)) if heads is None else list(heads)
    nw = workers or workers_available()
    per_head = max(1, -(-2 * nw // len(heads)))
    chunk = max(1, -(-part.M // per_head))
    tasks = []
    for h in heads:
        for b0 in range(0, part.M, chunk):
            blocks = list(range(b0, min(part.M, b0 + chunk)))
            tasks.append((h, (blocks, np.asarray(sel_gpu[h, b0:b0 + len(blocks)]))))
    st = Stats()
    counts = {"exact": 0, "near": 0}
    with HeadPool(inp, shared={"ktil": ktil, "vtil": vtil}, workers=nw) as hp:
        results = hp.map(pool_forward_task, tasks)
    for (h, _), (pieces, c) in zip(tasks, results):
        for kk in counts:
            counts[kk] += c[kk]
        for rows, ref in pieces:
            st.add(out_gpu[rows, h], ref)
    assert st.n == N * len(heads) * d
    mx, rel = st.check(TOL[inp["dtype"]], f"all outputs of {len(heads)} heads")
    return counts, mx, rel


def pool_backward_task(inp_h, h, payload, shared):
    """Worker (oracle.parallel): the oracle's float64 backward of head h with the selection held
    fixed.  Returns (dq, dk, dv, dg), each [N, 1, .]."""
    sel_h = np.asarray(payload)[None]
    return oracle.backward(inp_h, sel_h, inp_h["do"], scale=inp_h.get("scale") or None)


def check_backward_all(inp, sel_gpu, grads_gpu, heads=None, workers=None):
    """dq, dk, dv, dgates of every head against the oracle's backward in a process pool."""
    from oracle.parallel import HeadPool
    H = inp["q"].shape[1]
    heads = list(range(H)) if heads is None else list(heads)
    stats = [Stats() for _ in range(4)]
    with HeadPool(inp, workers=workers) as hp:
        results = hp.map(pool_backward_task, [(h, np.asarray(sel_gpu[h])) for h in heads])
    for h, ref in zip(heads, results):
        for s, got, r in zip(stats, grads_gpu, ref):
            s.add(got[:, h], r[:, 0])
    out = {}
    for name, s in zip(("dq", "dk", "dv", "dgates"), stats):
        out[name] = s.check(GRAD_TOL[inp["dtype"]], name)
    return out

"""Benchmark: SSA forward on one MI355X at the 80k-voxel sparse-transformer shape.

Workload "shells80k": 80,000 voxels from a seeded union of six ellipsoid shells in a
64^3 grid (about 30% occupancy, 1..512 tokens per 8^3 block), 22 heads x 96, fp16,
block 8^3, top-k 8, window 8^3 -- the shape of the first refinement pass on the
Sparc3D/Hi3D pipeline page ("How the pipeline works", "Stage 3").

A step is one pass of the whole path over resident inputs: the block partition
(ssa_plan_create) and the forward's three stages (pooled keys, compressed branch
+ selection, selected/window branches + gated combine).  HIP events on the launch
stream time every stage of every step.  The CPU baseline is the float64 oracle
timed on a bounded sample of the same workload on the host.
Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu] [--no-bwd] [--no-full] [--copy-probe]
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOAD = "shells80k"
PEAK_F16_TFLOPS = 2500.0      # MI355X dense fp16/bf16 MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def attend_traffic():
    """HBM bytes per k_attend dispatch at this workload from the committed rocprofv3 summary
    (FETCH_SIZE + WRITE_SIZE, calibrated), or None when the kernel sources it was measured on
    have changed since (digest mismatch) or the summary is missing."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "ssa_forward_shells80k_hbm_traffic.md")
    try:
        line = next(l for l in open(path) if l.startswith("traffic-record: "))
        rec = json.loads(line[len("traffic-record: "):])
        h = hashlib.sha256()
        for f in rec["digest_files"]:
            h.update(open(os.path.join(ROOT, "spatial_sparse_attention_amd", "csrc", f), "rb").read())
        if h.hexdigest()[:16] != rec["source_digest"]:
            return None
        return float(rec["fetch_bytes"] + rec["write_bytes"])
    except (OSError, StopIteration, ValueError, KeyError):
        return None


def attended_pairs(plan_arrays, sel, window_is_block):
    """Per-head sum over queries of (M + |selected keys| + |window keys|)."""
    blk_off = plan_arrays["blk_off"].astype(np.int64)
    sizes = np.diff(blk_off)
    M = len(sizes)
    H = sel.shape[0]
    sel_keys = np.where(sel >= 0, sizes[np.clip(sel, 0, M - 1)], 0).sum(axis=2)  # [H, M]
    cell_off = plan_arrays["cell_off"].astype(np.int64)
    cell_blk = plan_arrays["cell_blk"].astype(np.int64)
    cell_sizes = np.add.reduceat(sizes[cell_blk], cell_off[:-1]) if M else np.zeros(0)
    win_keys = cell_sizes[plan_arrays["blk_cell"].astype(np.int64)]           # [M]
    per_head = (sizes[None, :] * (M + sel_keys + win_keys[None, :])).sum(axis=1)
    return per_head, sizes


def workload_record(sizes, sel):
    """Per-run workload facts: blocks, occupancy histogram (block rows in powers of two),
    sum of squared block sizes (window pairs) and the mean size of a selected block."""
    edges = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1 << 30]
    hist = np.histogram(sizes, bins=edges)[0].tolist()
    chosen = sel[sel >= 0]
    return {"blocks": int(len(sizes)),
            "occupancy_hist": {f"{edges[i]}-{edges[i + 1] - 1}": int(hist[i]) for i in range(len(hist) - 1)
                               if edges[i] <= sizes.max()},
            "occupancy_min_median_mean_max": [int(sizes.min()), float(np.median(sizes)),
                                              float(sizes.mean()), int(sizes.max())],
            "sum_nb2": int((sizes.astype(np.int64) ** 2).sum()),
            "mean_selected_block_rows": float(sizes[chosen].mean()) if chosen.size else 0.0}


def cpu_baseline(inp, heads_sample):
    """The float64 oracle, as it stands, on `heads_sample` heads of the workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    t0 = time.perf_counter()
    part = oracle.partition(inp["coords"], inp["block"], inp["grid"])
    ktv = oracle.pool(inp["k"], inp["v"], inp["wk"], inp["wv"], part)
    items = [(h, b) for h in range(heads_sample) for b in range(part.M)]
    oracle.forward_items(inp, items, ktv=ktv)
    dt = time.perf_counter() - t0
    H = inp["q"].shape[1]
    N = inp["q"].shape[0]
    return {"value": N * (heads_sample / H) / dt, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"partition + pooling of all {H} heads, then all {part.M} blocks of "
                      f"{heads_sample} of {H} heads ({dt:.1f} s); tokens/s scaled by the head fraction"}


def full_attention_timing(ssa, coords, dev, wl, torch, stream, sparse_fwd_ms, reps=2):
    """Dense attention over every occupied voxel on the same kernels: a window cell covering
    the whole grid makes the window branch full attention (every query attends to all N
    keys); the selected and window branches' stage is timed (HIP events) and credited
    4 d N^2 H FLOPs.  The ratio to the sparse forward is the speed-up the method gives here."""
    q = dev["q"]
    N, H, d = q.shape
    plan = ssa.Plan(coords, wl.grid, wl.block, wl.grid)  # one window cell = the whole grid
    out = torch.empty_like(q)
    sel = torch.empty((H, plan.num_blocks, wl.topk), dtype=torch.int32, device="cuda")
    ws = torch.empty(ssa.forward_workspace_size(plan, q.dtype, H, d, wl.topk), dtype=torch.uint8, device="cuda")
    run = lambda st: ssa.forward(plan, q, dev["k"], dev["v"], dev["wk"], dev["wv"], dev["gates"], wl.topk, 0.0,
                                 out=out, sel_out=sel, ws=ws, stages=st)
    run(ssa.STAGE_POOL)
    run(ssa.STAGE_SELECT)
    run(ssa.STAGE_ATTEND)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run(ssa.STAGE_ATTEND)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = 4.0 * d * float(N) * float(N) * H
    return {"ms": ms, "tflops": flops / (ms * 1e-3) / 1e12, "reps": reps,
            "sparse_speedup": ms / sparse_fwd_ms,
            "what": "window cell = whole grid (dense attention over all voxels) on the same kernels; "
                    "selected/window stage only"}


def backward_timing(ssa, plan, dev, wl, torch, stream, reps=5):
    """Forward with saved state, then the backward (fixed selection, seeded dout), timed
    apart from the step: HIP events around `reps` backward calls."""
    q = dev["q"]
    N, H, d = q.shape
    gen = torch.Generator(device="cuda").manual_seed(5)
    dout = torch.randn(q.shape, generator=gen, device="cuda", dtype=torch.float32).to(q.dtype)
    fws = torch.empty(ssa.forward_workspace_size(plan, q.dtype, H, d, wl.topk, save_for_bwd=True),
                      dtype=torch.uint8, device="cuda")
    sel = torch.empty((H, plan.num_blocks, wl.topk), dtype=torch.int32, device="cuda")
    ssa.forward(plan, q, dev["k"], dev["v"], dev["wk"], dev["wv"], dev["gates"], wl.topk, 0.0,
                sel_out=sel, ws=fws, save_for_bwd=True)
    bws = torch.empty(ssa.backward_workspace_size(plan, q.dtype, H, d, wl.topk), dtype=torch.uint8,
                      device="cuda")
    run = lambda: ssa.backward(plan, q, dev["k"], dev["v"], dev["wk"], dev["wv"], dev["gates"],
                               wl.topk, sel, dout, fws, ws=bws)
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    return {"ms": e0.elapsed_time(e1) / reps, "reps": reps,
            "what": "dQ, dK, dV, dgates with the forward's selection held fixed (fp32 outputs)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-heads", type=int, default=22,
                    help="heads of the workload the CPU oracle runs (all 22: about 15 s)")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward timing")
    ap.add_argument("--no-full", action="store_true", help="skip the dense full-attention baseline")
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy 3 times (HBM counter calibration)")
    args = ap.parse_args()
    if args.copy_probe:
        import torch
        x = torch.ones(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": x.numel() * 4, "launches": 3}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: SSA shards by head with no exchange, and this "
              "build runs and reports the single-GPU path (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    import spatial_sparse_attention_amd as ssa

    wl, inp = W.make_inputs(args.workload)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[wl.dtype]
    dev = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).cuda().to(tdt)
           for k in ("q", "k", "v", "wk", "wv", "gates")}
    coords = torch.from_numpy(inp["coords"]).cuda()
    N, H, d = dev["q"].shape
    stream = torch.cuda.current_stream()

    plan = ssa.Plan(coords, wl.grid, wl.block, wl.window)
    out = torch.empty_like(dev["q"])
    sel = torch.empty((H, plan.num_blocks, wl.topk), dtype=torch.int32, device="cuda")
    ws = torch.empty(ssa.forward_workspace_size(plan, tdt, H, d, wl.topk), dtype=torch.uint8,
                     device="cuda")

    def step(evs=None):
        rec = (lambda i: evs[i].record(stream)) if evs else (lambda i: None)
        rec(0)
        p = ssa.Plan(coords, wl.grid, wl.block, wl.window)
        rec(1)
        for si, stage in enumerate((ssa.STAGE_POOL, ssa.STAGE_SELECT, ssa.STAGE_ATTEND)):
            ssa.forward(p, dev["q"], dev["k"], dev["v"], dev["wk"], dev["wv"], dev["gates"],
                        wl.topk, 0.0, out=out, sel_out=sel, ws=ws, stages=stage)
            rec(2 + si)
        return p

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    names = ["plan", "pool", "select", "attend"]
    stage_ms = {nm: float(np.mean([evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(args.steps)]))
                for i, nm in enumerate(names)}
    ms_step = wall * 1e3 / args.steps
    step_ev = [evs[s][0].elapsed_time(evs[s][4]) for s in range(args.steps)]
    fwd_ms = stage_ms["pool"] + stage_ms["select"] + stage_ms["attend"]

    # credited work: 4 d FLOPs per attended (query, key, head) pair over the three branches
    arrays = {k: v.cpu().numpy() for k, v in plan.arrays().items()}
    sel_np = sel.cpu().numpy()
    per_head, sizes = attended_pairs(arrays, sel_np, plan.num_cells == plan.num_blocks)
    flops = 4.0 * d * float(per_head.sum())
    M = plan.num_blocks
    cmp_flops = 4.0 * d * H * N * M               # the compressed branch alone
    es = 4 if wl.dtype == "f32" else 2
    alg_bytes = N * H * es * (4 * d + 3) + 12 * N + 2 * d * d * es
    peak = PEAK_F32_TFLOPS if wl.dtype == "f32" else PEAK_F16_TFLOPS
    sel_tflops = cmp_flops / (stage_ms["select"] * 1e-3) / 1e12
    # the dominant kernel: k_attend, the attend stage's only launch (selected + window branches
    # and the combine), credited 4 d FLOPs per attended selected or window pair
    att_flops = flops - cmp_flops
    att_tflops = att_flops / (stage_ms["attend"] * 1e-3) / 1e12
    res = {
        "metric": "SSA fwd tokens/s and TFLOP/s (% MFMA peak) at 80k voxels, 22h×96d fp16",
        "value": N / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {N} voxels, union of ellipsoid shells in a {wl.grid}^3 grid, "
                               f"block {wl.block}^3, top-k {wl.topk}, window {wl.window}^3, "
                               f"{H} heads x {d}, {wl.dtype}",
                   "N": N, "heads": H, "dim": d, "block": wl.block, "topk": wl.topk,
                   "window": wl.window, "blocks": M, "max_block_rows": int(sizes.max()),
                   "parallelism": "single GPU"},
        "tflops": flops / (ms_step * 1e-3) / 1e12,
        "mfma_peak_frac": flops / (ms_step * 1e-3) / 1e12 / peak,
        "forward_only": {"ms": fwd_ms, "tokens_per_s": N / (fwd_ms * 1e-3),
                         "tflops": flops / (fwd_ms * 1e-3) / 1e12,
                         "mfma_peak_frac": flops / (fwd_ms * 1e-3) / 1e12 / peak},
        "stage_ms": stage_ms,
        "step_ms_events": {"median": float(np.median(step_ev)), "min": float(np.min(step_ev))},
        "recorded": workload_record(sizes, sel_np),
        "credited_flops": flops,
        "algorithmic_bytes": alg_bytes,
        "roofline": {"kernel": "k_attend (selected + window branches, gated combine)", "bound": "mfma",
                     "achieved": att_tflops, "peak": peak, "unit": "TFLOP/s",
                     "frac": att_tflops / peak,
                     "traffic": attend_traffic() if wl.name == WORKLOAD else None,
                     "work_per_launch_flops": att_flops},
        "compressed_branch": {"kernels": "k_compress + k_select + k_topk", "ms": stage_ms["select"],
                              "tflops": sel_tflops, "mfma_peak_frac": sel_tflops / peak,
                              "work_flops": cmp_flops},
    }
    if not args.no_bwd:
        res["backward"] = backward_timing(ssa, plan, dev, wl, torch, stream)
    if not args.no_full:
        res["full_attention"] = full_attention_timing(ssa, coords, dev, wl, torch, stream, fwd_ms)
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(inp, min(args.cpu_heads, H))
    print(json.dumps(res))


if __name__ == "__main__":
    main()

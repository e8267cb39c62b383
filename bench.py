"""Benchmark: SSA forward on one MI355X at the 80k-voxel sparse-transformer shape.

Headline workload "shells80k": 80,000 voxels from a seeded union of six ellipsoid shells
in a 64^3 grid (1..487 tokens per occupied 8^3 block), 22 heads x 96, fp16, block 8^3,
top-k 8, window 8^3 -- the shape of the first refinement pass on the Sparc3D/Hi3D
pipeline page ("How the pipeline works", "Stage 3").

A step is one pass of the whole path over resident inputs: the block partition
(ssa_plan_create) and the forward's three stages (pooled keys, compressed branch +
selection, selected/window branches + gated combine).  HIP events on the launch stream
time every stage of every step.  The same line also reports the other workloads'
forwards (sphere2k, torus20k, shells110k), the backward at the 80k shape, dense
attention over every voxel on the same kernels at the 20k/80k/110k shapes, and the
float64 CPU oracle timed on a bounded sample of the headline workload in a process pool.
Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--quick] [--no-cpu] [--no-bwd]
                       [--no-full] [--no-others] [--workload NAME] [--copy-probe]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOAD = "shells80k"
BWD_WORKLOAD = "shells80k_bwd"
OTHERS = ("sphere2k", "torus20k", "shells110k")
DENSE = ("torus20k", "shells80k", "shells110k")
PEAK_F16_TFLOPS = 2500.0      # MI355X dense fp16/bf16 MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
SHAPES = {"sphere": "sphere shell of radius 12 in a {g}^3 grid",
          "torus": "torus surface (radii 80 and 30) in a {g}^3 grid",
          "ellipsoids6": "union of six ellipsoid shells in a {g}^3 grid",
          "ellipsoids10": "union of ten ellipsoid shells in a {g}^3 grid"}


def attend_traffic():
    """HBM bytes per k_attend dispatch at the headline workload from the committed rocprofv3
    summary (FETCH_SIZE + WRITE_SIZE, calibrated), or None when the kernel sources it was
    measured on have changed since (digest mismatch) or the summary is missing."""
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


HBM_PEAK_GBS = 8000.0


def attend_roofline(flops, alg_bytes, ms, peak_tflops, traffic):
    """Roofline of k_attend, the attend stage's one launch.  Its work: flops (4 d per attended
    selected or window pair).  Its algorithmic bytes are the method's: Q, K, V and gates read
    and O written -- all of which this kernel moves (every key is in some window cell); the
    compressed branch's output, an intermediate of the split into kernels that it also reads,
    is not counted.  The binding roof is the one its arithmetic intensity falls under: HBM
    below the ridge (peak FLOP/s over HBM bandwidth), MFMA above it; both fractions are given."""
    ai = flops / alg_bytes
    ridge = peak_tflops * 1e12 / (HBM_PEAK_GBS * 1e9)
    tflops = flops / (ms * 1e-3) / 1e12
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    hbm = ai < ridge
    return {"kernel": "k_attend (selected + window branches, gated combine)",
            "bound": "hbm" if hbm else "mfma",
            "achieved": gbs if hbm else tflops, "peak": HBM_PEAK_GBS if hbm else peak_tflops,
            "unit": "GB/s" if hbm else "TFLOP/s",
            "frac": gbs / HBM_PEAK_GBS if hbm else tflops / peak_tflops,
            "traffic": traffic,
            "arithmetic_intensity": ai, "ridge": ridge,
            "bytes_per_launch": alg_bytes, "flops_per_launch": flops,
            "mfma_tflops": tflops, "mfma_frac": tflops / peak_tflops,
            "hbm_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "launch_us_hip_events": ms * 1e3}


def attended_pairs(plan_arrays, sel):
    """Per-head sum over queries of (M + |selected keys| + |window keys|)."""
    blk_off = plan_arrays["blk_off"].astype(np.int64)
    sizes = np.diff(blk_off)
    M = len(sizes)
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


def describe(wl, N, H, d):
    shape = SHAPES[wl.shape].format(g=wl.grid)
    return (f"{wl.name}: {N} voxels, {shape}, block {wl.block}^3, top-k {wl.topk}, "
            f"window {wl.window}^3, {H} heads x {d}, {wl.dtype}")


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, heads_sample):
    """The float64 oracle, as it stands, on `heads_sample` heads of the workload, in a process
    pool (one BLAS thread per worker, one worker per host core this process may use)."""
    import oracle
    from oracle.parallel import HeadPool, forward_blocks_task, workers_available
    workers = workers_available()
    t0 = time.perf_counter()
    part = oracle.partition(inp["coords"], inp["block"], inp["grid"])
    ktil, vtil = oracle.pool(inp["k"], inp["v"], inp["wk"], inp["wv"], part)
    t_pool = time.perf_counter() - t0
    with HeadPool(inp, shared={"ktil": ktil, "vtil": vtil}, workers=workers) as hp:
        per_head = max(1, -(-2 * workers // heads_sample))
        chunk = max(1, -(-part.M // per_head))
        tasks = [(h, list(range(b0, min(part.M, b0 + chunk))))
                 for h in range(heads_sample) for b0 in range(0, part.M, chunk)]
        hp.map(forward_blocks_task, tasks[:workers])   # warm the workers (imports) outside the clock
        t1 = time.perf_counter()
        hp.map(forward_blocks_task, tasks)
        t_items = time.perf_counter() - t1
    H, N = inp["q"].shape[1], inp["q"].shape[0]
    dt = t_pool + t_items
    return {"value": N * (heads_sample / H) / dt, "unit": "tokens/s", "cores": int(workers),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"partition + pooling of all {H} heads ({t_pool:.1f} s, one process), then "
                      f"all {part.M} blocks of {heads_sample} of {H} heads in a pool of {workers} "
                      f"single-threaded processes ({t_items:.1f} s); tokens/s scaled by the head "
                      f"fraction"}


class Runner:
    """Inputs of one workload resident on the GPU, its plan and forward buffers."""

    def __init__(self, name, torch, ssa, W, distinct_w=False):
        self.torch, self.ssa = torch, ssa
        self.wl, self.inp = W.make_inputs(name, distinct_w=distinct_w)
        wl = self.wl
        self.tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[wl.dtype]
        self.dev = {k: torch.from_numpy(np.ascontiguousarray(self.inp[k])).cuda().to(self.tdt)
                    for k in ("q", "k", "v", "wk", "wv", "gates")}
        self.coords = torch.from_numpy(self.inp["coords"]).cuda()
        self.N, self.H, self.d = self.dev["q"].shape
        self.stream = torch.cuda.current_stream()
        self.plan = ssa.Plan(self.coords, wl.grid, wl.block, wl.window)
        self.out = torch.empty_like(self.dev["q"])
        self.sel = torch.empty((self.H, self.plan.num_blocks, wl.topk), dtype=torch.int32, device="cuda")
        self.ws = torch.empty(ssa.forward_workspace_size(self.plan, self.tdt, self.H, self.d, wl.topk),
                              dtype=torch.uint8, device="cuda")
        self.peak = PEAK_F32_TFLOPS if wl.dtype == "f32" else PEAK_F16_TFLOPS

    def fwd(self, plan, stage, out=None, sel=None, ws=None, save=False):
        d, wl = self.dev, self.wl
        return self.ssa.forward(plan, d["q"], d["k"], d["v"], d["wk"], d["wv"], d["gates"], wl.topk, 0.0,
                                out=self.out if out is None else out, sel_out=self.sel if sel is None else sel,
                                ws=self.ws if ws is None else ws, stages=stage, save_for_bwd=save)

    def step(self, evs=None):
        rec = (lambda i: evs[i].record(self.stream)) if evs else (lambda i: None)
        wl, ssa = self.wl, self.ssa
        rec(0)
        p = ssa.Plan(self.coords, wl.grid, wl.block, wl.window)
        rec(1)
        for si, stage in enumerate((ssa.STAGE_POOL, ssa.STAGE_SELECT, ssa.STAGE_ATTEND)):
            self.fwd(p, stage)
            rec(2 + si)
        return p

    def timed_steps(self, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(steps):
            self.step(evs[s])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        names = ["plan", "pool", "select", "attend"]
        stage_ms = {nm: float(np.mean([evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(steps)]))
                    for i, nm in enumerate(names)}
        step_ev = [evs[s][0].elapsed_time(evs[s][4]) for s in range(steps)]
        return wall * 1e3 / steps, stage_ms, step_ev

    def work(self):
        """Credited FLOPs (total, compressed branch, selected + window), bytes, sizes, sel."""
        arrays = {k: v.cpu().numpy() for k, v in self.plan.arrays().items()}
        sel_np = self.sel.cpu().numpy()
        per_head, sizes = attended_pairs(arrays, sel_np)
        d, H, N, M = self.d, self.H, self.N, self.plan.num_blocks
        flops = 4.0 * d * float(per_head.sum())
        cmp_flops = 4.0 * d * H * N * M
        es = 4 if self.wl.dtype == "f32" else 2
        alg_bytes = N * H * es * (4 * d + 3) + 12 * N + 2 * d * d * es
        return flops, cmp_flops, alg_bytes, sizes, sel_np, float(per_head.sum())

    def summary(self, steps, warmup):
        """Forward figures of this workload (for the non-headline entries)."""
        ms_step, stage_ms, step_ev = self.timed_steps(steps, warmup)
        flops, cmp_flops, _, sizes, sel_np, _ = self.work()
        fwd_ms = stage_ms["pool"] + stage_ms["select"] + stage_ms["attend"]
        tf = flops / (fwd_ms * 1e-3) / 1e12
        return {"workload": describe(self.wl, self.N, self.H, self.d), "steps": steps,
                "ms_per_step": ms_step, "stage_ms": stage_ms, "forward_ms": fwd_ms,
                "tokens_per_s": self.N / (ms_step * 1e-3), "credited_flops": flops,
                "forward_tflops": tf, "mfma_peak": self.peak, "mfma_peak_frac": tf / self.peak,
                "compressed_branch_frac": cmp_flops / (stage_ms["select"] * 1e-3) / 1e12 / self.peak,
                "attend_frac": (flops - cmp_flops) / (stage_ms["attend"] * 1e-3) / 1e12 / self.peak,
                "blocks": self.plan.num_blocks,
                "mean_selected_block_rows": workload_record(sizes, sel_np)["mean_selected_block_rows"]}


def full_attention_timing(r, sparse_fwd_ms, reps=2):
    """Dense attention over every occupied voxel on the same kernels: a window cell covering
    the whole grid makes the window branch full attention (every query attends to all N
    keys); the selected and window branches' stage is timed (HIP events) and credited
    4 d N^2 H FLOPs.  The ratio to the sparse forward is the speed-up the method gives here."""
    torch, ssa, wl = r.torch, r.ssa, r.wl
    N, H, d = r.N, r.H, r.d
    plan = ssa.Plan(r.coords, wl.grid, wl.block, wl.grid)  # one window cell = the whole grid
    out = torch.empty_like(r.dev["q"])
    sel = torch.empty((H, plan.num_blocks, wl.topk), dtype=torch.int32, device="cuda")
    ws = torch.empty(ssa.forward_workspace_size(plan, r.tdt, H, d, wl.topk), dtype=torch.uint8, device="cuda")
    run = lambda st: r.fwd(plan, st, out=out, sel=sel, ws=ws)
    run(ssa.STAGE_POOL)
    run(ssa.STAGE_SELECT)
    run(ssa.STAGE_ATTEND)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(r.stream)
    for _ in range(reps):
        run(ssa.STAGE_ATTEND)
    e1.record(r.stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = 4.0 * d * float(N) * float(N) * H
    tf = flops / (ms * 1e-3) / 1e12
    return {"ms": ms, "tflops": tf, "mfma_peak_frac": tf / r.peak, "reps": reps,
            "sparse_forward_ms": sparse_fwd_ms, "dense_over_sparse": ms / sparse_fwd_ms,
            "what": "window cell = whole grid (dense attention over all voxels) on the same "
                    "kernels; selected/window stage only"}


def window_variant_timing(r, label, window=None, reps=10, **plan_kw):
    """The forward (all stages) with a window partition of its own (cells that are not unions
    of blocks: a separate window pass over a token-level sort), HIP events around `reps`
    calls; credited 4 d FLOPs per attended pair, the window pairs counted per cell."""
    torch, ssa, wl = r.torch, r.ssa, r.wl
    N, H, d = r.N, r.H, r.d
    plan = ssa.Plan(r.coords, wl.grid, wl.block, window or wl.window, **plan_kw)
    out = torch.empty_like(r.dev["q"])
    sel = torch.empty((H, plan.num_blocks, wl.topk), dtype=torch.int32, device="cuda")
    ws = torch.empty(ssa.forward_workspace_size(plan, r.tdt, H, d, wl.topk), dtype=torch.uint8, device="cuda")
    run = lambda: r.fwd(plan, ssa.STAGE_ALL, out=out, sel=sel, ws=ws)
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(r.stream)
    for _ in range(reps):
        run()
    e1.record(r.stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    a = {k: v.cpu().numpy().astype(np.int64) for k, v in plan.arrays().items()}
    sizes = np.diff(a["blk_off"])
    M = len(sizes)
    sel_np = sel.cpu().numpy()
    sel_keys = np.where(sel_np >= 0, sizes[np.clip(sel_np, 0, M - 1)], 0).sum(axis=2)
    wsz = np.diff(a["wcell_off"]).astype(np.float64)
    pairs = H * (N * M + (wsz ** 2).sum()) + float((sizes[None, :] * sel_keys).sum())
    flops = 4.0 * d * pairs
    tf = flops / (ms * 1e-3) / 1e12
    return {"what": label, "forward_ms": ms, "reps": reps, "window_cells": int(plan.num_wcells),
            "largest_window": int(wsz.max()), "credited_flops": flops, "tflops": tf,
            "mfma_peak_frac": tf / r.peak}


def conv_timing(r, reps=10):
    """The forward with the sparse-convolution compressor (B^3 position weights per K and V):
    HIP events around `reps` calls of all stages; credited as the mean-pool forward (the
    attention pairs do not change) plus 4 N H d^2 FLOPs of position-weight products."""
    torch, ssa, wl = r.torch, r.ssa, r.wl
    N, H, d = r.N, r.H, r.d
    import workloads as W
    wkc, wvc = W.conv_weights(wl.block, d, wl.dtype, seed=7)
    wkc, wvc = torch.from_numpy(wkc).cuda().to(r.tdt), torch.from_numpy(wvc).cuda().to(r.tdt)
    dv = r.dev
    run = lambda: ssa.forward(r.plan, dv["q"], dv["k"], dv["v"], wkc, wvc, dv["gates"], wl.topk, 0.0, out=r.out,
                              sel_out=r.sel, ws=r.ws)
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(r.stream)
    for _ in range(reps):
        run()
    e1.record(r.stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = r.work()[0] + 4.0 * N * H * d * d
    tf = flops / (ms * 1e-3) / 1e12
    return {"what": f"forward with the sparse-convolution compressor ({wl.block}^3 position weights)",
            "forward_ms": ms, "reps": reps, "credited_flops": flops, "tflops": tf, "mfma_peak_frac": tf / r.peak}


def producer_timing(r, channels=2112, reps=5):
    """The step before SSA at the workload's shape (width 2,112 = 22 x 96 on the Hi3D page's
    Stage 3): q, k, v and gates from token features (ssa_qkv_gates: projections on MFMA, RMS
    norm and 3D rotary embedding of q and k, sigmoid gates).  Credited 2 N C (3 H d + 3 H)
    FLOPs."""
    torch, ssa, wl = r.torch, r.ssa, r.wl
    N, H, d = r.N, r.H, r.d
    import workloads as W
    pin = W.producer_inputs(N, channels, H, d, wl.dtype, seed=11)
    dev = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda().to(r.tdt) for k, v in pin.items()}
    out = (torch.empty_like(r.dev["q"]), torch.empty_like(r.dev["q"]), torch.empty_like(r.dev["q"]),
           torch.empty_like(r.dev["gates"]))
    run = lambda: ssa.qkv_gates(dev["x"], dev["w_qkv"], dev["w_gate"], dev["b_gate"], dev["gamma_q"],
                                dev["gamma_k"], r.coords, H, d, out=out)
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(r.stream)
    for _ in range(reps):
        run()
    e1.record(r.stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = 2.0 * N * channels * (3 * H * d + 3 * H)
    tf = flops / (ms * 1e-3) / 1e12
    return {"what": f"k_qkv_gates: x [{N},{channels}] -> q, k, v [{N},{H},{d}], gates [{N},{H},3]",
            "ms": ms, "reps": reps, "credited_flops": flops, "tflops": tf, "mfma_peak": r.peak,
            "mfma_peak_frac": tf / r.peak}


def backward_timing(r, reps=5):
    """Forward with saved state, then the backward (fixed selection, the workload's dO), timed
    apart from the step: HIP events around `reps` backward calls.  Credited 10 d FLOPs per
    attended (query, key, head) pair over the three branches."""
    torch, ssa, wl = r.torch, r.ssa, r.wl
    N, H, d = r.N, r.H, r.d
    dout = torch.from_numpy(np.ascontiguousarray(r.inp["do"])).cuda().to(r.tdt)
    fws = torch.empty(ssa.forward_workspace_size(r.plan, r.tdt, H, d, wl.topk, save_for_bwd=True),
                      dtype=torch.uint8, device="cuda")
    r.fwd(r.plan, ssa.STAGE_ALL, ws=fws, save=True)
    bws = torch.empty(ssa.backward_workspace_size(r.plan, r.tdt, H, d, wl.topk), dtype=torch.uint8,
                      device="cuda")
    dv = r.dev
    run = lambda: ssa.backward(r.plan, dv["q"], dv["k"], dv["v"], dv["wk"], dv["wv"], dv["gates"],
                               wl.topk, r.sel, dout, fws, ws=bws)
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(r.stream)
    for _ in range(reps):
        run()
    e1.record(r.stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    _, _, _, _, _, pairs = r.work()
    flops = 10.0 * d * pairs
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": describe(wl, N, H, d) + " + backward, dO ~ N(0,1)", "ms": ms, "reps": reps,
            "credited_flops": flops, "tflops": tf, "mfma_peak": r.peak, "mfma_peak_frac": tf / r.peak,
            "what": "dQ, dK, dV, dgates with the forward's selection held fixed (fp32 outputs)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-heads", type=int, default=22,
                    help="heads of the headline workload the CPU oracle runs (all 22: about 10 s)")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward timing")
    ap.add_argument("--no-full", action="store_true", help="skip the dense full-attention baselines")
    ap.add_argument("--no-others", action="store_true", help="skip the other workloads' forwards")
    ap.add_argument("--quick", action="store_true", help="headline only (= --no-cpu --no-bwd --no-full --no-others)")
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy 3 times (HBM counter calibration)")
    args = ap.parse_args()
    if args.quick:
        args.no_cpu = args.no_bwd = args.no_full = args.no_others = True
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

    def progress(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    r = Runner(args.workload, torch, ssa, W)
    wl, N, H, d = r.wl, r.N, r.H, r.d
    progress(f"{wl.name}: inputs resident, timing {args.steps} steps")
    ms_step, stage_ms, step_ev = r.timed_steps(args.steps, args.warmup)
    fwd_ms = stage_ms["pool"] + stage_ms["select"] + stage_ms["attend"]
    flops, cmp_flops, alg_bytes, sizes, sel_np, _ = r.work()
    M = r.plan.num_blocks
    peak = r.peak
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
        "config": {"workload": describe(wl, N, H, d),
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
        "roofline": attend_roofline(att_flops, alg_bytes, stage_ms["attend"], peak,
                                    attend_traffic() if wl.name == WORKLOAD else None),
        "compressed_branch": {"kernels": "k_compress + k_select (+ k_topk when M <= 1024)",
                              "ms": stage_ms["select"], "tflops": sel_tflops,
                              "mfma_peak_frac": sel_tflops / peak, "work_flops": cmp_flops},
    }
    if not args.no_full and wl.name in DENSE:
        progress("dense baseline")
        res["full_attention"] = {wl.name: full_attention_timing(r, fwd_ms)}
    if not args.no_full and wl.name == WORKLOAD:
        progress("window partitions")
        res["window_variants"] = {
            "shifted8": window_variant_timing(r, "8^3 cells shifted by (4,4,4) (alternate-layer shifted windows)",
                                              shift=(4, 4, 4)),
            "sfc512": window_variant_timing(r, "windows of 512 tokens along the Morton order", sfc_tokens=512),
            "cube4": window_variant_timing(r, "4^3 cells (smaller than the 8^3 blocks)", window=4),
        }
    if not args.no_full and wl.name == WORKLOAD and wl.dtype != "f32":
        progress("producer")
        res["producer"] = producer_timing(r)
        progress("convolution compressor")
        res["conv_compressor"] = conv_timing(r)
    inp0 = r.inp
    del r
    torch.cuda.empty_cache()
    if not args.no_others:
        res["other_workloads"] = {}
        for name in OTHERS:
            if name == wl.name:
                continue
            progress(f"{name}")
            ro = Runner(name, torch, ssa, W)
            steps = 20 if ro.N <= 20000 else 5
            res["other_workloads"][name] = ro.summary(steps, 2)
            if not args.no_full and name in DENSE:
                res.setdefault("full_attention", {})[name] = full_attention_timing(
                    ro, res["other_workloads"][name]["forward_ms"])
            del ro
            torch.cuda.empty_cache()
    if not args.no_bwd:
        progress("backward")
        rb = Runner(BWD_WORKLOAD, torch, ssa, W)
        res["backward"] = backward_timing(rb)
        del rb
        torch.cuda.empty_cache()
    if not args.no_cpu:
        progress("cpu baseline")
        res["cpu_baseline"] = cpu_baseline(inp0, min(args.cpu_heads, H))
    print(json.dumps(res))


if __name__ == "__main__":
    main()

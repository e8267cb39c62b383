"""GPU parity: the HIP library through its C ABI against the float64 oracle."""
import numpy as np
import pytest

import oracle
import workloads as W
from brute import tiny_case
from parity import check_forward_all, check_items, check_selection, compare, gpu_forward, to_dev

pytestmark = pytest.mark.gpu

FULL = ["sphere2k", "torus20k", "shells80k", "shells110k"]
_cache = {}


def _workload(name, distinct_w=False):
    key = (name, distinct_w)
    if key not in _cache:
        _cache.clear()   # one full workload at a time (host memory)
        _cache[key] = W.make_inputs(name, distinct_w=distinct_w)
    return _cache[key]


def _plan_arrays(plan):
    return {k: v.cpu().numpy().astype(np.int64) for k, v in plan.arrays().items()}


# ------------------------------------------------------------------ plan
def _check_plan(inp, plan):
    ref = oracle.partition(inp["coords"], inp["block"], inp["grid"])
    a = _plan_arrays(plan)
    assert plan.num_blocks == ref.M
    np.testing.assert_array_equal(a["perm"], ref.perm)
    np.testing.assert_array_equal(a["blk_off"], ref.blk_off)
    np.testing.assert_array_equal(a["blk_key"], ref.blk_key)
    np.testing.assert_array_equal(a["tok2blk"], ref.tok2blk)
    sizes = np.diff(ref.blk_off)
    assert plan.max_block_rows == sizes.max()
    np.testing.assert_array_equal(a["lpt"], np.lexsort((np.arange(ref.M), -sizes)))
    # window cells: blocks grouped by cell, ascending inside a cell
    wp = oracle.window_partition(inp["coords"], inp["window"], inp["grid"])
    cell_of_block = wp.tok2blk[ref.perm[ref.blk_off[:-1]]]
    assert plan.num_cells == wp.M
    np.testing.assert_array_equal(a["blk_cell"], cell_of_block)
    for cidx in range(wp.M):
        blocks = a["cell_blk"][a["cell_off"][cidx]:a["cell_off"][cidx + 1]]
        np.testing.assert_array_equal(blocks, np.nonzero(cell_of_block == cidx)[0])


@pytest.mark.parametrize("name", FULL)
def test_plan_full_workloads(name):
    import spatial_sparse_attention_amd as ssa
    wl, inp = _workload(name)
    dev = to_dev(inp)
    plan = ssa.Plan(dev["coords"], inp["grid"], inp["block"], inp["window"])
    _check_plan(inp, plan)


@pytest.mark.parametrize("N,G,B,w", [(500, 16, 1, 1), (3000, 40, 3, 6), (4000, 64, 5, 64),
                                     (700, 12, 2, 8), (1, 4, 2, 2), (900, 10, 16, 16),
                                     (2500, 30, 4, 100)])
def test_plan_random(N, G, B, w):
    import spatial_sparse_attention_amd as ssa
    rng = np.random.default_rng(N + G)
    coords = rng.integers(0, G, (N, 3)).astype(np.int32)   # duplicates allowed
    inp = {"coords": coords, "grid": G, "block": B, "window": w}
    import torch
    plan = ssa.Plan(torch.from_numpy(coords).cuda(), G, B, w)
    _check_plan(inp, plan)


def test_plan_rejects_out_of_grid():
    import torch
    import spatial_sparse_attention_amd as ssa
    coords = torch.tensor([[0, 0, 0], [3, 8, 1]], dtype=torch.int32, device="cuda")
    with pytest.raises(ssa.SSAError) as e:
        ssa.Plan(coords, 8, 2, 2)
    assert e.value.status == 4


# ------------------------------------------------------------------ forward, small and exhaustive
SMALL = [  # (N, G, H, d, B, w, k, dtype)
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
    (800, 10, 2, 64, 2, 100, 100, "bf16"),   # every block selected; one window cell
    (700, 9, 1, 32, 1, 1, 6, "f32"),         # single-token blocks
    (400, 8, 2, 96, 8, 8, 3, "f16"),         # one block holds every token
    (512, 8, 1, 64, 8, 8, 2, "f16"),         # one full 8^3 block (512 rows)
    (1, 4, 1, 32, 2, 2, 4, "f32"),           # one token
    (3000, 40, 2, 64, 2, 2, 4, "f16"),       # ~2,500 blocks: in-kernel radix top-k (M > 1024)
    (3000, 40, 1, 96, 2, 4, 6, "bf16"),      # the same path with three key planes
    (2600, 36, 2, 32, 2, 2, 3, "f32"),       # and in fp32
    (7000, 40, 1, 32, 1, 1, 8, "f16"),       # 7,000 single-token blocks: beyond 6,144 blocks
]


def _small_inputs(case, distinct=True, scale=None, seed_extra=0):
    N, G, H, d, B, w, k, dt = case
    rng = np.random.default_rng(N * 7 + d + seed_extra)
    if N == 512 and G == 8:
        flat = np.arange(512)
        coords = np.stack(np.unravel_index(rng.permutation(flat), (8, 8, 8)), -1).astype(np.int32)
        c = tiny_case(rng, N, G, H, d)
        c["coords"] = coords
    else:
        c = tiny_case(rng, N, G, H, d, distinct=distinct)
    inp = W.random_inputs(c["coords"], H, d, dt, seed=N + d + seed_extra, grid=G)
    inp.update(block=B, window=w, topk=k)
    if scale is not None:
        inp["scale"] = scale
    return inp


def _check_small(inp):
    """Every output of a small case, every selection row by the near-tie rule."""
    out, sel, plan = gpu_forward(inp)
    H, k, dt = inp["q"].shape[1], inp["topk"], inp["dtype"]
    ref = oracle.forward(inp, scale=inp.get("scale"))
    M = ref["part"].M
    assert plan.num_blocks == M
    near = {}
    for h in range(H):
        for b in range(M):
            if check_selection(ref["sigma"][h, b], k, sel[h, b]) == "near":
                near[(h, b)] = sel[h, b]
    if near:
        ref = oracle.forward(inp, sel_override=near, scale=inp.get("scale"))
    compare(out, ref["out"], dt, "all outputs")
    return M


@pytest.mark.parametrize("case", SMALL, ids=[f"{c[7]}_d{c[3]}_B{c[4]}_w{c[5]}_k{c[6]}_N{c[0]}" for c in SMALL])
def test_forward_small(case):
    M = _check_small(_small_inputs(case))
    if case[0] >= 2600:
        assert M > 1024          # the top-k inside the selection kernel
    if case[0] == 7000:
        assert M > 6144


def test_forward_refuses_beyond_max_blocks():
    """A plan with more occupied blocks than the selection's on-chip memory holds for the
    dtype and d is refused before any launch (f32 at d = 128 has the lowest bound)."""
    import torch
    import spatial_sparse_attention_amd as ssa
    lim = ssa.forward_max_blocks(torch.float32, 128)
    assert 6000 < lim < 20000
    assert ssa.forward_max_blocks(torch.float16, 96) > lim
    N = lim + 500
    rng = np.random.default_rng(5)
    flat = rng.choice(64 ** 3, N, replace=False)
    coords = torch.from_numpy(np.stack(np.unravel_index(flat, (64, 64, 64)), -1).astype(np.int32)).cuda()
    plan = ssa.Plan(coords, 64, 1, 1)
    assert plan.num_blocks == N
    x = torch.zeros((N, 1, 128), dtype=torch.float32, device="cuda")
    w = torch.zeros((128, 128), dtype=torch.float32, device="cuda")
    g = torch.zeros((N, 1, 3), dtype=torch.float32, device="cuda")
    with pytest.raises(ssa.SSAError) as e:
        ssa.forward(plan, x, x, x, w, w, g, 4)
    assert e.value.status == 2


@pytest.mark.parametrize("case,scale", [((1500, 20, 2, 64, 4, 4, 4, "f16"), 0.05),
                                        ((600, 12, 2, 32, 2, 4, 3, "f32"), 0.3),
                                        ((1200, 16, 2, 96, 4, 8, 3, "bf16"), 0.08)])
def test_forward_explicit_scale(case, scale):
    """A softmax scale other than 1/sqrt(d) in all three branches."""
    _check_small(_small_inputs(case, scale=scale))


@pytest.mark.parametrize("case", [(1500, 12, 2, 64, 4, 4, 4, "f16"), (600, 8, 2, 32, 2, 4, 3, "f32"),
                                  (3000, 24, 1, 96, 2, 2, 5, "bf16")])
def test_forward_duplicate_coordinates(case):
    """Several tokens on one voxel (the coordinates drawn with replacement)."""
    inp = _small_inputs(case, distinct=False)
    assert len(np.unique(inp["coords"], axis=0)) < len(inp["coords"])
    _check_small(inp)


def test_forward_shared_w():
    """One matrix passed as both W_k and W_v (the pointers may alias)."""
    inp = _small_inputs((1500, 20, 2, 64, 4, 4, 4, "f16"))
    inp["wv"] = inp["wk"].copy()
    _check_small(inp)


def test_forward_side_stream():
    """A forward on a stream other than torch's current one (the binding allocates its
    outputs and workspace for that stream)."""
    import torch
    inp = _small_inputs((1500, 20, 2, 64, 4, 4, 4, "f16"))
    ref_out, ref_sel, plan = gpu_forward(inp)
    s = torch.cuda.Stream()
    outs = []
    for _ in range(3):
        out, sel, _ = gpu_forward(inp, plan=plan, stream=s)
        outs.append((out, sel))
        torch.empty(1 << 22, device="cuda").fill_(7.0)   # churn the allocator meanwhile
    for out, sel in outs:
        np.testing.assert_array_equal(sel, ref_sel)
        np.testing.assert_array_equal(out, ref_out)


def test_forward_sphere2k_all_items():
    wl, inp = _workload("sphere2k")
    out, sel, plan = gpu_forward(inp)
    items = [(h, b) for h in range(wl.heads) for b in range(plan.num_blocks)]
    counts = check_items(inp, out, sel, items)
    assert counts["exact"] + counts["near"] == len(items)


def _check_full(inp, heads=None):
    out, sel, plan = gpu_forward(inp)
    M = plan.num_blocks
    kk = min(inp["topk"], M)
    assert (sel[:, :, :kk] >= 0).all() and (sel[:, :, kk:] == -1).all()
    counts, mx, rel = check_forward_all(inp, out, sel, heads=heads)
    H = inp["q"].shape[1] if heads is None else len(heads)
    assert counts["exact"] + counts["near"] == H * M
    print(f"rows exact {counts['exact']} near {counts['near']}; max-abs {mx:.3g} rel-L2 {rel:.3g}")
    return plan


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,distinct", [("torus20k", False), ("shells80k", True),
                                           ("shells110k", True)])
def test_forward_full_all(name, distinct):
    """The full workloads in the configuration the benchmark times: every output element and
    every (head, block) selection row against the oracle (run in a process pool).  The
    80k and 110k shapes use W_v != W_k."""
    wl, inp = _workload(name, distinct)
    plan = _check_full(inp)
    if name == "shells110k":
        assert plan.num_blocks > 1024   # in-kernel radix select at full size


@pytest.mark.timeout(900)
@pytest.mark.parametrize("dtype,dim", [("f32", 32), ("f16", 128), ("bf16", 96)])
def test_forward_resident_streams_all(dtype, dim):
    """The torus geometry (20,000 voxels) at 16 heads: 1,264 (head, 256-row chunk) units, so
    each resident compressed-branch workgroup streams several units back to back (output
    stores and next-unit query prefetch inside the stream); covers the fp32 path, the
    d = 128 path without query prefetch (three stage buffers) and bf16 at d = 96.  Every
    output and selection row is compared."""
    wl, base = _workload("torus20k")
    inp = W.random_inputs(base["coords"], 16, dim, dtype, seed=21, grid=wl.grid)
    inp.update(block=wl.block, window=wl.window, topk=wl.topk)
    _check_full(inp)


def test_forward_deterministic():
    wl, inp = _workload("torus20k")
    o1, s1, plan = gpu_forward(inp)
    o2, s2, _ = gpu_forward(inp, plan=plan)
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(o1, o2)


def test_forward_within_block_permutation():
    rng = np.random.default_rng(3)
    c = tiny_case(rng, 1500, 20, 2, 64)
    inp = W.random_inputs(c["coords"], 2, 64, "f16", seed=9, grid=20)
    inp.update(block=4, window=4, topk=4)
    o1, s1, _ = gpu_forward(inp)
    part = oracle.partition(inp["coords"], 4, 20)
    pi = np.arange(1500)
    for b in range(part.M):
        t = part.tokens(b)
        pi[t] = rng.permutation(t)
    inp2 = dict(inp)
    for key in ("coords", "q", "k", "v", "gates"):
        inp2[key] = inp[key][pi]
    o2, s2, _ = gpu_forward(inp2)
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_allclose(o2, o1[pi], atol=2e-3)


# ------------------------------------------------------------------ dense attention (one window cell)
@pytest.mark.timeout(900)
def test_dense_torus_geometry_all():
    """Dense attention over every voxel (one window cell covering the 256^3 grid) at the torus
    geometry's 20,000 voxels, 2 heads x 64 in bf16: every output element and selection row."""
    wl, base = _workload("torus20k")
    inp = W.random_inputs(base["coords"], 2, 64, "bf16", seed=31, grid=wl.grid)
    inp.update(block=wl.block, window=wl.grid, topk=wl.topk)
    plan = _check_full(inp)
    assert plan.num_cells == 1


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["shells80k", "shells110k"])
def test_dense_full_shape_sampled(name):
    """Dense attention over every voxel in the configuration the benchmark times as its dense
    baseline (the workload's own 22 x 96 fp16 inputs, one window cell covering the grid):
    sampled (head, block) items, largest and smallest blocks included, plus properties of
    every output."""
    wl, inp0 = _workload(name)
    inp = dict(inp0)
    inp["window"] = wl.grid
    out, sel, plan = gpu_forward(inp)
    assert plan.num_cells == 1
    a = _plan_arrays(plan)
    sizes = np.diff(a["blk_off"])
    rng = np.random.default_rng(11)
    blocks = [int(np.argmax(sizes)), int(np.argmin(sizes))] + [int(b) for b in rng.choice(plan.num_blocks, 2, replace=False)]
    items = sorted({(int(h), b) for b in blocks for h in (0, wl.heads - 1)})
    check_items(inp, out, sel, items)
    assert np.isfinite(out).all()



# ------------------------------------------------------------------ window partitions of their own
def _check_window_plan(inp, plan):
    wp = oracle.window_cells(inp)
    a = _plan_arrays(plan)
    assert not plan.cells_are_block_unions and plan.num_wcells == wp.M
    np.testing.assert_array_equal(a["wperm"], wp.perm)
    np.testing.assert_array_equal(a["wcell_off"], wp.blk_off)
    sizes = np.diff(wp.blk_off)
    np.testing.assert_array_equal(a["wlpt"], np.lexsort((np.arange(wp.M), -sizes)))


WINDOWS = [  # (N, G, H, d, B, k, dtype, window options)
    (1500, 20, 2, 64, 4, 4, "f16", dict(window=2)),                          # w < B
    (1500, 20, 2, 96, 4, 4, "f16", dict(window=6)),                          # w not a multiple of B
    (1200, 16, 2, 64, 4, 3, "bf16", dict(window=8, window_shift=(4, 4, 4))),  # shifted windows
    (1200, 16, 1, 32, 4, 3, "f32", dict(window=3, window_shift=(1, 0, 2))),
    (1500, 20, 2, 64, 4, 4, "f16", dict(window=4, sfc_tokens=64)),            # Morton-order windows
    (900, 12, 2, 96, 2, 5, "bf16", dict(window=4, sfc_tokens=37)),
    (700, 12, 1, 64, 2, 4, "f16", dict(window=4, sfc_tokens=5000)),           # one window: dense
    (3000, 40, 1, 64, 2, 4, "f16", dict(window=3, window_shift=(2, 1, 0))),   # > 1024 blocks
]


@pytest.mark.parametrize("case", WINDOWS, ids=[f"{c[6]}_d{c[3]}_B{c[4]}_{'_'.join(f'{k}{v}' for k, v in c[7].items())}"
                                               .replace(' ', '').replace(',', '-') for c in WINDOWS])
def test_forward_window_partitions(case):
    N, G, H, d, B, k, dt, win = case
    rng = np.random.default_rng(N + d + B)
    c = tiny_case(rng, N, G, H, d)
    inp = W.random_inputs(c["coords"], H, d, dt, seed=N + 3 * d, grid=G)
    inp.update(block=B, topk=k, **win)
    import torch
    import spatial_sparse_attention_amd as ssa
    from parity import make_plan
    plan = make_plan(inp, torch.from_numpy(inp["coords"]).cuda())
    _check_window_plan(inp, plan)
    _check_small(inp)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("win", [dict(window=8, window_shift=(4, 4, 4)), dict(sfc_tokens=512)],
                         ids=["shifted8", "sfc512"])
def test_forward_window_partitions_full(win):
    """The 80k-voxel workload (22 x 96 fp16) with shifted 8^3 windows and with 512-token windows
    along the Morton order: every output element and selection row."""
    wl, inp0 = _workload("shells80k", True)
    inp = dict(inp0)
    inp.update(win)
    plan = _check_full(inp)
    assert not plan.cells_are_block_unions


def test_general_windows_refuse_backward():
    import torch
    import spatial_sparse_attention_amd as ssa
    rng = np.random.default_rng(4)
    c = tiny_case(rng, 600, 12, 2, 64)
    inp = W.random_inputs(c["coords"], 2, 64, "f16", seed=4, grid=12)
    inp.update(block=4, window=2, topk=3)
    dev = to_dev(inp)
    plan = ssa.Plan(dev["coords"], 12, 4, 2)
    assert ssa.backward_workspace_size(plan, torch.float16, 2, 64, 3) == 0
    with pytest.raises(ssa.SSAError) as e:
        ssa.forward(plan, dev["q"], dev["k"], dev["v"], dev["wk"], dev["wv"], dev["gates"], 3,
                    save_for_bwd=True)
    assert e.value.status == 2


def test_forward_batch_varlen():
    """Three samples of different sizes in one ssa_forward_batch call: each equals its own
    ssa_forward call bit for bit and the oracle on that sample alone."""
    import torch
    import spatial_sparse_attention_amd as ssa
    H, d, dt, k = 2, 64, "f16", 4
    samples = []
    for i, (N, G) in enumerate(((1500, 20), (300, 10), (2600, 36))):
        rng = np.random.default_rng(40 + i)
        c = tiny_case(rng, N, G, H, d)
        inp = W.random_inputs(c["coords"], H, d, dt, seed=50 + i, grid=G)
        inp.update(block=2 if G == 36 else 4, window=4, topk=k)
        samples.append(inp)
    wk = samples[0]["wk"]
    wv = samples[0]["wv"]
    for s in samples:       # the projection is shared by the batch
        s["wk"], s["wv"] = wk, wv
    cat = {x: np.concatenate([s[x] for s in samples]) for x in ("q", "k", "v", "gates")}
    dev = {x: torch.from_numpy(cat[x]).cuda().half() for x in cat}
    wkd, wvd = torch.from_numpy(wk).cuda().half(), torch.from_numpy(wv).cuda().half()
    plans = [ssa.Plan(torch.from_numpy(s["coords"]).cuda(), s["grid"], s["block"], s["window"]) for s in samples]
    off = np.cumsum([0] + [len(s["coords"]) for s in samples])
    out = ssa.forward_batch(plans, off, dev["q"], dev["k"], dev["v"], wkd, wvd, dev["gates"], k)
    torch.cuda.synchronize()
    out = out.double().cpu().numpy()
    for i, s in enumerate(samples):
        o1, s1, _ = gpu_forward(s, plan=plans[i])
        np.testing.assert_array_equal(out[off[i]:off[i + 1]], o1)
        ref = oracle.forward(s)
        near = {}
        for h in range(H):
            for b in range(ref["part"].M):
                if check_selection(ref["sigma"][h, b], k, s1[h, b]) == "near":
                    near[(h, b)] = s1[h, b]
        if near:
            ref = oracle.forward(s, sel_override=near)
        compare(out[off[i]:off[i + 1]], ref["out"], dt, f"sample {i}")

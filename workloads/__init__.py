"""Seeded synthetic inputs for Spatial Sparse Attention (SSA).

This module only *draws inputs*: voxel geometries and random tensors.  It holds
none of SSA's arithmetic, so that both the float64 oracle's tests and the HIP
library's tests and benchmark can use it without sharing any method code.

Five workloads are defined (``WORKLOADS``).  Their shapes follow the sparse
volumes described on the pages: a sphere shell for a tiny fp32 case, a torus
surface in a 256^3 grid, and unions of ellipsoid shells sized like the voxel
budgets of the Sparc3D/Hi3D pipeline page ("How the pipeline works" pass table:
80,000 voxels at 64^3, 110,000 at 192^3; "Stage 3": 22 heads, width 2,112,
fp16).  Every value is drawn in float64 from ``numpy.random.SeedSequence(n)``
streams spawned in the fixed order [geometry, subsample, Q, K, V, W, gates, dO]
and rounded (via float32, round-to-nearest-even) to the workload dtype.  Arrays
are returned as float32 numpy arrays whose values are exactly representable in
the workload dtype.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_inputs", "make_geometry", "round_to_dtype",
           "random_inputs", "producer_inputs", "conv_weights"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    n: int            # number of voxels (tokens)
    grid: int         # grid edge G (cubic grid G^3)
    block: int        # block edge B
    window: int       # window-cell edge w
    topk: int         # selected blocks per (query block, head)
    heads: int
    dim: int
    dtype: str        # "f32" | "f16" | "bf16"
    shape: str        # geometry recipe
    backward: bool = False


WORKLOADS = {
    "sphere2k": Workload("sphere2k", 1, 2048, 32, 4, 4, 4, 2, 32, "f32", "sphere"),
    "torus20k": Workload("torus20k", 2, 20000, 256, 8, 8, 16, 16, 64, "bf16", "torus"),
    "shells80k": Workload("shells80k", 3, 80000, 64, 8, 8, 8, 22, 96, "f16", "ellipsoids6"),
    "shells110k": Workload("shells110k", 4, 110000, 192, 8, 8, 16, 22, 96, "f16", "ellipsoids10"),
    "shells80k_bwd": Workload("shells80k_bwd", 5, 80000, 64, 8, 8, 8, 22, 96, "f16", "ellipsoids6",
                              backward=True),
}


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to ``dtype`` (RNE via float32) and return them as float32."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return x32
    if dtype == "f16":
        return x32.astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        u = x32.view(np.uint32).astype(np.uint64)
        lsb = (u >> 16) & 1
        u = ((u + 0x7FFF + lsb) >> 16) << 16
        return u.astype(np.uint32).view(np.float32)
    raise ValueError(f"unknown dtype {dtype}")


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    names = ["geometry", "subsample", "q", "k", "v", "w", "gates", "do"]
    return {nm: np.random.default_rng(s) for nm, s in zip(names, ss.spawn(len(names)))}


def _grid_points(lo, hi):
    axes = [np.arange(lo[i], hi[i], dtype=np.int32) for i in range(3)]
    g = np.stack(np.meshgrid(*axes, indexing="ij"), -1).reshape(-1, 3)
    return g


def _sphere(G, rng_geo):
    g = _grid_points((0, 0, 0), (G, G, G))
    r = np.linalg.norm(g + 0.5 - G / 2.0, axis=1)
    return g[np.abs(r - 12.0) <= 1.0]


def _torus(G, rng_geo):
    # axis z through the grid centre, major radius 80, minor radius 30, thickness 2
    c = G / 2.0
    lo = (int(c - 112), int(c - 112), int(c - 32))
    hi = (int(c + 112), int(c + 112), int(c + 32))
    g = _grid_points(lo, hi)
    p = g.astype(np.float64) + 0.5 - c
    rho = np.hypot(p[:, 0], p[:, 1])
    t = np.hypot(rho - 80.0, p[:, 2])
    return g[np.abs(t - 30.0) <= 1.0]


def _ellipsoid_shell_distance(G, n_shells, amin, amax, rng_geo):
    """Approximate distance of every voxel centre to the nearest of n random ellipsoid surfaces."""
    shells = []
    for _ in range(n_shells):
        a = rng_geo.uniform(amin, amax, 3)
        c = rng_geo.uniform(0.6 * a.max(), G - 0.6 * a.max(), 3)
        R = np.linalg.qr(rng_geo.normal(size=(3, 3)))[0]
        shells.append((a, c, R))
    best = np.full(G ** 3, np.inf, dtype=np.float32)
    g_all = _grid_points((0, 0, 0), (G, G, G))
    chunk = 1 << 21
    for s0 in range(0, len(g_all), chunk):
        g = g_all[s0:s0 + chunk].astype(np.float32) + 0.5
        b = best[s0:s0 + chunk]
        for a, c, R in shells:
            q = (g - c.astype(np.float32)) @ R.astype(np.float32)
            rr = np.sqrt(((q / a.astype(np.float32)) ** 2).sum(1))
            np.minimum(b, np.abs(rr - 1.0) * np.float32(a.min()), out=b)
    return g_all, best


def make_geometry(wl: Workload) -> np.ndarray:
    """Distinct voxel coordinates, int32 [N,3], in a seeded random (caller) order."""
    st = _streams(wl.seed)
    G = wl.grid
    if wl.shape == "sphere":
        pool = _sphere(G, st["geometry"])
        idx = st["subsample"].choice(len(pool), wl.n, replace=False)
        return np.ascontiguousarray(pool[idx].astype(np.int32))
    if wl.shape == "torus":
        pool = _torus(G, st["geometry"])
        idx = st["subsample"].choice(len(pool), wl.n, replace=False)
        return np.ascontiguousarray(pool[idx].astype(np.int32))
    if wl.shape.startswith("ellipsoids"):
        n_sh = int(wl.shape[len("ellipsoids"):])
        amin, amax = (10.0, 30.0) if n_sh == 6 else (15.0, 80.0)
        g_all, dist = _ellipsoid_shell_distance(G, n_sh, amin, amax, st["geometry"])
        # a common shell thickness: keep the N voxels closest to any surface
        # (equal distances broken by a seeded random key), in a seeded random order
        tie = st["subsample"].random(len(dist))
        keep = np.lexsort((tie, dist))[: wl.n]
        keep = keep[st["subsample"].permutation(wl.n)]
        return np.ascontiguousarray(g_all[keep].astype(np.int32))
    raise ValueError(wl.shape)


def random_inputs(coords: np.ndarray, heads: int, dim: int, dtype: str, seed: int,
                  grid: int, backward: bool = False, distinct_w: bool = True) -> dict:
    """Q, K, V ~ N(0,1) [N,H,d]; W_k ~ N(0, 1/d) [d,d]; gates ~ U(0,1) [N,H,3] (order:
    compressed, selected, window); dO ~ N(0,1).  W_v is a second draw from the W stream
    (distinct_w) or the same matrix as W_k (one projection W, as the workload tables
    state it)."""
    st = _streams(seed)
    n = len(coords)
    out = {
        "coords": np.ascontiguousarray(coords.astype(np.int32)),
        "grid": grid,
        "dtype": dtype,
        "q": round_to_dtype(st["q"].standard_normal((n, heads, dim)), dtype),
        "k": round_to_dtype(st["k"].standard_normal((n, heads, dim)), dtype),
        "v": round_to_dtype(st["v"].standard_normal((n, heads, dim)), dtype),
    }
    w = round_to_dtype(st["w"].standard_normal((dim, dim)) / math.sqrt(dim), dtype)
    out["wk"] = w
    out["wv"] = (round_to_dtype(st["w"].standard_normal((dim, dim)) / math.sqrt(dim), dtype)
                 if distinct_w else w.copy())
    out["gates"] = round_to_dtype(st["gates"].random((n, heads, 3)), dtype)
    if backward:
        out["do"] = round_to_dtype(st["do"].standard_normal((n, heads, dim)), dtype)
    return out


def make_inputs(name_or_wl, distinct_w: bool = False) -> tuple[Workload, dict]:
    """A named workload's inputs.  By default one projection W serves as W_k and W_v (the
    workload tables name a single W); distinct_w draws W_v separately."""
    wl = WORKLOADS[name_or_wl] if isinstance(name_or_wl, str) else name_or_wl
    coords = make_geometry(wl)
    inp = random_inputs(coords, wl.heads, wl.dim, wl.dtype, wl.seed, wl.grid, wl.backward,
                        distinct_w=distinct_w)
    inp.update(block=wl.block, window=wl.window, topk=wl.topk)
    return wl, inp


def producer_inputs(n: int, channels: int, heads: int, dim: int, dtype: str, seed: int,
                    bias: bool = True) -> dict:
    """Token features and weights of the step that produces SSA's inputs: x ~ N(0,1) [N,C];
    W_qkv ~ N(0, 1/C) [3 H d, C] and W_gate ~ N(0, 1/C) [3 H, C] (linear-layer layout);
    b_gate ~ N(0, 1/4) [3 H] (or None); gamma_q, gamma_k ~ 1 + N(0, 0.1^2) [d]."""
    ss = np.random.SeedSequence([seed, 7])
    r = [np.random.default_rng(x) for x in ss.spawn(6)]
    sd = 1.0 / math.sqrt(channels)
    return {
        "x": round_to_dtype(r[0].standard_normal((n, channels)), dtype),
        "w_qkv": round_to_dtype(r[1].standard_normal((3 * heads * dim, channels)) * sd, dtype),
        "w_gate": round_to_dtype(r[2].standard_normal((3 * heads, channels)) * sd, dtype),
        "b_gate": round_to_dtype(r[3].standard_normal(3 * heads) * 0.5, dtype) if bias else None,
        "gamma_q": round_to_dtype(1.0 + 0.1 * r[4].standard_normal(dim), dtype),
        "gamma_k": round_to_dtype(1.0 + 0.1 * r[5].standard_normal(dim), dtype),
    }


def conv_weights(block: int, dim: int, dtype: str, seed: int) -> tuple:
    """Position weights of the sparse-convolution compressor: W_k, W_v ~ N(0, 1/d), each
    [B^3, d, d] (every position inside a block a linear-layer matrix [d_out, d_in])."""
    ss = np.random.SeedSequence([seed, 11])
    rk, rv = [np.random.default_rng(x) for x in ss.spawn(2)]
    shape = (block ** 3, dim, dim)
    return (round_to_dtype(rk.standard_normal(shape) / math.sqrt(dim), dtype),
            round_to_dtype(rv.standard_normal(shape) / math.sqrt(dim), dtype))

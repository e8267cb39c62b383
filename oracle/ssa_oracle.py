"""Spatial Sparse Attention (SSA), forward and backward, as a plain float64 CPU oracle.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's cpu_baseline leg, never by the HIP product path.

What SSA computes, as the pages state it (Direct3D-S2 pages: the pixal-3d.com
landing page, "What is Direct3D-S2?" and the FAQ entry "What is SSA?"; the
nav.superapi.store page, "Technical principles of Direct3D-S2", first bullet):
tokens carrying 3D coordinates are partitioned into blocks by coordinate; a
compression module reduces each block to one token by pooling and attends to
those block tokens (global context); the attention scores of the compression
module pick the important blocks, whose tokens are attended at full
resolution (selection); a local window module attends to nearby tokens; and the
three outputs are summed with per-branch weights (gates) that the model predicts.

The pages give no equations.  The readings taken where they are silent:
  * blocks are axis-aligned B^3 cubes anchored at the origin, ids ordered by the
    x-major linear block key; only occupied blocks exist;
  * compression = arithmetic mean of the block's token keys/values followed by a
    linear map (k~ = kbar @ W_k, row-vector convention, shared by all heads);
  * softmax scale tau = 1/sqrt(d) in every branch unless given; no masks, no
    position terms; a token attends to every compressed block, its own included;
  * block importance sigma_h(Bq, b) = sum over the query block's tokens of their
    compressed softmax probabilities for block b;
  * selection = the min(k, M) blocks with the largest sigma, ties to the lower
    block id, reported in ascending id order and padded with -1;
  * the selected branch is one softmax over the union of the selected blocks'
    tokens; the window branch is one softmax over all tokens in the query's
    window cell (non-overlapping w^3 cells anchored at the origin, optionally
    shifted, or fixed-size runs along the Morton order of the voxels);
  * gates are used as given, layout [N,H,3] in the order (compressed, selected,
    window).
Everything is float64; inputs are the dtype-rounded values, upcast exactly.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


# --------------------------------------------------------------------------- partition
@dataclasses.dataclass
class Partition:
    """Blocks of a coordinate set.

    perm[r]    token index at sorted position r (tokens ordered by block key, then index)
    blk_off    [M+1] first sorted position of each block, blk_off[M] = N
    blk_key    [M] linear block key kappa of each block (ascending)
    tok2blk    [N] block id of each token (caller order)
    """
    perm: np.ndarray
    blk_off: np.ndarray
    blk_key: np.ndarray
    tok2blk: np.ndarray
    edge: int
    dims: tuple

    @property
    def M(self) -> int:
        return len(self.blk_key)

    def tokens(self, b: int) -> np.ndarray:
        return self.perm[self.blk_off[b]:self.blk_off[b + 1]]


def partition(coords: np.ndarray, edge: int, grid) -> Partition:
    """Partition tokens into edge^3 blocks by their 3D coordinates.

    Follows the partition step of nav.superapi.store, Direct3D-S2, "Technical principles
    of Direct3D-S2" (tokens grouped into blocks by their 3D coordinates): beta =
    floor(c / edge) per axis, block key kappa = (beta_x * n_y + beta_y) * n_z + beta_z
    with n_a = ceil(G_a / edge); blocks are the distinct keys in ascending order;
    tokens within a block keep index order.
    """
    c = np.asarray(coords, dtype=np.int64)
    g = np.broadcast_to(np.asarray(grid, dtype=np.int64), (3,))
    if c.size and (c.min() < 0 or np.any(c >= g[None, :])):
        raise ValueError("coordinate outside the grid")
    dims = tuple(int(-(-int(x) // edge)) for x in g)
    beta = c // edge
    key = (beta[:, 0] * dims[1] + beta[:, 1]) * dims[2] + beta[:, 2]
    order = np.argsort(key, kind="stable")
    ks = key[order]
    if len(ks):
        uniq, starts, counts = np.unique(ks, return_index=True, return_counts=True)
    else:
        uniq = starts = counts = np.zeros(0, dtype=np.int64)
    blk_off = np.append(starts, len(ks)).astype(np.int64)
    tok2blk = np.empty(len(ks), dtype=np.int64)
    tok2blk[order] = np.repeat(np.arange(len(uniq)), counts)
    return Partition(order.astype(np.int64), blk_off, uniq.astype(np.int64), tok2blk, edge, dims)


# --------------------------------------------------------------------------- compression
def pool(k: np.ndarray, v: np.ndarray, wk: np.ndarray, wv: np.ndarray, part: Partition):
    """Compressed keys/values per block and head: mean over the block's tokens, then W.

    The pages' compression extracts block-level information by convolution and pooling
    (nav.superapi.store, "Technical principles of Direct3D-S2"); the reading here is
    a mean-pool followed by one linear map.  Returns (ktil, vtil), each [H, M, d].
    """
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    H, d = k.shape[1], k.shape[2]
    kbar = np.empty((part.M, H, d))
    vbar = np.empty((part.M, H, d))
    for b in range(part.M):
        t = part.tokens(b)
        kbar[b] = k[t].mean(axis=0)
        vbar[b] = v[t].mean(axis=0)
    ktil = np.einsum("bhi,ij->hbj", kbar, np.asarray(wk, dtype=np.float64))
    vtil = np.einsum("bhi,ij->hbj", vbar, np.asarray(wv, dtype=np.float64))
    return ktil, vtil


def block_offsets(coords, edge: int) -> np.ndarray:
    """Position of each voxel inside its block: (c mod B) per axis, as the x-major index
    (o_x * B + o_y) * B + o_z in [0, B^3)."""
    o = np.asarray(coords, dtype=np.int64) % edge
    return (o[:, 0] * edge + o[:, 1]) * edge + o[:, 2]


def pool_conv(k, v, wck, wcv, part: Partition, coords):
    """Compressed keys/values by a sparse 3D convolution then pooling (nav.superapi.store,
    "Technical principles of Direct3D-S2": block-level information through sparse 3D
    convolution and pooling).  Reading: a convolution with kernel size and stride B over the
    occupied voxels, so every block is one output site and every voxel's weight depends on its
    position inside the block, followed by the mean over the block's occupied voxels:
    ktil[h, b] = (1/n_b) sum_{i in b} k[i, h] @ Wc_k[o(i)]^T with Wc [B^3, d_out, d_in] (each
    position a linear-layer matrix).  Returns (ktil, vtil), each [H, M, d]."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    wck = np.asarray(wck, dtype=np.float64)
    wcv = np.asarray(wcv, dtype=np.float64)
    H, d = k.shape[1], k.shape[2]
    off = block_offsets(coords, part.edge)
    ktil = np.zeros((H, part.M, d))
    vtil = np.zeros((H, part.M, d))
    for b in range(part.M):
        t = part.tokens(b)
        for i in t:
            ktil[:, b] += k[i] @ wck[off[i]].T
            vtil[:, b] += v[i] @ wcv[off[i]].T
        ktil[:, b] /= len(t)
        vtil[:, b] /= len(t)
    return ktil, vtil


def compress(inp: dict, k, v, part: Partition):
    """The compression module an input dict asks for: the sparse-convolution compressor when
    it carries "wk_conv", "wv_conv" [B^3, d, d], else mean-pool + linear map (wk, wv)."""
    if inp.get("wk_conv") is not None:
        return pool_conv(k, v, inp["wk_conv"], inp["wv_conv"], part, inp["coords"])
    return pool(k, v, inp["wk"], inp["wv"], part)


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=1, keepdims=True)


def compressed_block(qb: np.ndarray, ktil_h: np.ndarray, vtil_h: np.ndarray, scale: float):
    """Compressed branch for the queries of one block and one head.

    Each query attends to every compressed block token (global context; pixal-3d.com
    "What is Direct3D-S2?").  The block importance vector is the column sum of the
    probabilities over the query block: the selection is driven by the compression
    branch's attention scores (nav.superapi.store, "Technical principles of
    Direct3D-S2").  Returns (o_c [n,d], sigma [M]).
    """
    s = scale * (np.asarray(qb, dtype=np.float64) @ ktil_h.T)
    p = _softmax_rows(s)
    return p @ vtil_h, p.sum(axis=0)


def select_topk(sigma: np.ndarray, k: int) -> np.ndarray:
    """The min(k, M) most important blocks (ties to the lower id), ascending, -1 padded."""
    M = len(sigma)
    order = np.lexsort((np.arange(M), -np.asarray(sigma, dtype=np.float64)))
    chosen = np.sort(order[:min(k, M)])
    out = np.full(k, -1, dtype=np.int64)
    out[:len(chosen)] = chosen
    return out


def _attend(qb, kj, vj, scale):
    s = scale * (qb @ kj.T)
    return _softmax_rows(s) @ vj


def selected_block(qb, k_h, v_h, part: Partition, sel_row: np.ndarray, scale: float):
    """Fine branch: one softmax over all tokens of the selected blocks, which are attended
    at full resolution (nav.superapi.store, "Technical principles of Direct3D-S2")."""
    blocks = [int(b) for b in sel_row if b >= 0]
    j = np.concatenate([part.tokens(b) for b in blocks]) if blocks else np.zeros(0, np.int64)
    return _attend(np.asarray(qb, np.float64), k_h[j], v_h[j], scale)


def window_partition(coords, w: int, grid, shift=(0, 0, 0)) -> Partition:
    """Window cells: non-overlapping w^3 cells, the cell of a voxel being floor((c + shift)/w)
    per axis (shift 0: anchored at the origin; shift w/2: the shifted windows of alternate
    layers).  The same construction as the block partition, on the shifted coordinates in
    the grid extended by the shift."""
    s = np.asarray(shift, dtype=np.int64).reshape(3)
    g = np.broadcast_to(np.asarray(grid, dtype=np.int64), (3,))
    return partition(np.asarray(coords, np.int64) + s[None, :], w, g + s)


def morton_codes(coords, bits: int) -> np.ndarray:
    """Morton (Z-order) code of each voxel: the bits of x, y and z interleaved from the most
    significant down, x first in each triple."""
    c = np.asarray(coords, dtype=np.int64)
    code = np.zeros(len(c), dtype=np.int64)
    for b in range(bits - 1, -1, -1):
        for axis in range(3):
            code = code * 2 + ((c[:, axis] >> b) & 1)
    return code


def sfc_windows(coords, tokens: int, grid) -> Partition:
    """Fixed-size windows along a space-filling curve (the Hi3D pipeline page, "Stage 4"):
    tokens ordered by the Morton code of their voxel (equal codes keep token order), cut into
    consecutive runs of `tokens` tokens, the last one shorter."""
    g = np.broadcast_to(np.asarray(grid, dtype=np.int64), (3,))
    bits = int(max(int(g.max()) - 1, 0)).bit_length()
    order = np.argsort(morton_codes(coords, bits), kind="stable")
    n = len(order)
    ncell = -(-n // tokens)
    blk_off = np.minimum(np.arange(ncell + 1, dtype=np.int64) * tokens, n)
    tok2blk = np.empty(n, dtype=np.int64)
    tok2blk[order] = np.arange(n) // tokens
    return Partition(order.astype(np.int64), blk_off, np.arange(ncell, dtype=np.int64), tok2blk,
                     tokens, (ncell,))


def window_cells(inp: dict) -> Partition:
    """The window partition an input dict asks for: "sfc_tokens" > 0 selects Morton-order
    windows, else cubic cells of edge "window" shifted by "window_shift" (default none)."""
    if inp.get("sfc_tokens"):
        return sfc_windows(inp["coords"], int(inp["sfc_tokens"]), inp["grid"])
    return window_partition(inp["coords"], inp["window"], inp["grid"], inp.get("window_shift", (0, 0, 0)))


def window_attention(q, k, v, wpart: Partition, scale: float) -> np.ndarray:
    """Local window branch: every token attends to all tokens of its own window cell, the
    local-feature module (nav.superapi.store, "Technical principles of Direct3D-S2")."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    N, H, d = q.shape
    out = np.empty((N, H, d))
    for c in range(wpart.M):
        t = wpart.tokens(c)
        for h in range(H):
            out[t, h] = _attend(q[t, h], k[t, h], v[t, h], scale)
    return out


def combine(gates, oc, os_, ow):
    """Gated aggregation of the three branch outputs: predicted gates weight the three
    modules' outputs (nav.superapi.store, "Technical principles of Direct3D-S2")."""
    g = np.asarray(gates, np.float64)
    return g[..., 0:1] * oc + g[..., 1:2] * os_ + g[..., 2:3] * ow


# --------------------------------------------------------------------------- driver
def _scale(scale, d):
    return 1.0 / math.sqrt(d) if (scale is None or scale == 0) else float(scale)


def forward_items(inp: dict, items, sel_override=None, scale=None, ktv=None):
    """Forward outputs for chosen (head, query block) items only.

    Returns a dict keyed by (h, Bq) with the block's sorted rows' outputs:
      'rows'  the token indices (caller order) of the block, in sorted order
      'out'   [n, d] combined output      'oc','os','ow' the branch outputs
      'sigma' [M] importance vector      'sel' [k] selected ids (or the override)
    plus 'part', 'ktil', 'vtil'.  sel_override maps (h, Bq) -> forced selection.
    """
    q = np.asarray(inp["q"], np.float64)
    k = np.asarray(inp["k"], np.float64)
    v = np.asarray(inp["v"], np.float64)
    N, H, d = q.shape
    sc = _scale(scale, d)
    part = partition(inp["coords"], inp["block"], inp["grid"])
    wpart = window_cells(inp)
    if ktv is None:
        ktil, vtil = compress(inp, k, v, part)
    else:
        ktil, vtil = ktv
    g = np.asarray(inp["gates"], np.float64)
    res = {"part": part, "ktil": ktil, "vtil": vtil}
    for (h, bq) in items:
        rows = part.tokens(bq)
        qb = q[rows, h]
        oc, sigma = compressed_block(qb, ktil[h], vtil[h], sc)
        if sel_override is not None and (h, bq) in sel_override:
            sel = np.asarray(sel_override[(h, bq)], np.int64)
        else:
            sel = select_topk(sigma, inp["topk"])
        os_ = selected_block(qb, k[:, h], v[:, h], part, sel, sc)
        ow = np.empty_like(oc)
        cells = wpart.tok2blk[rows]
        for c in np.unique(cells):
            m = cells == c
            t = wpart.tokens(int(c))
            ow[m] = _attend(qb[m], k[t, h], v[t, h], sc)
        out = combine(g[rows, h], oc, os_, ow)
        res[(h, bq)] = {"rows": rows, "out": out, "oc": oc, "os": os_, "ow": ow,
                        "sigma": sigma, "sel": sel}
    return res


def forward(inp: dict, sel_override=None, scale=None, keep_sigma=True):
    """Full SSA forward.  Returns dict with 'out' [N,H,d], 'sel' [H,M,k], branch outputs
    'oc','os','ow' [N,H,d], 'sigma' [H,M,M] (if keep_sigma) and the partition."""
    q = np.asarray(inp["q"])
    N, H, d = q.shape
    part = partition(inp["coords"], inp["block"], inp["grid"])
    items = [(h, b) for h in range(H) for b in range(part.M)]
    r = forward_items(inp, items, sel_override=sel_override, scale=scale)
    out = np.zeros((N, H, d))
    oc = np.zeros((N, H, d))
    os_ = np.zeros((N, H, d))
    ow = np.zeros((N, H, d))
    sel = np.full((H, part.M, inp["topk"]), -1, np.int64)
    sigma = np.zeros((H, part.M, part.M)) if keep_sigma else None
    for (h, b) in items:
        it = r[(h, b)]
        rows = it["rows"]
        out[rows, h] = it["out"]
        oc[rows, h] = it["oc"]
        os_[rows, h] = it["os"]
        ow[rows, h] = it["ow"]
        sel[h, b] = it["sel"]
        if keep_sigma:
            sigma[h, b] = it["sigma"]
    return {"out": out, "oc": oc, "os": os_, "ow": ow, "sel": sel, "sigma": sigma,
            "part": part, "ktil": r["ktil"], "vtil": r["vtil"]}


# --------------------------------------------------------------------------- backward
def _attend_bwd(qb, kj, vj, do_x, scale):
    """Backward of o = softmax(scale q k^T) v for one query set.  Returns dq, dk, dv."""
    s = scale * (qb @ kj.T)
    p = _softmax_rows(s)
    o = p @ vj
    dv = p.T @ do_x
    dp = do_x @ vj.T
    dd = (do_x * o).sum(axis=1, keepdims=True)
    ds = p * (dp - dd)
    dq = scale * (ds @ kj)
    dk = scale * (ds.T @ qb)
    return dq, dk, dv


def backward(inp: dict, sel: np.ndarray, dout: np.ndarray, scale=None):
    """Analytic float64 backward of the forward above with the selection held fixed.

    Gradients flow into Q, K, V (through all three branches; the compressed branch
    reaches K and V through the mean pool and W) and into the gates.  sigma and
    the top-k carry no gradient; W gets none.  Returns dq, dk, dv, dgates.
    """
    q = np.asarray(inp["q"], np.float64)
    k = np.asarray(inp["k"], np.float64)
    v = np.asarray(inp["v"], np.float64)
    wk = np.asarray(inp["wk"], np.float64)
    wv = np.asarray(inp["wv"], np.float64)
    g = np.asarray(inp["gates"], np.float64)
    do = np.asarray(dout, np.float64)
    N, H, d = q.shape
    sc = _scale(scale, d)
    part = partition(inp["coords"], inp["block"], inp["grid"])
    wpart = window_cells(inp)
    ktil, vtil = compress(inp, k, v, part)
    conv = inp.get("wk_conv") is not None
    if conv:
        off = block_offsets(inp["coords"], inp["block"])
        wck = np.asarray(inp["wk_conv"], np.float64)
        wcv = np.asarray(inp["wv_conv"], np.float64)
    dq = np.zeros((N, H, d))
    dk = np.zeros((N, H, d))
    dv = np.zeros((N, H, d))
    dg = np.zeros((N, H, 3))
    dktil = np.zeros_like(ktil)
    dvtil = np.zeros_like(vtil)
    for h in range(H):
        for b in range(part.M):
            rows = part.tokens(b)
            qb = q[rows, h]
            # compressed branch
            s = sc * (qb @ ktil[h].T)
            p = _softmax_rows(s)
            oc = p @ vtil[h]
            dg[rows, h, 0] = (do[rows, h] * oc).sum(1)
            dqc, dkc, dvc = _attend_bwd(qb, ktil[h], vtil[h], g[rows, h, 0:1] * do[rows, h], sc)
            dq[rows, h] += dqc
            dktil[h] += dkc
            dvtil[h] += dvc
            # selected branch
            blocks = [int(x) for x in sel[h, b] if x >= 0]
            j = np.concatenate([part.tokens(x) for x in blocks])
            os_ = _attend(qb, k[j, h], v[j, h], sc)
            dg[rows, h, 1] = (do[rows, h] * os_).sum(1)
            dqs, dks, dvs = _attend_bwd(qb, k[j, h], v[j, h], g[rows, h, 1:2] * do[rows, h], sc)
            dq[rows, h] += dqs
            np.add.at(dk[:, h], j, dks)
            np.add.at(dv[:, h], j, dvs)
        # window branch
        for c in range(wpart.M):
            t = wpart.tokens(c)
            ow = _attend(q[t, h], k[t, h], v[t, h], sc)
            dg[t, h, 2] = (do[t, h] * ow).sum(1)
            dqw, dkw, dvw = _attend_bwd(q[t, h], k[t, h], v[t, h], g[t, h, 2:3] * do[t, h], sc)
            dq[t, h] += dqw
            dk[t, h] += dkw
            dv[t, h] += dvw
    # through the projection and the mean pool
    for b in range(part.M):
        t = part.tokens(b)
        n = len(t)
        if conv:  # each voxel's own position weight
            for i in t:
                dk[i] += dktil[:, b] @ wck[off[i]] / n
                dv[i] += dvtil[:, b] @ wcv[off[i]] / n
        else:
            dk[t] += (dktil[:, b] @ wk.T)[None] / n
            dv[t] += (dvtil[:, b] @ wv.T)[None] / n
    return dq, dk, dv, dg


# --------------------------------------------------------------------------- inputs of SSA
# The step before the path: the transformer block produces each token's queries, keys,
# values and gates from its features (the Sparc3D/Hi3D pipeline page, "Stage 3": RMS
# normalisation of the self-attention queries and keys, rotary position embeddings; the
# nav.superapi.store page, "Technical principles of Direct3D-S2": the model predicts the per-branch gates).
def rms_norm(x, gamma, eps):
    """x / sqrt(mean(x^2) + eps) * gamma over the last axis."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps) * np.asarray(gamma, np.float64)


def rope_3d(x, coords, base):
    """Rotary position embedding from a voxel's three coordinates: the head dimension d is cut
    into three parts of 2P = 2 floor(d / 6) dimensions (x, y, z axes; the last d - 6P stay as
    they are); pair i of axis a, dimensions (2Pa + 2i, 2Pa + 2i + 1), is rotated by the angle
    c_a * base^(-i / P).  x: [N, H, d]; coords: [N, 3]."""
    x = np.asarray(x, np.float64)
    c = np.asarray(coords, np.float64)
    d = x.shape[-1]
    P = d // 6
    out = x.copy()
    for a in range(3):
        for i in range(P):
            ang = c[:, a] * base ** (-i / P)                      # [N]
            cs, sn = np.cos(ang)[:, None], np.sin(ang)[:, None]
            j = 2 * P * a + 2 * i
            u, v = x[:, :, j], x[:, :, j + 1]
            out[:, :, j] = u * cs - v * sn
            out[:, :, j + 1] = u * sn + v * cs
    return out


def qkv_gates(x, w_qkv, w_gate, b_gate, gamma_q, gamma_k, coords, heads, dim, base=10000.0, eps=1e-6):
    """Queries, keys, values and gates of every token from its features x [N, C]:
    y = x W_qkv^T (W_qkv [3 H d, C], output features in the order q | k | v, each head-major);
    q = rope(rmsnorm(y_q, gamma_q)), k = rope(rmsnorm(y_k, gamma_k)), v = y_v; gates =
    sigmoid(x W_gate^T + b_gate) with W_gate [3 H, C], feature h * 3 + branch.  Returns
    float64 q, k, v [N, H, d] and gates [N, H, 3]."""
    x = np.asarray(x, np.float64)
    N = x.shape[0]
    H, d = heads, dim
    y = x @ np.asarray(w_qkv, np.float64).T
    yq = y[:, :H * d].reshape(N, H, d)
    yk = y[:, H * d:2 * H * d].reshape(N, H, d)
    yv = y[:, 2 * H * d:].reshape(N, H, d)
    q = rope_3d(rms_norm(yq, gamma_q, eps), coords, base)
    k = rope_3d(rms_norm(yk, gamma_k, eps), coords, base)
    z = x @ np.asarray(w_gate, np.float64).T
    if b_gate is not None:
        z = z + np.asarray(b_gate, np.float64)
    gates = (1.0 / (1.0 + np.exp(-z))).reshape(N, H, 3)
    return q, k, yv, gates


# --------------------------------------------------------------------------- textbook
def sdpa_dense(q, k, v, scale):
    """Textbook dense softmax attention per head via torch's float64 CPU SDPA (a library
    routine used only by pins that reduce a branch to full attention)."""
    import torch
    qt = torch.from_numpy(np.ascontiguousarray(np.asarray(q, np.float64).transpose(1, 0, 2)))
    kt = torch.from_numpy(np.ascontiguousarray(np.asarray(k, np.float64).transpose(1, 0, 2)))
    vt = torch.from_numpy(np.ascontiguousarray(np.asarray(v, np.float64).transpose(1, 0, 2)))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return o.numpy().transpose(1, 0, 2)

"""Brute-force dense masked SSA on tiny inputs: an implementation written apart from the
oracle, used only to pin it.

Nothing here sorts tokens or computes block keys.  Blocks are the distinct tuples
floor(c / B) in lexicographic (x-major) order; membership, the selected-key mask and
the window mask are dense N x N / M x N boolean matrices built from coordinate
comparisons; each branch is a masked softmax over all N keys (or over the M
pooled keys) evaluated with scipy's logsumexp.
"""
import numpy as np
from scipy.special import logsumexp


def _masked_softmax(s, mask):
    s = np.where(mask, s, -np.inf)
    return np.exp(s - logsumexp(s, axis=1, keepdims=True))


def _spread3(x):
    """Bits of x (< 1024) moved to every third position (bit i -> bit 3i)."""
    x = np.asarray(x, np.int64) & 0x3FF
    x = (x | (x << 16)) & 0x030000FF
    x = (x | (x << 8)) & 0x0300F00F
    x = (x | (x << 4)) & 0x030C30C3
    x = (x | (x << 2)) & 0x09249249
    return x


def spread_morton(coords):
    """Morton codes by bit spreading (x in the top bit of each triple)."""
    c = np.asarray(coords, np.int64)
    return (_spread3(c[:, 0]) << 2) | (_spread3(c[:, 1]) << 1) | _spread3(c[:, 2])


def brute_window_mask(c, w, shift=(0, 0, 0), sfc_tokens=0):
    """N x N mask: j is in i's window.  Cubic cells by comparing floor((c + shift) / w);
    Morton-order windows by comparing rank // tokens (rank from bit-spread codes)."""
    if sfc_tokens:
        code = spread_morton(c)
        rank = np.empty(len(c), np.int64)
        rank[np.lexsort((np.arange(len(c)), code))] = np.arange(len(c))
        wid = rank // sfc_tokens
        return wid[:, None] == wid[None, :]
    s = np.asarray(shift, np.int64)
    cs = np.asarray(c, np.int64) + s
    return np.all((cs[:, None, :] // w) == (cs[None, :, :] // w), axis=2)


def brute_forward(coords, q, k, v, wk, wv, gates, B, w, topk, scale=None, sel_force=None,
                  shift=(0, 0, 0), sfc_tokens=0):
    c = np.asarray(coords, np.int64)
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    wk = np.asarray(wk, np.float64)
    wv = np.asarray(wv, np.float64)
    g = np.asarray(gates, np.float64)
    N, H, d = q.shape
    tau = 1.0 / np.sqrt(d) if not scale else scale
    tuples = [tuple(int(x) for x in (ci // B)) for ci in c]
    blocks = sorted(set(tuples))
    M = len(blocks)
    bid = np.array([blocks.index(t) for t in tuples])
    member = np.zeros((M, N), bool)
    member[bid, np.arange(N)] = True
    pool_mat = member / member.sum(axis=1, keepdims=True)
    win = brute_window_mask(c, w, shift, sfc_tokens)
    out = np.zeros((N, H, d))
    oc = np.zeros((N, H, d))
    os_ = np.zeros((N, H, d))
    ow = np.zeros((N, H, d))
    sel_all = np.full((H, M, topk), -1, np.int64)
    sigma_all = np.zeros((H, M, M))
    for h in range(H):
        kt = (pool_mat @ k[:, h]) @ wk
        vt = (pool_mat @ v[:, h]) @ wv
        pc = _masked_softmax(tau * q[:, h] @ kt.T, np.ones((N, M), bool))
        oc[:, h] = pc @ vt
        sigma = member.astype(np.float64) @ pc          # [M query blocks, M key blocks]
        sigma_all[h] = sigma
        selmask = np.zeros((N, N), bool)
        for bq in range(M):
            if sel_force is not None:
                chosen = [int(x) for x in sel_force[h, bq] if x >= 0]
            else:
                chosen = sorted(range(M), key=lambda b: (-sigma[bq, b], b))[:topk]
            sel_all[h, bq, :len(chosen)] = sorted(chosen)
            keymask = np.isin(bid, chosen)
            selmask[bid == bq] = keymask[None, :]
        s_full = tau * q[:, h] @ k[:, h].T
        os_[:, h] = _masked_softmax(s_full, selmask) @ v[:, h]
        ow[:, h] = _masked_softmax(s_full, win) @ v[:, h]
    out = g[..., 0:1] * oc + g[..., 1:2] * os_ + g[..., 2:3] * ow
    return {"out": out, "oc": oc, "os": os_, "ow": ow, "sel": sel_all, "sigma": sigma_all,
            "M": M, "bid": bid}


def tiny_case(rng, N, G, H, d, distinct=True):
    """Random tiny inputs (float64 values, no dtype rounding)."""
    if distinct:
        flat = rng.choice(G ** 3, N, replace=False)
        coords = np.stack(np.unravel_index(flat, (G, G, G)), -1).astype(np.int32)
    else:
        coords = rng.integers(0, G, (N, 3)).astype(np.int32)
    return {
        "coords": coords, "grid": G,
        "q": rng.standard_normal((N, H, d)), "k": rng.standard_normal((N, H, d)),
        "v": rng.standard_normal((N, H, d)),
        "wk": rng.standard_normal((d, d)) / np.sqrt(d), "wv": rng.standard_normal((d, d)) / np.sqrt(d),
        "gates": rng.random((N, H, 3)),
    }

"""Pins of the oracle's sparse-convolution compressor (nav.superapi.store, "Technical
principles of Direct3D-S2": block-level information by sparse 3D convolution and pooling;
read as a convolution with kernel size and stride B over the occupied voxels, then the mean
over the block's occupied voxels)."""
import numpy as np
import pytest

import oracle
from brute import tiny_case


def _case(seed, N=60, G=6, H=2, d=4, B=2):
    rng = np.random.default_rng(seed)
    c = tiny_case(rng, N, G, H, d)
    c.update(block=B, window=B, topk=2)
    c["wk_conv"] = rng.standard_normal((B ** 3, d, d)) / np.sqrt(d)
    c["wv_conv"] = rng.standard_normal((B ** 3, d, d)) / np.sqrt(d)
    return c, rng


def test_uniform_position_weights_give_mean_pool_and_linear():
    c, rng = _case(1)
    B, d = 2, 4
    c["wk_conv"] = np.broadcast_to(c["wk"].T, (B ** 3, d, d)).copy()
    c["wv_conv"] = np.broadcast_to(c["wv"].T, (B ** 3, d, d)).copy()
    part = oracle.partition(c["coords"], B, c["grid"])
    a = oracle.pool_conv(c["k"], c["v"], c["wk_conv"], c["wv_conv"], part, c["coords"])
    b = oracle.pool(c["k"], c["v"], c["wk"], c["wv"], part)
    np.testing.assert_allclose(a[0], b[0], atol=1e-13)
    np.testing.assert_allclose(a[1], b[1], atol=1e-13)


def test_unit_blocks_apply_one_weight():
    c, rng = _case(2, B=1)
    part = oracle.partition(c["coords"], 1, c["grid"])
    kt, vt = oracle.pool_conv(c["k"], c["v"], c["wk_conv"], c["wv_conv"], part, c["coords"])
    np.testing.assert_allclose(kt.transpose(1, 0, 2), c["k"][part.perm] @ c["wk_conv"][0].T, atol=1e-13)


def test_against_grouping_by_position():
    """The same sums taken position by position: for each block and each of the B^3 positions,
    the tokens at that position (found by comparing coordinates with the block corner) summed
    first, then multiplied by that position's weight."""
    c, rng = _case(3, N=120, G=8, B=2)
    B = 2
    coords = np.asarray(c["coords"], np.int64)
    part = oracle.partition(coords, B, c["grid"])
    kt, _ = oracle.pool_conv(c["k"], c["v"], c["wk_conv"], c["wv_conv"], part, coords)
    for b in range(part.M):
        t = part.tokens(b)
        corner = coords[t[0]] // B * B
        acc = np.zeros((2, 4))
        for ox in range(B):
            for oy in range(B):
                for oz in range(B):
                    at = [i for i in t if tuple(coords[i] - corner) == (ox, oy, oz)]
                    if at:
                        acc += c["k"][at].sum(axis=0) @ c["wk_conv"][(ox * B + oy) * B + oz].T
        np.testing.assert_allclose(kt[:, b], acc / len(t), atol=1e-13)


def test_translation_by_whole_blocks():
    c, rng = _case(4)
    part = oracle.partition(c["coords"], 2, c["grid"])
    a = oracle.pool_conv(c["k"], c["v"], c["wk_conv"], c["wv_conv"], part, c["coords"])
    sh = np.asarray(c["coords"]) + 4
    part2 = oracle.partition(sh, 2, c["grid"] + 4)
    b = oracle.pool_conv(c["k"], c["v"], c["wk_conv"], c["wv_conv"], part2, sh)
    np.testing.assert_allclose(a[0], b[0], atol=1e-13)


@pytest.mark.parametrize("seed", [5, 6])
def test_backward_finite_differences_conv(seed):
    c, rng = _case(seed, N=24, G=5, H=2, d=3)
    c["wk_conv"] = rng.standard_normal((8, 3, 3))
    c["wv_conv"] = rng.standard_normal((8, 3, 3))
    do = rng.standard_normal((24, 2, 3))
    base = oracle.forward(c)
    ov = {(h, b): base["sel"][h, b] for h in range(2) for b in range(base["part"].M)}
    dq, dk, dv, dg = oracle.backward(c, base["sel"], do)
    loss = lambda: float((oracle.forward(c, sel_override=ov, keep_sigma=False)["out"] * do).sum())
    eps = 1e-6
    for name, grad in (("k", dk), ("v", dv), ("q", dq)):
        arr = c[name]
        for _ in range(10):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            old = arr[idx]
            arr[idx] = old + eps
            lp = loss()
            arr[idx] = old - eps
            lm = loss()
            arr[idx] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[idx]) < 1e-7 + 1e-6 * abs(fd), (name, idx, fd, grad[idx])

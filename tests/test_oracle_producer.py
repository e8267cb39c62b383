"""Pins of the oracle's producer of SSA's inputs: RMS norm of queries and keys, the 3D rotary
embedding, the projections and the sigmoid gates (the Hi3D pipeline page, "Stage 3";
nav.superapi.store, "Technical principles of Direct3D-S2": the model predicts the per-branch gates)."""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "rope_rmsnorm.json")))


def test_rms_norm_golden_and_properties():
    np.testing.assert_allclose(oracle.rms_norm(np.array(GOLD["rms"]["x"]), 1.0, 0.0), GOLD["rms"]["out"],
                               rtol=1e-14)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 3, 96))
    y = oracle.rms_norm(x, 1.0, 0.0)
    np.testing.assert_allclose((y * y).mean(-1), 1.0, rtol=1e-12)             # unit RMS
    np.testing.assert_allclose(oracle.rms_norm(7.5 * x, 1.0, 0.0), y, rtol=1e-12)   # scale invariant
    g = rng.random(96)
    np.testing.assert_allclose(oracle.rms_norm(x, g, 0.0), y * g, rtol=1e-12)


def test_rope_golden():
    for case in GOLD["rope"]:
        x = np.array(case["x"], np.float64)[None, None, :]
        out = oracle.rope_3d(x, np.array([case["coord"]]), 10000.0)[0, 0]
        np.testing.assert_allclose(out, case["out"], atol=1e-14)


@pytest.mark.parametrize("d", [32, 64, 96, 128])
def test_rope_properties(d):
    rng = np.random.default_rng(d)
    q = rng.standard_normal((40, 2, d))
    k = rng.standard_normal((40, 2, d))
    c1 = rng.integers(0, 200, (40, 3))
    c2 = rng.integers(0, 200, (40, 3))
    t = rng.integers(-50, 50, (1, 3))
    np.testing.assert_allclose(oracle.rope_3d(q, np.zeros((40, 3)), 1e4), q, atol=1e-14)   # origin: identity
    rq = oracle.rope_3d(q, c1, 1e4)
    np.testing.assert_allclose(np.linalg.norm(rq, axis=-1), np.linalg.norm(q, axis=-1), rtol=1e-12)
    # scores depend only on the coordinate difference (translation of both voxels)
    s1 = (oracle.rope_3d(q, c1, 1e4) * oracle.rope_3d(k, c2, 1e4)).sum(-1)
    s2 = (oracle.rope_3d(q, c1 + t, 1e4) * oracle.rope_3d(k, c2 + t, 1e4)).sum(-1)
    np.testing.assert_allclose(s1, s2, atol=1e-9)
    # rotations compose
    np.testing.assert_allclose(oracle.rope_3d(oracle.rope_3d(q, c1, 1e4), c2, 1e4),
                               oracle.rope_3d(q, c1 + c2, 1e4), atol=1e-9)
    P = d // 6          # dimensions past 6P are not rotated
    np.testing.assert_array_equal(rq[..., 6 * P:], q[..., 6 * P:])


def test_qkv_gates_layout():
    """One-hot features pick single weight columns, so every output can be read off the
    weights: v is the weight column itself, the gates are sigmoid of weight + bias, and q, k
    are the normalised, rotated weight columns."""
    rng = np.random.default_rng(5)
    N, C, H, d = 4, 6, 2, 12
    x = np.eye(N, C)
    wqkv = rng.standard_normal((3 * H * d, C))
    wg = rng.standard_normal((3 * H, C))
    bg = rng.standard_normal(3 * H)
    gq, gk = rng.random(d), rng.random(d)
    coords = rng.integers(0, 9, (N, 3))
    q, k, v, g = oracle.qkv_gates(x, wqkv, wg, bg, gq, gk, coords, H, d, base=100.0, eps=1e-6)
    for n in range(N):
        for h in range(H):
            np.testing.assert_allclose(v[n, h], wqkv[2 * H * d + h * d: 2 * H * d + (h + 1) * d, n])
            for b in range(3):
                assert abs(g[n, h, b] - 1 / (1 + np.exp(-(wg[h * 3 + b, n] + bg[h * 3 + b])))) < 1e-15
            col = wqkv[h * d:(h + 1) * d, n]
            ref = col / np.sqrt((col ** 2).mean() + 1e-6) * gq
            ref = oracle.rope_3d(ref[None, None], coords[n:n + 1], 100.0)[0, 0]
            np.testing.assert_allclose(q[n, h], ref, rtol=1e-12)
            colk = wqkv[H * d + h * d:H * d + (h + 1) * d, n]
            refk = oracle.rope_3d((colk / np.sqrt((colk ** 2).mean() + 1e-6) * gk)[None, None],
                                  coords[n:n + 1], 100.0)[0, 0]
            np.testing.assert_allclose(k[n, h], refk, rtol=1e-12)

"""Pins of the oracle's analytic backward: float64 central finite differences of
L = sum(dO * O) with the selection held fixed, plus two exact sum rules."""
import numpy as np
import pytest

import oracle
from brute import tiny_case


def _setup(seed, N=24, G=5, H=2, d=3, B=2, w=2, k=2):
    rng = np.random.default_rng(seed)
    c = tiny_case(rng, N, G, H, d)
    c.update(block=B, window=w, topk=k)
    do = rng.standard_normal((N, H, d))
    base = oracle.forward(c)
    ov = {(h, b): base["sel"][h, b] for h in range(H) for b in range(base["part"].M)}
    return c, do, base, ov


def _loss(c, do, ov):
    return float((oracle.forward(c, sel_override=ov, keep_sigma=False)["out"] * do).sum())


@pytest.mark.parametrize("seed,B,w", [(0, 2, 2), (1, 2, 4), (2, 3, 1)])
def test_backward_finite_differences(seed, B, w):
    c, do, base, ov = _setup(seed, B=B, w=w)
    dq, dk, dv, dg = oracle.backward(c, base["sel"], do)
    rng = np.random.default_rng(100 + seed)
    eps = 1e-6
    for name, grad in (("q", dq), ("k", dk), ("v", dv), ("gates", dg)):
        arr = c[name]
        for _ in range(12):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            old = arr[idx]
            arr[idx] = old + eps
            lp = _loss(c, do, ov)
            arr[idx] = old - eps
            lm = _loss(c, do, ov)
            arr[idx] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[idx]) < 1e-7 + 1e-6 * abs(fd), (name, idx, fd, grad[idx])


def test_gate_gradients_closed_form():
    c, do, base, ov = _setup(3)
    _, _, _, dg = oracle.backward(c, base["sel"], do)
    for x, key in enumerate(("oc", "os", "ow")):
        np.testing.assert_allclose(dg[..., x], (do * base[key]).sum(axis=2), rtol=1e-12, atol=1e-13)


def test_backward_sum_rules():
    c, do, base, ov = _setup(4, N=40, G=6)
    dq, dk, dv, dg = oracle.backward(c, base["sel"], do)
    g = c["gates"]
    # every row of dS sums to zero and the mean pool keeps sums: sum_i dK_i = 0 per head
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    # every row of P sums to one: sum_j dV_j = sum_i (g1+g2) dO_i + (sum_i g0 dO_i) W_v^T
    exp = ((g[..., 1:2] + g[..., 2:3]) * do).sum(axis=0) + (g[..., 0:1] * do).sum(axis=0) @ c["wv"].T
    np.testing.assert_allclose(dv.sum(axis=0), exp, rtol=1e-12, atol=1e-12)

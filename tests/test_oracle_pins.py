"""Pins of the float64 oracle against things other than itself: a brute-force dense
masked implementation (brute.py), hand-derived closed forms (golden/), textbook
attention (torch SDPA, float64) in the cases where a branch reduces to it, and
invariants the method must satisfy."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from brute import brute_forward, tiny_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _inp(case, B, w, k):
    d = dict(case)
    d.update(block=B, window=w, topk=k)
    return d


# ---------------------------------------------------------------- golden closed forms
def _ev(x):
    if isinstance(x, str):
        return float(eval(x, {"__builtins__": {}}, {"sqrt": math.sqrt, "log": math.log}))
    return float(x)


@pytest.mark.parametrize("idx", [0, 1])
def test_golden_closed_forms(idx):
    fx = json.load(open(os.path.join(GOLDEN, "hand_closed_forms.json")))["cases"][idx]
    n = len(fx["coords"])
    arr = lambda key: np.array([_ev(x) for x in fx[key]]).reshape(n, 1, 1)
    inp = {"coords": np.array(fx["coords"], np.int32), "grid": fx["grid"],
           "q": arr("q"), "k": arr("k"), "v": arr("v"),
           "wk": np.array([[fx["w"]]]), "wv": np.array([[fx["w"]]]),
           "gates": np.array(fx["gates"], np.float64).reshape(n, 1, 3),
           "block": fx["block"], "window": fx["window"], "topk": fx["topk"]}
    r = oracle.forward(inp, scale=fx["scale"])
    for key in ("oc", "os", "ow", "out"):
        np.testing.assert_allclose(r[key][:, 0, 0], arr(key).ravel(), rtol=0, atol=1e-12, err_msg=key)
    np.testing.assert_allclose(r["sigma"][0], np.array(fx["sigma"]), atol=1e-12)
    np.testing.assert_array_equal(r["sel"][0], np.array(fx["sel"]))


# ---------------------------------------------------------------- brute force
CASES = [  # (N, G, H, d, B, w, k, distinct)
    (40, 6, 2, 4, 2, 2, 2, True),
    (60, 8, 1, 8, 3, 2, 3, True),
    (50, 8, 2, 3, 4, 4, 1, True),
    (30, 5, 2, 4, 1, 1, 4, True),
    (70, 8, 1, 5, 2, 4, 5, True),
    (45, 6, 2, 4, 2, 3, 100, True),
    (50, 4, 2, 4, 2, 2, 2, False),   # duplicate coordinates allowed
    (1, 4, 1, 4, 2, 2, 3, True),     # a single token
]


@pytest.mark.parametrize("case", CASES)
def test_oracle_vs_brute(case):
    N, G, H, d, B, w, k, distinct = case
    rng = np.random.default_rng(hash(case) % (2 ** 32))
    c = tiny_case(rng, N, G, H, d, distinct)
    inp = _inp(c, B, w, k)
    r = oracle.forward(inp)
    b = brute_forward(c["coords"], c["q"], c["k"], c["v"], c["wk"], c["wv"], c["gates"], B, w, k)
    assert r["part"].M == b["M"]
    np.testing.assert_array_equal(r["part"].tok2blk, b["bid"])
    np.testing.assert_allclose(r["sigma"], b["sigma"], rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(r["sel"], b["sel"])
    for key in ("oc", "os", "ow", "out"):
        np.testing.assert_allclose(r[key], b[key], rtol=1e-11, atol=1e-12, err_msg=key)


def test_forced_selection_matches_brute():
    rng = np.random.default_rng(5)
    c = tiny_case(rng, 50, 6, 2, 4)
    inp = _inp(c, 2, 2, 2)
    M = oracle.partition(c["coords"], 2, 6).M
    forced = np.full((2, M, 2), -1)
    for h in range(2):
        for b in range(M):
            forced[h, b, :2] = np.sort(rng.choice(M, 2, replace=False))
    ov = {(h, b): forced[h, b] for h in range(2) for b in range(M)}
    r = oracle.forward(inp, sel_override=ov)
    bb = brute_forward(c["coords"], c["q"], c["k"], c["v"], c["wk"], c["wv"], c["gates"], 2, 2, 2,
                       sel_force=forced)
    np.testing.assert_allclose(r["out"], bb["out"], rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- partition
def test_partition_against_grouping():
    rng = np.random.default_rng(11)
    for G, B, N in [(16, 4, 300), (9, 2, 200), (30, 7, 500), (5, 8, 20)]:
        coords = rng.integers(0, G, (N, 3))
        part = oracle.partition(coords, B, G)
        groups = {}
        for i, cc in enumerate(coords):
            groups.setdefault(tuple(int(x) // B for x in cc), []).append(i)
        keys = sorted(groups)
        assert part.M == len(keys)
        for b, kk in enumerate(keys):
            assert list(part.tokens(b)) == groups[kk]          # ascending token index
            assert all(part.tok2blk[i] == b for i in groups[kk])
        nb = -(-G // B)
        assert list(part.blk_key) == [(x * nb + y) * nb + z for x, y, z in keys]
        assert part.blk_off[0] == 0 and part.blk_off[-1] == N


def test_partition_rejects_out_of_grid():
    with pytest.raises(ValueError):
        oracle.partition(np.array([[0, 0, 8]]), 2, 8)
    with pytest.raises(ValueError):
        oracle.partition(np.array([[-1, 0, 0]]), 2, 8)


# ---------------------------------------------------------------- closed forms / textbook
def _full(c, scale=None):
    d = c["q"].shape[2]
    return oracle.sdpa_dense(c["q"], c["k"], c["v"], 1 / math.sqrt(d) if scale is None else scale)


def test_topk_covering_all_blocks_is_full_attention():
    rng = np.random.default_rng(1)
    c = tiny_case(rng, 60, 8, 2, 4)
    r = oracle.forward(_inp(c, 2, 2, 10 ** 4))
    np.testing.assert_allclose(r["os"], _full(c), rtol=1e-11, atol=1e-12)
    M = r["part"].M
    assert (r["sel"][:, :, :M] == np.arange(M)).all() and (r["sel"][:, :, M:] == -1).all()


def test_window_covering_grid_is_full_attention():
    rng = np.random.default_rng(2)
    c = tiny_case(rng, 60, 8, 2, 4)
    r = oracle.forward(_inp(c, 2, 8, 2))
    np.testing.assert_allclose(r["ow"], _full(c), rtol=1e-11, atol=1e-12)
    r = oracle.forward(_inp(c, 2, 1000, 2))
    np.testing.assert_allclose(r["ow"], _full(c), rtol=1e-11, atol=1e-12)


def test_unit_window_returns_own_value():
    rng = np.random.default_rng(3)
    c = tiny_case(rng, 40, 6, 2, 4)
    r = oracle.forward(_inp(c, 2, 1, 2))
    np.testing.assert_allclose(r["ow"], c["v"], rtol=0, atol=1e-14)


def test_unit_blocks_identity_projection_is_full_attention():
    rng = np.random.default_rng(4)
    c = tiny_case(rng, 50, 6, 2, 4)
    c["wk"] = np.eye(4)
    c["wv"] = np.eye(4)
    r = oracle.forward(_inp(c, 1, 1, 2))
    np.testing.assert_allclose(r["oc"], _full(c), rtol=1e-11, atol=1e-12)


def test_single_block_pool_closed_form():
    rng = np.random.default_rng(5)
    c = tiny_case(rng, 30, 4, 2, 4)
    r = oracle.forward(_inp(c, 4, 2, 3))
    assert r["part"].M == 1
    kt = c["k"].mean(axis=0) @ c["wk"]
    vt = c["v"].mean(axis=0) @ c["wv"]
    np.testing.assert_allclose(r["ktil"][:, 0], kt, atol=1e-14)
    np.testing.assert_allclose(r["oc"], np.broadcast_to(vt, r["oc"].shape), atol=1e-14)
    assert (r["sel"][:, 0] == np.array([0, -1, -1])).all()


def test_unit_block_identity_pool_is_identity():
    rng = np.random.default_rng(6)
    c = tiny_case(rng, 30, 5, 2, 4)
    part = oracle.partition(c["coords"], 1, 5)
    kt, vt = oracle.pool(c["k"], c["v"], np.eye(4), np.eye(4), part)
    np.testing.assert_allclose(kt, c["k"][part.perm].transpose(1, 0, 2), atol=0)
    np.testing.assert_allclose(vt, c["v"][part.perm].transpose(1, 0, 2), atol=0)


def test_importance_sums_to_block_size():
    rng = np.random.default_rng(7)
    c = tiny_case(rng, 80, 8, 2, 4)
    r = oracle.forward(_inp(c, 2, 2, 2))
    n = np.diff(r["part"].blk_off)
    np.testing.assert_allclose(r["sigma"].sum(axis=2), np.broadcast_to(n, (2, len(n))), rtol=1e-13)


def test_topk_brute_and_ties():
    rng = np.random.default_rng(8)
    for _ in range(50):
        M = int(rng.integers(1, 30))
        k = int(rng.integers(1, 35))
        sig = rng.integers(0, 5, M).astype(np.float64)      # many exact ties
        got = oracle.select_topk(sig, k)
        full = sorted(range(M), key=lambda b: (-sig[b], b))[:k]
        exp = np.full(k, -1)
        exp[:len(full)] = sorted(full)
        np.testing.assert_array_equal(got, exp)


def test_constant_values_identity_projection():
    rng = np.random.default_rng(9)
    c = tiny_case(rng, 50, 6, 2, 4)
    c["v"] = np.full_like(c["v"], 0.75)
    c["wv"] = np.eye(4)
    r = oracle.forward(_inp(c, 2, 2, 2))
    gs = c["gates"].sum(axis=2, keepdims=True)
    np.testing.assert_allclose(r["out"], 0.75 * np.broadcast_to(gs, r["out"].shape), rtol=1e-13)


def test_gates_linear_and_isolate_branches():
    rng = np.random.default_rng(10)
    c = tiny_case(rng, 50, 6, 2, 4)
    base = oracle.forward(_inp(c, 2, 2, 2))
    for x, key in enumerate(("oc", "os", "ow")):
        c2 = dict(c)
        g = np.zeros_like(c["gates"])
        g[..., x] = 1.0
        c2["gates"] = g
        r = oracle.forward(_inp(c2, 2, 2, 2))
        np.testing.assert_allclose(r["out"], base[key], atol=1e-15)


# ---------------------------------------------------------------- invariants
def test_token_permutation_equivariance():
    rng = np.random.default_rng(12)
    c = tiny_case(rng, 70, 8, 2, 4)
    r = oracle.forward(_inp(c, 2, 2, 3))
    pi = rng.permutation(70)
    c2 = {kk: (vv[pi] if isinstance(vv, np.ndarray) and vv.shape[:1] == (70,) else vv) for kk, vv in c.items()}
    r2 = oracle.forward(_inp(c2, 2, 2, 3))
    np.testing.assert_array_equal(r2["sel"], r["sel"])
    np.testing.assert_allclose(r2["out"], r["out"][pi], rtol=1e-12, atol=1e-13)


def test_within_block_permutation_invariance():
    rng = np.random.default_rng(13)
    c = tiny_case(rng, 70, 8, 2, 4)
    r = oracle.forward(_inp(c, 4, 4, 3))
    part = r["part"]
    # swap the caller positions of tokens only inside each block
    pi = np.arange(70)
    for b in range(part.M):
        t = part.tokens(b)
        pi[t] = rng.permutation(t)
    c2 = {kk: (vv[pi] if isinstance(vv, np.ndarray) and vv.shape[:1] == (70,) else vv) for kk, vv in c.items()}
    r2 = oracle.forward(_inp(c2, 4, 4, 3))
    np.testing.assert_array_equal(r2["sel"], r["sel"])
    np.testing.assert_allclose(r2["out"], r["out"][pi], rtol=1e-12, atol=1e-13)


def test_translation_invariance():
    rng = np.random.default_rng(14)
    c = tiny_case(rng, 60, 8, 2, 4)
    c["grid"] = 16
    r = oracle.forward(_inp(c, 2, 4, 3))
    c2 = dict(c)
    c2["coords"] = c["coords"] + np.array([4, 8, 4], np.int32)
    r2 = oracle.forward(_inp(c2, 2, 4, 3))
    np.testing.assert_array_equal(r2["sel"], r["sel"])
    np.testing.assert_allclose(r2["out"], r["out"], rtol=1e-13, atol=1e-14)


def test_query_scale_tradeoff():
    rng = np.random.default_rng(15)
    c = tiny_case(rng, 60, 8, 2, 4)
    r = oracle.forward(_inp(c, 2, 2, 3), scale=0.5)
    c2 = dict(c)
    c2["q"] = c["q"] * 4.0
    r2 = oracle.forward(_inp(c2, 2, 2, 3), scale=0.125)
    np.testing.assert_array_equal(r2["sel"], r["sel"])
    np.testing.assert_allclose(r2["out"], r["out"], rtol=1e-12, atol=1e-13)


def test_forward_items_matches_forward():
    rng = np.random.default_rng(16)
    c = tiny_case(rng, 60, 8, 2, 4)
    inp = _inp(c, 2, 2, 3)
    r = oracle.forward(inp)
    items = [(1, 3), (0, 0)]
    ri = oracle.forward_items(inp, items)
    for it in items:
        np.testing.assert_array_equal(ri[it]["out"], r["out"][ri[it]["rows"], it[0]])

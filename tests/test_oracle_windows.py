"""Pins of the oracle's window partitions beyond cells that are unions of blocks: shifted
cubic cells of any edge and fixed-size windows along the Morton order (the pages' local
windows: pixal-3d.com "What is Direct3D-S2?"; the Hi3D pipeline page, "Stage 4")."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W
from brute import brute_forward, spread_morton, tiny_case

GOLD = os.path.join(os.path.dirname(__file__), "golden", "morton_codes.json")


def _groups_by_dict(coords, w, shift):
    cells = {}
    for i, c in enumerate(np.asarray(coords, np.int64)):
        key = tuple(int(x) for x in (c + np.asarray(shift)) // w)
        cells.setdefault(key, []).append(i)
    return [cells[k] for k in sorted(cells)]


@pytest.mark.parametrize("w,shift", [(3, (1, 2, 0)), (4, (2, 2, 2)), (1, (0, 0, 0)), (5, (4, 0, 3)),
                                     (16, (8, 8, 8))])
def test_shifted_cells_group_like_dict(w, shift):
    rng = np.random.default_rng(w + sum(shift))
    coords = rng.integers(0, 13, (400, 3)).astype(np.int32)     # duplicates allowed
    wp = oracle.window_partition(coords, w, 13, shift)
    got = [list(wp.tokens(c)) for c in range(wp.M)]
    assert got == _groups_by_dict(coords, w, shift)


def test_shift_is_a_translation():
    rng = np.random.default_rng(3)
    coords = rng.integers(0, 20, (300, 3)).astype(np.int32)
    s = (3, 1, 4)
    a = oracle.window_partition(coords, 6, 20, s)
    b = oracle.window_partition(coords + np.asarray(s, np.int32), 6, 26)
    np.testing.assert_array_equal(a.perm, b.perm)
    np.testing.assert_array_equal(a.blk_off, b.blk_off)


def test_morton_golden():
    gold = json.load(open(GOLD))
    for case in gold["cases"]:
        code = oracle.morton_codes(np.asarray([case["coord"]]), case["bits"])[0]
        assert code == case["code"], case


def test_morton_matches_bit_spreading():
    rng = np.random.default_rng(7)
    coords = rng.integers(0, 1024, (5000, 3))
    np.testing.assert_array_equal(oracle.morton_codes(coords, 10), spread_morton(coords))


@pytest.mark.parametrize("tokens", [1, 7, 64, 1000])
def test_sfc_windows_structure(tokens):
    rng = np.random.default_rng(tokens)
    coords = rng.integers(0, 32, (500, 3))
    wp = oracle.sfc_windows(coords, tokens, 32)
    sizes = np.diff(wp.blk_off)
    assert sizes.sum() == 500 and (sizes[:-1] == tokens).all() and 0 < sizes[-1] <= tokens
    code = spread_morton(coords)
    rank = np.empty(500, np.int64)
    rank[np.lexsort((np.arange(500), code))] = np.arange(500)
    np.testing.assert_array_equal(wp.tok2blk, rank // tokens)
    for c in range(wp.M):   # each window lists its tokens in Morton order
        t = wp.tokens(c)
        assert (np.diff(code[t]) >= 0).all()


def _inp(N, G, H, d, B, w, k, seed, **win):
    rng = np.random.default_rng(seed)
    c = tiny_case(rng, N, G, H, d)
    c.update(block=B, window=w, topk=k, **win)
    return c


@pytest.mark.parametrize("win", [dict(window_shift=(1, 0, 2)), dict(window_shift=(2, 2, 2)),
                                 dict(sfc_tokens=9), dict(sfc_tokens=40)])
@pytest.mark.parametrize("w", [3, 4])
def test_forward_matches_brute(win, w):
    inp = _inp(120, 9, 2, 8, 2, w, 3, seed=w * 10 + len(str(win)), **win)
    if "window_shift" in win:
        win = dict(win)
        win["window_shift"] = tuple(min(x, w - 1) for x in win["window_shift"])
        inp.update(win)
    ref = oracle.forward(inp)
    b = brute_forward(inp["coords"], inp["q"], inp["k"], inp["v"], inp["wk"], inp["wv"], inp["gates"],
                      2, w, 3, sel_force=ref["sel"], shift=inp.get("window_shift", (0, 0, 0)),
                      sfc_tokens=inp.get("sfc_tokens", 0))
    np.testing.assert_allclose(ref["ow"], b["ow"], atol=1e-12)
    np.testing.assert_allclose(ref["out"], b["out"], atol=1e-12)


def test_sfc_one_window_is_dense_attention():
    inp = _inp(150, 8, 2, 16, 2, 2, 3, seed=1, sfc_tokens=150)
    ref = oracle.forward(inp)
    dense = oracle.sdpa_dense(inp["q"], inp["k"], inp["v"], 1 / np.sqrt(16))
    np.testing.assert_allclose(ref["ow"], dense, atol=1e-12)


@pytest.mark.parametrize("win", [dict(sfc_tokens=1), dict(window=1, window_shift=(0, 0, 0))])
def test_unit_windows_return_v(win):
    inp = _inp(150, 8, 2, 16, 2, 2, 3, seed=2)
    inp.update(win)
    ref = oracle.forward(inp)
    np.testing.assert_allclose(ref["ow"], inp["v"], atol=1e-12)

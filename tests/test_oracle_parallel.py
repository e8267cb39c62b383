"""The process-pool driver of the oracle (used for parity at full size) reproduces the
single-process oracle, and the full-size checkers built on it catch wrong outputs and
wrong selections."""
import numpy as np
import pytest

import oracle
import workloads as W
from brute import tiny_case
from parity import check_backward_all, check_forward_all


def _case(dt="f32", N=600, G=12, H=3, d=32, B=2, w=4, k=3):
    rng = np.random.default_rng(17)
    c = tiny_case(rng, N, G, H, d)
    inp = W.random_inputs(c["coords"], H, d, dt, seed=5, grid=G, backward=True)
    inp.update(block=B, window=w, topk=k)
    return inp


def test_pool_forward_matches_single_process():
    inp = _case()
    ref = oracle.forward(inp)
    counts, mx, rel = check_forward_all(inp, ref["out"], ref["sel"], workers=3)
    assert counts["exact"] + counts["near"] == 3 * ref["part"].M
    assert mx <= 1e-12


def test_pool_forward_catches_errors():
    inp = _case()
    ref = oracle.forward(inp)
    bad = ref["out"].copy()
    bad[123, 1, 7] += 1e-3                     # above the fp32 bound
    with pytest.raises(AssertionError):
        check_forward_all(inp, bad, ref["sel"], workers=2)
    sel = ref["sel"].copy()
    h, b = 2, 5
    M = ref["part"].M
    row = sel[h, b]
    sigma = ref["sigma"][h, b]
    worst = int(np.argmin(sigma))                # a block that is clearly not selected
    assert worst not in row
    row = np.sort(np.concatenate([row[1:], [worst]]))
    sel[h, b] = row
    with pytest.raises(AssertionError):
        check_forward_all(inp, ref["out"], sel, workers=2)
    assert M > 3


def test_pool_backward_matches_single_process():
    inp = _case(H=2)
    ref = oracle.forward(inp)
    grads = oracle.backward(inp, ref["sel"], inp["do"])
    res = check_backward_all(inp, ref["sel"], grads, workers=2)
    for name, (mx, rel) in res.items():
        assert mx <= 1e-12, name
    bad = [g.copy() for g in grads]
    bad[2][10, 1, 3] += 1e-3
    with pytest.raises(AssertionError):
        check_backward_all(inp, ref["sel"], bad, workers=2)

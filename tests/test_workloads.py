"""The seeded generators: deterministic per seed, exact N, distinct in-grid voxels."""
import numpy as np
import pytest

import workloads as W


@pytest.mark.parametrize("name", ["sphere2k", "torus20k", "shells80k"])
def test_geometry_deterministic_distinct(name):
    wl = W.WORKLOADS[name]
    a = W.make_geometry(wl)
    b = W.make_geometry(wl)
    np.testing.assert_array_equal(a, b)
    assert a.shape == (wl.n, 3) and a.dtype == np.int32
    assert len(np.unique(a, axis=0)) == wl.n
    assert a.min() >= 0 and a.max() < wl.grid


def test_dtype_rounding_exact():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(1000)
    for dt, bits in (("f16", 11), ("bf16", 8)):
        y = W.round_to_dtype(x, dt)
        # representable: a second rounding is the identity
        np.testing.assert_array_equal(W.round_to_dtype(y, dt), y)
        assert np.max(np.abs(y - x) / np.abs(x)) <= 2.0 ** -bits + 1e-9


def test_inputs_shapes():
    wl, inp = W.make_inputs("sphere2k")
    assert inp["q"].shape == (2048, 2, 32) and inp["gates"].shape == (2048, 2, 3)
    assert inp["wk"].shape == (32, 32)
    assert 0 <= inp["gates"].min() and inp["gates"].max() <= 1

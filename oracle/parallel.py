"""Process-pool driver for the float64 oracle.

TEST INFRASTRUCTURE ONLY: used by tests/ (parity at the full workload sizes) and by
the benchmark's cpu_baseline leg, never by the HIP product path.

It adds no arithmetic.  SSA is computed independently per head (every branch, the
pooling and the selection act on one head's slice), so the oracle's functions can
be called on a one-head slice of the inputs; this module runs such calls in worker
processes, one BLAS thread each, with the large arrays shared through read-only
memory-mapped files instead of being copied into every worker.

    with HeadPool(inp) as hp:
        results = hp.map(fn, tasks)      # fn(head_inputs, h, payload, shared) -> anything

`fn` must be a module-level function (workers are spawned, so it is imported by
name); `head_inputs` is a dict like the oracle's input dict with q, k, v, gates (and
do) restricted to head h, as float32 arrays of shape [N, 1, d] / [N, 1, 3].
`shared` maps extra array names given to HeadPool (e.g. pooled keys) to memory maps.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import shutil
import tempfile

import numpy as np

_TOKEN_ARRAYS = ("q", "k", "v", "gates", "do")
_G: dict = {}


def workers_available() -> int:
    """Host cores this process may run on (the machine's CPU share), at most 16 workers."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _init(path, meta, names):
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass
    _G["meta"] = meta
    _G["arrays"] = {nm: np.load(os.path.join(path, nm + ".npy"), mmap_mode="r") for nm in names}


def _head_inputs(h):
    a = _G["arrays"]
    inp = dict(_G["meta"])
    for key in _TOKEN_ARRAYS:
        if key in a:
            inp[key] = np.ascontiguousarray(a[key][:, h:h + 1])
    inp["coords"] = np.asarray(a["coords"])
    inp["wk"] = np.asarray(a["wk"])
    inp["wv"] = np.asarray(a["wv"])
    for nm in ("wk_conv", "wv_conv"):
        if nm in a:
            inp[nm] = np.asarray(a[nm])
    return inp


def _run(job):
    fn, h, payload = job
    return fn(_head_inputs(h), h, payload, _G["arrays"])


class HeadPool:
    """A spawned process pool over one SSA input dict (see the module docstring)."""

    def __init__(self, inp: dict, shared: dict | None = None, workers: int | None = None):
        self.workers = workers or workers_available()
        self.dir = tempfile.mkdtemp(prefix="ssa_oracle_pool_")
        names = []
        arrays = {k: inp[k] for k in _TOKEN_ARRAYS if k in inp}
        arrays.update(coords=inp["coords"], wk=inp["wk"], wv=inp["wv"])
        for nm in ("wk_conv", "wv_conv"):
            if inp.get(nm) is not None:
                arrays[nm] = inp[nm]
        arrays.update(shared or {})
        for nm, arr in arrays.items():
            np.save(os.path.join(self.dir, nm + ".npy"), np.ascontiguousarray(arr))
            names.append(nm)
        meta = {k: inp[k] for k in ("grid", "block", "window", "topk", "dtype", "window_shift", "sfc_tokens")
                if k in inp}
        if "scale" in inp:
            meta["scale"] = inp["scale"]
        ctx = mp.get_context("spawn")
        self.pool = ctx.Pool(self.workers, initializer=_init, initargs=(self.dir, meta, names))

    def map(self, fn, tasks):
        """tasks: iterable of (h, payload).  Results in task order."""
        return self.pool.map(_run, [(fn, h, p) for h, p in tasks], chunksize=1)

    def close(self):
        if self.pool is not None:
            self.pool.close()
            self.pool.join()
            self.pool = None
        shutil.rmtree(self.dir, ignore_errors=True)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        if exc[0] is not None and self.pool is not None:
            self.pool.terminate()
            self.pool.join()
            self.pool = None
        self.close()


def forward_blocks_task(inp_h, h, payload, shared):
    """The oracle forward of the blocks `payload` of head h (pooled keys shared as "ktil",
    "vtil" [H, M, d]).  Returns the number of blocks done."""
    import oracle
    ktv = (np.asarray(shared["ktil"][h:h + 1]), np.asarray(shared["vtil"][h:h + 1]))
    oracle.forward_items(inp_h, [(0, int(b)) for b in payload], ktv=ktv)
    return len(payload)

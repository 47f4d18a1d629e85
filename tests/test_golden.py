"""The stored full-size samples must be what the current oracle computes.

tests/golden/large_slices.json is written only by tests/golden/make_golden.py,
which calls the oracle.  Re-running the cheapest stored case (a [1408,2048]
expert slice, about a second of float64 BLAS) checks that the file is in step
with the oracle's arithmetic; the other cases are structural checks.
"""

from __future__ import annotations

import json
import os

import numpy as np

import oracle
import workloads

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
GOLDEN = os.path.join(GOLDEN_DIR, "large_slices.json")
TILES = os.path.join(GOLDEN_DIR, "large_last_tiles.json")
TILE_VALUES = os.path.join(GOLDEN_DIR, "large_last_tiles.npz")


def _load():
    with open(GOLDEN) as f:
        return json.load(f)


def test_golden_structure():
    d = _load()
    assert d["samples"] == 1024
    for c in d["cases"]:
        wl = workloads.WORKLOADS[c["workload"]]
        spec = wl.params[c["param"]]
        assert list(spec.shape[-2:]) == c["shape"]
        assert c["ns_steps"] == wl.ns_steps and tuple(c["coeffs"]) == tuple(wl.coeffs)
        idx = np.asarray(c["index"])
        assert len(set(idx.tolist())) == idx.size == 1024
        assert idx.min() >= 0 and idx.max() < c["shape"][0] * c["shape"][1]
        assert np.all(np.isfinite(c["value"])) and c["frobenius"] > 0


def test_golden_matches_oracle_expert_slice():
    d = _load()
    c = next(c for c in d["cases"] if c["shape"] == [1408, 2048])
    wl = workloads.WORKLOADS[c["workload"]]
    g = workloads.gradient(wl, c["param"])[c["slice"]]
    m = oracle.momentum_update(np.zeros(g.shape, np.float32), g, wl.beta)
    o = oracle.orthogonalize(m, wl.ns_steps, *wl.coeffs)
    np.testing.assert_allclose(o.reshape(-1)[c["index"]], c["value"], rtol=0, atol=1e-12)
    assert abs(np.linalg.norm(o) - c["frobenius"]) < 1e-9


def test_last_tiles_structure():
    """One tile per large bucket, of the bucket's last slice, at the
    bottom-right 256-aligned corner of the stored shape."""
    with open(TILES) as f:
        d = json.load(f)
    values = np.load(TILE_VALUES)
    buckets = set()
    for c in d["cases"]:
        wl = workloads.WORKLOADS[c["workload"]]
        spec = wl.params[c["param"]]
        rows, cols = spec.shape[-2:]
        assert c["shape"] == [rows, cols]
        key = (c["workload"], min(rows, cols), max(rows, cols))
        # the last parameter and slice of this oriented shape in the workload
        last = max(i for i, p in enumerate(wl.params) if (min(p.shape[-2:]), max(p.shape[-2:])) == key[1:])
        assert c["param"] == last
        assert c["slice"] == (spec.shape[0] - 1 if len(spec.shape) == 3 else 0)
        assert c["row0"] == (rows - 1) // 256 * 256 and c["col0"] == (cols - 1) // 256 * 256
        t = values[c["array"]]
        assert t.shape == (rows - c["row0"], cols - c["col0"]) and np.all(np.isfinite(t))
        assert abs(float(np.linalg.norm(t.astype(np.float64))) - c["tile_frobenius"]) < 1e-5 * c["tile_frobenius"]
        buckets.add(key)
    large = {(n, min(p.shape[-2:]), max(p.shape[-2:])) for n, wl in workloads.WORKLOADS.items()
             for p in wl.params if min(p.shape[-2:]) >= 129}
    assert buckets == large


def test_last_tile_matches_oracle_expert_slice():
    """Re-derive the cheapest stored tile (the last [1408,2048] expert, with
    its ragged 128-row tile row)."""
    with open(TILES) as f:
        c = next(c for c in json.load(f)["cases"] if c["shape"] == [1408, 2048])
    wl = workloads.WORKLOADS[c["workload"]]
    g = workloads.gradient(wl, c["param"])[c["slice"]]
    m = oracle.momentum_update(np.zeros(g.shape, np.float32), g, wl.beta)
    o = oracle.orthogonalize(m, wl.ns_steps, *wl.coeffs)
    tile = np.load(TILE_VALUES)[c["array"]]
    assert tile.shape == (128, 256)
    np.testing.assert_allclose(tile, o[c["row0"]:, c["col0"]:].astype(np.float32), rtol=0, atol=0)
    assert abs(np.linalg.norm(o) - c["frobenius"]) < 1e-9

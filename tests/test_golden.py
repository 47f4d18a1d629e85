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

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "large_slices.json")


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

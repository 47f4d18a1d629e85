"""Write the expected values for the full-size parity tests.

    python tests/golden/make_golden.py        # a few minutes of float64 on the host

For one slice of every large bucket of the workloads, run the CPU oracle (the
only code that produces the expected values) on the seeded gradient of that
parameter (zero momentum, zero weights, so the update is -lr O) and store
1024 sampled entries of O together with the sample positions and ||O||_F
(large_slices.json).

For the LAST slice of every large bucket, store the contiguous bottom-right
tile of O: rows and columns from the last multiple of 256 below the stored
shape to its end, the 256 x 256 output tile of the products that holds the
ragged edge where the shape is not a multiple of 256 (large_last_tiles.json
for the positions and norms, large_last_tiles.npz for the values as float32).

The GPU test runs the full fused workload, with these parameters' gradients
bit-identical, and compares the sampled entries and the tiles.
"""

from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

N_SAMPLES = 1024

# (workload, parameter index, slice index): one slice per large oriented shape.
CASES = [
    ("moe_experts", 1, 5),        # [1408, 2048] expert slice
    ("dense_h4096_l8", 0, 0),     # [4096, 12288]
    ("dense_h4096_l8", 1, 0),     # [4096, 4096]
    ("dense_h4096_l8", 2, 0),     # [4096, 16384]
    ("dense_h4096_l8", 3, 0),     # [16384, 4096] (transposed)
    ("large_share", 0, 0),        # [8192, 8192]
    ("large_share", 4, 0),        # [16384, 4096] (transposed)
]


# (workload, parameter index, slice index): the last slice of each large bucket.
LAST_TILE_CASES = [
    ("moe_experts", 1, 63),       # [1408, 2048]: 1408 = 5 x 256 + 128, a ragged tile row
    ("dense_h4096_l8", 28, 0),    # [4096, 12288], layer 7
    ("dense_h4096_l8", 29, 0),    # [4096, 4096], layer 7
    ("dense_h4096_l8", 31, 0),    # [16384, 4096] (transposed), layer 7: the last of the 16 [4096, 16384]
    ("large_share", 3, 0),        # [8192, 8192]
    ("large_share", 7, 0),        # [16384, 4096] (transposed)
]
TILE = 256


def oracle_o(name, pidx, sidx):
    wl = workloads.WORKLOADS[name]
    spec = wl.params[pidx]
    g = workloads.gradient(wl, pidx)
    g2 = g[sidx] if len(spec.shape) == 3 else g
    m_new = oracle.momentum_update(np.zeros(g2.shape, np.float32), g2, wl.beta)
    return wl, oracle.orthogonalize(m_new, wl.ns_steps, *wl.coeffs)


def last_tiles():
    meta, arrays = [], {}
    for k, (name, pidx, sidx) in enumerate(LAST_TILE_CASES):
        t0 = time.time()
        wl, o = oracle_o(name, pidx, sidx)
        rows, cols = o.shape
        r0, c0 = (rows - 1) // TILE * TILE, (cols - 1) // TILE * TILE
        arrays[f"tile{k}"] = o[r0:, c0:].astype(np.float32)
        meta.append({"workload": name, "param": pidx, "slice": sidx, "shape": [rows, cols],
                     "ns_steps": wl.ns_steps, "beta": wl.beta, "coeffs": list(wl.coeffs),
                     "frobenius": float(np.linalg.norm(o)), "row0": r0, "col0": c0,
                     "tile_frobenius": float(np.linalg.norm(o[r0:, c0:])), "array": f"tile{k}"})
        print(f"{name} param {pidx} slice {sidx} {o.shape}: tile [{r0}:, {c0}:] {time.time() - t0:.1f} s",
              flush=True)
    np.savez_compressed(os.path.join(HERE, "large_last_tiles.npz"), **arrays)
    with open(os.path.join(HERE, "large_last_tiles.json"), "w") as f:
        json.dump({"note": "written by tests/golden/make_golden.py from the float64 oracle",
                   "tile": TILE, "cases": meta}, f, indent=1)


def main():
    if "--tiles-only" not in sys.argv:
        sampled()
    last_tiles()


def sampled():
    out = []
    for name, pidx, sidx in CASES:
        wl = workloads.WORKLOADS[name]
        spec = wl.params[pidx]
        g = workloads.gradient(wl, pidx)
        g2 = g[sidx] if len(spec.shape) == 3 else g
        t0 = time.time()
        m_new = oracle.momentum_update(np.zeros(g2.shape, np.float32), g2, wl.beta)
        o = oracle.orthogonalize(m_new, wl.ns_steps, *wl.coeffs)
        dt = time.time() - t0
        rng = np.random.default_rng(12345 + len(out))
        flat = rng.choice(o.size, size=N_SAMPLES, replace=False)
        out.append({
            "workload": name, "param": pidx, "slice": sidx, "shape": list(g2.shape),
            "ns_steps": wl.ns_steps, "beta": wl.beta, "coeffs": list(wl.coeffs),
            "frobenius": float(np.linalg.norm(o)),
            "index": [int(i) for i in flat],
            "value": [float(v) for v in o.reshape(-1)[flat]],
        })
        print(f"{name} param {pidx} slice {sidx} {g2.shape}: {dt:.1f} s", flush=True)
    with open(os.path.join(HERE, "large_slices.json"), "w") as f:
        json.dump({"note": "written by tests/golden/make_golden.py from the float64 oracle",
                   "samples": N_SAMPLES, "cases": out}, f)


if __name__ == "__main__":
    main()

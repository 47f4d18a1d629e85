"""Seeded random plans against the oracle.

Each case draws a plan of 1-5 parameters from every kernel path: tiny
slices, skinny (m <= 32), small streamed (m <= 256), the tiled products
(float32 mode, m > 256) and the large tiles (bf16 mode, m >= 129).  It also
draws the stored orientation, 3-D stacks, gradient and weight storage types,
the update variants, the number of rounds (0-6) and the coefficient set
(quintic or cubic).  Inputs are the seeded generators' Gaussians with nonzero
weights and momentum.

Checks per slice: the change of W against the oracle's, within the mode's
bar and the block-local check (float32 weights); one bf16 rounding of W on
top of that bar (bf16 weights); momentum within 1 ulp of the oracle's
float32 value.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import TOL, gpu_step, make_inputs, max_ulp_diff, oracle_step, slice_rel_errors

pytestmark = pytest.mark.gpu

CASES = 160
CUBIC = (1.5, -0.5, 0.0)


def _draw(case):
    rng = np.random.default_rng(7000 + case)
    mode = "bf16" if case % 2 == 0 else "fp32"
    shapes, gds, pds = [], [], []
    for _ in range(int(rng.integers(1, 6))):
        kind = str(rng.choice(["tiny", "skinny", "small", "mid"]))
        if kind == "tiny":
            m = int(rng.integers(1, 9))
            n = int(rng.integers(m, 40))
        elif kind == "skinny":
            m = int(rng.integers(1, 33))
            n = int(rng.integers(33, 3000))
        elif kind == "small":
            m = int(rng.integers(33, 257))
            n = int(rng.integers(m, 900))
        else:
            m = int(rng.integers(257, 700))
            n = int(rng.integers(m, 1100))
        shape = (n, m) if rng.random() < 0.4 else (m, n)
        if rng.random() < 0.25:
            shape = (int(rng.integers(2, 4)),) + shape
        shapes.append(shape)
        gds.append(str(rng.choice(["bf16", "f32"])))
        pds.append("bf16" if rng.random() < 0.3 else "f32")
    variant = dict(nesterov=bool(rng.random() < 0.3), weight_decay=0.1 if rng.random() < 0.3 else 0.0,
                   update_scale=str(rng.choice(["none", "aspect", "rms"])))
    ns = int(rng.integers(0, 7))
    coeffs = workloads.QUINTIC if rng.random() < 0.7 else CUBIC
    return mode, shapes, gds, pds, variant, ns, coeffs


@pytest.mark.parametrize("case", range(CASES))
def test_random_plan(case):
    mode, shapes, gds, pds, variant, ns, coeffs = _draw(case)
    print(f"case {case}: {mode} {shapes} grads {gds} params {pds} {variant} ns={ns} coeffs={coeffs}", flush=True)
    params, grads, moms = make_inputs(shapes, gds, 7100 + 10 * case, 1e-3, pds, w_std=0.02, m_std=1e-3)
    w_gpu, m_gpu = gpu_step(params, grads, moms, mode=mode, lr=0.02, beta=0.9, ns_steps=ns, coeffs=coeffs,
                            plan_kw=variant)
    w_ref, m_ref, _ = oracle_step(params, grads, moms, lr=0.02, beta=0.9, ns_steps=ns, coeffs=coeffs, **variant)
    tol = TOL[mode]
    for i, shape in enumerate(shapes):
        assert max_ulp_diff(m_gpu[i], m_ref[i]) <= 1, f"momentum of parameter {i} {shape}"
        w0 = oracle.decode(params[i]) if params[i].dtype == np.uint16 else params[i].astype(np.float64)
        if pds[i] == "bf16":
            got = oracle.decode(w_gpu[i])
            err = np.linalg.norm(got - w_ref[i])
            bound = 2.0 ** -8 * np.linalg.norm(w_ref[i]) + tol * np.linalg.norm(w_ref[i] - w0)
            assert err <= bound, (i, shape, err, bound)
        else:
            errs = slice_rel_errors(w_gpu[i].astype(np.float64) - w0, w_ref[i] - w0, tol)
            assert max(errs) <= tol, (i, shape, max(errs))

"""Parity of the opt-in update variants (Nesterov momentum, decoupled weight
decay, shape factor of the update) on every kernel path: skinny (m <= 32),
128-tile streamed, and the large bf16 products, both storage orientations.

The oracle applies the variants to the same seeded inputs; the check is the
change of W per slice, ||dW_gpu - dW_ref||_F / ||dW_ref||_F, against the
mode's bar (the change is lr f O plus the exactly known decay term)."""

from __future__ import annotations

import numpy as np
import pytest

from gpu_helpers import TOL, gpu_step, make_inputs, oracle_step, slice_rel_errors

pytestmark = pytest.mark.gpu

Q = (3.4445, -4.7750, 2.0315)
PATHS = {
    "skinny": [(24, 1000), (1000, 24)],
    "streamed": [(96, 300), (300, 96)],
    "large": [(600, 700), (700, 600)],
}
VARIANTS = [
    dict(nesterov=True),
    dict(weight_decay=0.1),
    dict(update_scale="aspect"),
    dict(update_scale="rms", nesterov=True, weight_decay=0.05),
]


def _check(shapes, mode, variant, ns=5, seed=17):
    params, grads, moms = make_inputs(shapes, "bf16", seed, 1e-3, w_std=0.02, m_std=1e-3)
    w_gpu, m_gpu = gpu_step(params, grads, moms, mode=mode, lr=0.05, beta=0.9, ns_steps=ns, coeffs=Q,
                            plan_kw=variant)
    w_ref, m_ref, _ = oracle_step(params, grads, moms, lr=0.05, beta=0.9, ns_steps=ns, coeffs=Q, **variant)
    worst = 0.0
    for i in range(len(shapes)):
        w0 = params[i].astype(np.float64)
        worst = max(worst, max(slice_rel_errors(w_gpu[i].astype(np.float64) - w0, w_ref[i] - w0, TOL[mode])))
        assert max(slice_rel_errors(m_gpu[i], m_ref[i], 1e-6)) <= 1e-6
    print(f"{shapes} {mode} {variant} ns={ns}: worst {worst:.3e}", flush=True)
    assert worst <= TOL[mode], worst


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: "-".join(f"{k}={x}" for k, x in v.items()))
@pytest.mark.parametrize("mode", ["bf16", "fp32"])
@pytest.mark.parametrize("path", list(PATHS))
def test_update_variants(path, mode, variant):
    _check(PATHS[path], mode, variant)


@pytest.mark.parametrize("mode", ["bf16", "fp32"])
def test_update_variants_without_rounds(mode):
    """k = 0: the update is the normalised direction itself (skinny and
    streamed buckets take different kernels for it)."""
    _check([(24, 500), (96, 300), (300, 96), (600, 700)], mode,
           dict(update_scale="aspect", nesterov=True, weight_decay=0.1), ns=0)

"""Parity of the large-slice products (bf16 mode, m >= 129: 256 x 256 tiles,
float32 diagonal kept out of the bf16 operands, identity-shifted polynomial).

Sizes are chosen so that the oracle runs in seconds while the products still
span several 256-tiles and ragged edges: padding in m and n, both storage
orientations, 3-D stacks, rows of W that are not whole 16-byte groups, bf16
weights, every final-round position (k = 1, 2, 5) and repeated steps.
"""

from __future__ import annotations

import numpy as np
import pytest

from gpu_helpers import TOL, gpu_step, make_inputs, oracle_step, slice_rel_errors, update_errors

pytestmark = pytest.mark.gpu

Q = (3.4445, -4.7750, 2.0315)
# Expected worst error of this arithmetic at these sizes is about 4e-3 to
# 8e-3; the bar is the bf16-mode tolerance.
BAR = TOL["bf16"]


def _check(shapes, *, ns=5, steps=1, param_dtypes=None, w_std=0.0, m_std=0.0, seed=3, lr=1.0, plan_kw=None):
    params, grads, moms = make_inputs(shapes, "bf16", seed, 1e-3, param_dtypes, w_std, m_std)
    w_gpu, m_gpu = gpu_step(params, grads, moms, mode="bf16", lr=lr, beta=0.95, ns_steps=ns, coeffs=Q,
                            steps=steps, plan_kw=plan_kw)
    w_ref, m_ref, o_ref = oracle_step(params, grads, moms, lr=lr, beta=0.95, ns_steps=ns, coeffs=Q,
                                      steps=steps)
    worst = 0.0
    for i in range(len(shapes)):
        if steps == 1:
            errs = update_errors(w_gpu[i], params[i], lr, o_ref[i], BAR)
        else:  # compare the accumulated change of W, which the initial W would swamp
            w0 = params[i].astype(np.float64)
            errs = slice_rel_errors(w_gpu[i].astype(np.float64) - w0, w_ref[i] - w0, BAR)
        worst = max(worst, max(errs))
        assert max(slice_rel_errors(m_gpu[i], m_ref[i], 1e-6)) <= 1e-6
    print(f"{shapes} ns={ns} steps={steps}: worst {worst:.3e}", flush=True)
    assert worst <= BAR, worst
    return worst


@pytest.mark.parametrize("shape", [(600, 700), (700, 600), (1024, 1280), (514, 517), (2, 520, 1030),
                                   (2100, 2200)])
def test_large_shapes(shape):
    """(2100, 2200) has 9 row tiles of 256, so its tile table takes the
    4 x 8 blocks; the others have at most 8 and take whole-height blocks."""
    _check([shape])


@pytest.mark.parametrize("shape", [(129, 1000), (1000, 129), (200, 333), (256, 256), (2, 300, 520),
                                   (384, 1536), (512, 512)])
def test_mid_shapes(shape):
    """Slices with 129 <= m <= 512 take the large tiles too: one or two tile
    rows, so every tile of the symmetric phases sits on the diagonal, and
    m = 129 leaves all but one row of its tile row as padding."""
    _check([shape])


@pytest.mark.parametrize("shape", [(33, 500), (40, 400), (64, 1024), (1024, 64), (100, 300), (2, 120, 777)])
def test_large_tiles_down_to_m_33(shape):
    """large_min_m = 33 puts every streamed bf16 slice on the large tiles:
    one tile row holding 33 to 128 rows of the slice, so every tile of the
    Gram and polynomial is a half tile (its first 128 rows only), on the
    diagonal, where the waves whose columns lie past m skip their products."""
    _check([shape], plan_kw=dict(large_min_m=33))


@pytest.mark.parametrize("shape", [(257, 600), (600, 383), (640, 900), (900, 640), (385, 700), (2, 641, 700),
                                   (511, 1030), (2, 384, 520)])
def test_half_tile_boundaries(shape):
    """The symmetric phases' last tile row is a half tile when it holds at
    most 128 rows inside m (m mod 256 = 1, 127 and 128 here, stored either
    way round), and a full tile below the diagonal when it holds more
    (m mod 256 = 129 and 255).  Every 64 x 64 block of the update is
    checked, so a wrong or missing row of a half tile, or of its mirror
    writes, fails."""
    _check([shape])


def test_half_tiles_bf16_weights_and_steps():
    """Half tiles in a mixed plan over three steps, with nonzero W and M and
    a bf16 W next to float32 ones.  The bf16 W is rounded once per step
    (unit roundoff 2^-8 each time), the oracle's W not at all."""
    import oracle
    shapes = [(384, 700), (700, 384), (300, 520)]
    params, grads, moms = make_inputs(shapes, "bf16", 57, 1e-3, ["f32", "bf16", "f32"], 0.02, 1e-3)
    w_gpu, _ = gpu_step(params, grads, moms, mode="bf16", lr=0.02, beta=0.95, ns_steps=5, coeffs=Q, steps=3)
    w_ref, _, _ = oracle_step(params, grads, moms, lr=0.02, beta=0.95, ns_steps=5, coeffs=Q, steps=3)
    for i in range(len(shapes)):
        if i == 1:
            w0 = oracle.decode(params[i])
            err = np.linalg.norm(oracle.decode(w_gpu[i]) - w_ref[i])
            bound = 3 * 2.0 ** -8 * np.linalg.norm(w_ref[i]) + BAR * np.linalg.norm(w_ref[i] - w0)
            assert err <= bound, (shapes[i], err, bound)
        else:
            w0 = params[i].astype(np.float64)
            errs = slice_rel_errors(w_gpu[i].astype(np.float64) - w0, w_ref[i] - w0, BAR)
            assert max(errs) <= BAR, (shapes[i], max(errs))


def test_large_fusion_is_bitexact():
    """Fused large buckets give bitwise the W and M of one plan per slice:
    three [600,700] slices fused, the two slices of a [2,520,1030] stack,
    and two [2100,2200] slices (9 row tiles: the 4 x 8 block branch of the
    tile table) next to a transposed [700,600] and a [200,333] (one tile
    row).  A slice's products do not depend on which table entries or
    workgroups computed its tiles."""
    shapes = [(600, 700)] * 3 + [(2, 520, 1030), (2100, 2200), (2100, 2200), (700, 600), (200, 333)]
    params, grads, moms = make_inputs(shapes, "bf16", 83, w_std=0.02, m_std=1e-3)
    kw = dict(mode="bf16", lr=0.02, beta=0.95, ns_steps=5, coeffs=Q)
    w_f, m_f = gpu_step(params, grads, moms, **kw)
    for i, shp in enumerate(shapes):
        if len(shp) == 3:
            for e in range(shp[0]):
                w_1, m_1 = gpu_step([params[i][e]], [grads[i][e]], [moms[i][e]], **kw)
                assert np.array_equal(w_f[i][e], w_1[0]) and np.array_equal(m_f[i][e], m_1[0]), (i, e)
        else:
            w_1, m_1 = gpu_step([params[i]], [grads[i]], [moms[i]], **kw)
            assert np.array_equal(w_f[i], w_1[0]) and np.array_equal(m_f[i], m_1[0]), i


@pytest.mark.parametrize("ns", [0, 1, 2])
def test_large_round_counts(ns):
    _check([(640, 900), (900, 640)], ns=ns)


def test_large_bf16_weights_nonzero_state():
    """bf16 weights are rounded to nearest even after the update, so the check
    allows one bf16 rounding of W on top of the bf16-mode bar on lr O."""
    import oracle
    shapes = [(600, 1000), (1000, 600)]
    params, grads, moms = make_inputs(shapes, "bf16", 41, 1e-3, "bf16", 0.02, 1e-3)
    w_gpu, _ = gpu_step(params, grads, moms, mode="bf16", lr=0.02, beta=0.95, ns_steps=5, coeffs=Q)
    w_ref, _, o_ref = oracle_step(params, grads, moms, lr=0.02, beta=0.95, ns_steps=5, coeffs=Q)
    for i in range(len(shapes)):
        err = np.linalg.norm(oracle.decode(w_gpu[i]) - w_ref[i])
        bound = 2.0 ** -8 * np.linalg.norm(w_ref[i]) + 0.02 * BAR * np.linalg.norm(o_ref[i])
        print(f"bf16 W {shapes[i]}: {err:.3e} (bound {bound:.3e})", flush=True)
        assert err <= bound


def test_large_three_steps_and_mixed_plan():
    _check([(24, 3000), (96, 200), (600, 700), (700, 600)], steps=3, w_std=0.02, m_std=1e-3, lr=0.02)


def test_large_deterministic():
    shapes = [(600, 700), (2, 520, 1030)]
    params, grads, moms = make_inputs(shapes, "bf16", 12)
    a, _ = gpu_step(params, grads, moms, mode="bf16", lr=1.0, beta=0.95, ns_steps=5, coeffs=Q)
    b, _ = gpu_step(params, grads, moms, mode="bf16", lr=1.0, beta=0.95, ns_steps=5, coeffs=Q)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_large_graph_replay_matches_eager():
    import torch

    from gpu_helpers import to_device, to_host
    from muon_newton_schulz_05_amd import MuonPlan
    shapes = [(600, 700), (24, 800)]
    params, grads, moms = make_inputs(shapes, "bf16", 62, w_std=0.02)
    dev = "cuda:0"
    outs = []
    for use_graph in (False, True):
        p = [to_device(x, dev) for x in params]
        g = [to_device(x, dev) for x in grads]
        m = [to_device(x, dev) for x in moms]
        plan = MuonPlan(p, grad_dtypes=[x.dtype for x in g], mode="bf16", use_graph=use_graph)
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            for lr in (0.02, 0.01, 0.03):
                plan.step(g, m, lr=lr, beta=0.9, ns_steps=5, coeffs=Q)
                s.synchronize()
        torch.cuda.synchronize()
        outs.append([to_host(x) for x in p + m])
        plan.close()
    for x, y in zip(*outs):
        assert np.array_equal(x, y)


def test_several_large_shapes_share_the_grouped_launches():
    """Three different large oriented shapes (one of them stored transposed,
    one a 3-D stack) in one plan: every product phase is one launch over all
    of them, walking one tile table, and each slice must still match."""
    _check([(600, 700), (1100, 520), (2, 768, 1024), (24, 900)])

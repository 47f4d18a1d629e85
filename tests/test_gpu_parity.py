"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Bars: relative Frobenius error of every slice's update O <= 1e-4 in fp32 mode
and <= 2e-2 in bf16 matrix-core mode; momentum equal to the oracle's float32
value within 1 ulp (float32 FMA vs float64 then rounded); fused runs bitwise
equal to per-matrix runs; identical runs bitwise equal.
"""

from __future__ import annotations

import numpy as np
import pytest

import workloads
from gpu_helpers import (TOL, gpu_step, make_inputs, max_ulp_diff, oracle_step, slice_rel_errors,
                         to_device, to_host, update_errors)

pytestmark = pytest.mark.gpu

Q = workloads.QUINTIC


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import muon_newton_schulz_05_amd as m
    m.load_library()


def check(shapes, mode, *, grad_dtype="bf16", ns=5, lr=1.0, beta=0.95, seed=1, std=1e-3,
          w_std=0.0, m_std=0.0, param_dtype=None, steps=1, plan_kw=None, tol=None):
    params, grads, moms = make_inputs(shapes, grad_dtype, seed, std, param_dtype, w_std, m_std)
    w_gpu, m_gpu = gpu_step(params, grads, moms, mode=mode, lr=lr, beta=beta, ns_steps=ns, coeffs=Q,
                            steps=steps, plan_kw=plan_kw)
    w_ref, m_ref, o_ref = oracle_step(params, grads, moms, lr=lr, beta=beta, ns_steps=ns, coeffs=Q,
                                      steps=steps)
    tol = tol if tol is not None else TOL[mode]
    worst = 0.0
    for i in range(len(shapes)):
        if steps == 1:
            errs = update_errors(w_gpu[i], params[i], lr, o_ref[i], tol)
        else:
            errs = slice_rel_errors(w_gpu[i], w_ref[i], tol)
        worst = max(worst, max(errs))
        if steps == 1:
            assert max_ulp_diff(m_gpu[i], m_ref[i]) <= 1, f"momentum of parameter {i}"
    print(f"{shapes} {mode}: worst relative error {worst:.3e}")
    assert worst <= tol, f"{shapes} {mode}: {worst:.3e} > {tol}"
    return worst


def test_single_fp32_128x256():
    """One float32 [128,256] matrix, N(0,1) gradient, zero momentum, fp32 mode."""
    check([(128, 256)], "fp32", grad_dtype="f32", std=1.0, lr=0.02)


@pytest.mark.parametrize("ns", [0, 1, 2, 3, 4])
def test_single_fp32_128x256_after_each_round(ns):
    """The same matrix after 0 .. 4 rounds, so every round's Gram, polynomial
    and apply product meets the fp32 bar on its own (5 rounds above)."""
    check([(128, 256)], "fp32", grad_dtype="f32", std=1.0, lr=0.02, ns=ns)


@pytest.mark.parametrize("mode", ["bf16", "fp32"])
@pytest.mark.parametrize("shape", [(24, 10240), (10240, 24), (24, 1000), (7, 100), (32, 33),
                                   (1, 64), (16, 5000), (3, 24, 777), (17, 4099)])
def test_skinny_shapes(shape, mode):
    check([shape], mode)


@pytest.mark.parametrize("mode", ["bf16", "fp32"])
@pytest.mark.parametrize("shape", [(128, 256), (100, 300), (300, 100), (33, 500), (2, 200, 333),
                                   (256, 256), (600, 700)])
def test_streamed_shapes(shape, mode):
    check([shape], mode)


@pytest.mark.parametrize("shape", [(200, 333), (256, 256), (2, 150, 400), (300, 520), (513, 517),
                                   (600, 700)])
def test_bf16_streamed_products_without_large_tiles(shape):
    """With the large tiles switched off, bf16 slices with m >= 129 take the
    32-tile grouped products (m <= 256) or the 128-tile products with P as a
    hi/lo pair (m > 256), as slices longer than the large tiles can address
    always do."""
    check([shape], "bf16", plan_kw=dict(large_min_m=-1))


@pytest.mark.parametrize("mode", ["bf16", "fp32"])
def test_mixed_plan(mode):
    """Several buckets in one plan, both paths, transposed members, f32 and bf16 grads."""
    shapes = [(24, 3000), (3000, 24), (160, 96), (96, 160), (4, 24, 3000), (64, 64)]
    params, grads, moms = make_inputs(shapes, ["bf16", "f32", "bf16", "f32", "bf16", "bf16"], 5)
    w_gpu, _ = gpu_step(params, grads, moms, mode=mode, lr=1.0, beta=0.9, ns_steps=5, coeffs=Q)
    _, _, o_ref = oracle_step(params, grads, moms, lr=1.0, beta=0.9, ns_steps=5, coeffs=Q)
    for i in range(len(shapes)):
        assert max(update_errors(w_gpu[i], params[i], 1.0, o_ref[i], TOL[mode])) <= TOL[mode]


@pytest.mark.parametrize("mode", ["bf16", "fp32"])
def test_nonzero_state_and_bf16_params(mode):
    """Nonzero W and momentum exercise the read-modify-write; bf16 weights are
    rounded to nearest even, so their check allows one bf16 rounding of W."""
    check([(24, 2000), (200, 120)], mode, w_std=0.02, m_std=1e-3, lr=0.02)
    shapes = [(24, 2000), (200, 120)]
    params, grads, moms = make_inputs(shapes, "bf16", 9, param_dtypes="bf16", w_std=0.02)
    w_gpu, _ = gpu_step(params, grads, moms, mode=mode, lr=0.02, beta=0.95, ns_steps=5, coeffs=Q)
    w_ref, _, o_ref = oracle_step(params, grads, moms, lr=0.02, beta=0.95, ns_steps=5, coeffs=Q)
    import oracle
    for i in range(2):
        got = oracle.decode(w_gpu[i])
        err = np.linalg.norm(got - w_ref[i])
        bound = 2.0 ** -8 * np.linalg.norm(w_ref[i]) + 0.02 * TOL[mode] * np.linalg.norm(o_ref[i])
        assert err <= bound, (i, err, bound)


def test_tiled_products_bf16_weights():
    """float32 mode, slices on the tiled products (padded m > 256), stored
    both ways, with bf16 weights and nonzero state: the last round's
    epilogue reads and writes W in bf16 (rounded to nearest even)."""
    import oracle
    shapes = [(600, 700), (700, 600), (2, 300, 520)]
    params, grads, moms = make_inputs(shapes, "bf16", 19, param_dtypes="bf16", w_std=0.02, m_std=1e-3)
    w_gpu, _ = gpu_step(params, grads, moms, mode="fp32", lr=0.02, beta=0.95, ns_steps=5, coeffs=Q)
    w_ref, _, o_ref = oracle_step(params, grads, moms, lr=0.02, beta=0.95, ns_steps=5, coeffs=Q)
    for i in range(len(shapes)):
        err = np.linalg.norm(oracle.decode(w_gpu[i]) - w_ref[i])
        bound = 2.0 ** -8 * np.linalg.norm(w_ref[i]) + 0.02 * TOL["fp32"] * np.linalg.norm(o_ref[i])
        print(f"{shapes[i]} bf16 W fp32 mode: {err:.3e} (bound {bound:.3e})")
        assert err <= bound, (i, err, bound)


@pytest.mark.parametrize("mode", ["bf16", "fp32"])
def test_three_steps(mode):
    check([(24, 1500), (130, 260)], mode, steps=3, lr=0.02, w_std=0.02, tol=TOL[mode])


@pytest.mark.parametrize("mode", ["bf16", "fp32"])
@pytest.mark.parametrize("ns", [0, 1, 2, 7])
def test_ns_steps(ns, mode):
    check([(24, 700), (96, 300)], mode, ns=ns)


@pytest.mark.parametrize("mode", ["bf16", "fp32"])
def test_fusion_is_bitexact(mode):
    """A fused bucket gives bitwise the same W and M as one plan per matrix,
    also when skinny shapes of different m share the grouped launches."""
    shapes = [(24, 2500)] * 5 + [(96, 200)] * 3 + [(2500, 24), (32, 300), (7, 900), (16, 256)]
    params, grads, moms = make_inputs(shapes, "bf16", 21)
    w_f, m_f = gpu_step(params, grads, moms, mode=mode, lr=0.02, beta=0.95, ns_steps=5, coeffs=Q)
    for i in range(len(shapes)):
        w_1, m_1 = gpu_step([params[i]], [grads[i]], [moms[i]], mode=mode, lr=0.02, beta=0.95,
                            ns_steps=5, coeffs=Q)
        assert np.array_equal(w_f[i], w_1[0]) and np.array_equal(m_f[i], m_1[0]), f"slice {i}"


@pytest.mark.parametrize("mode", ["bf16", "fp32"])
def test_tiled_group_fusion_is_bitexact(mode):
    """Streamed buckets with padded m > 256 off the large tiles share one
    launch per product phase: here three oriented shapes (stored both ways,
    and in 3-D stacks) next to a small bucket.  The fused apply launch has
    266 tiles of 128 and takes 128-tiles; a single slice takes 64-tiles.
    Each slice must still get the bits of a plan of its own, and meet the
    bar.  (bf16 mode with the large tiles off.)"""
    shapes = [(300, 520), (520, 300), (2, 260, 700), (3, 400, 1200), (400, 1200), (1200, 400), (96, 200)]
    params, grads, moms = make_inputs(shapes, "bf16", 23, w_std=0.02, m_std=1e-3)
    kw = dict(mode=mode, lr=0.02, beta=0.95, ns_steps=5, coeffs=Q, plan_kw=dict(large_min_m=-1))
    w_f, m_f = gpu_step(params, grads, moms, **kw)
    _, _, o_ref = oracle_step(params, grads, moms, lr=0.02, beta=0.95, ns_steps=5, coeffs=Q)
    for i, shp in enumerate(shapes):
        errs = update_errors(w_f[i], params[i], 0.02, o_ref[i], TOL[mode])
        assert max(errs) <= TOL[mode], (shp, max(errs))
        if len(shp) == 3:
            for e in range(shp[0]):
                w_1, m_1 = gpu_step([params[i][e]], [grads[i][e]], [moms[i][e]], **kw)
                assert np.array_equal(w_f[i][e], w_1[0]) and np.array_equal(m_f[i][e], m_1[0]), (i, e)
        else:
            w_1, m_1 = gpu_step([params[i]], [grads[i]], [moms[i]], **kw)
            assert np.array_equal(w_f[i], w_1[0]) and np.array_equal(m_f[i], m_1[0]), i


@pytest.mark.parametrize("mode", ["bf16", "fp32"])
def test_small_product_tile_size_is_bitexact(mode):
    """Streamed buckets with padded m above 256 take 128 x 128 tiles when a
    launch has at least 256 of them, else 64 x 64 tiles; each output entry
    sums its k steps in the same order for either size, so 64 slices of
    [300,520] fused (128-wide tiles) and single slices (64-wide tiles) agree
    bit for bit.  (In bf16 mode the large tiles are switched off.)"""
    params, grads, moms = make_inputs([(64, 300, 520)], "bf16", 61, w_std=0.02, m_std=1e-3)
    kw = dict(mode=mode, lr=0.02, beta=0.95, ns_steps=5, coeffs=Q, plan_kw=dict(large_min_m=-1))
    w_f, m_f = gpu_step(params, grads, moms, **kw)
    for e in (0, 37, 63):
        w_1, m_1 = gpu_step([params[0][e]], [grads[0][e]], [moms[0][e]], **kw)
        assert np.array_equal(w_f[0][e], w_1[0]) and np.array_equal(m_f[0][e], m_1[0]), f"slice {e}"


@pytest.mark.parametrize("mode", ["bf16", "fp32"])
def test_resume_from_host_copies_is_bitexact(mode):
    """The plan holds no numeric state: one step, W and M copied to the host,
    the plan destroyed and a new one created for two more steps gives bitwise
    the W and M of three continuous steps (skinny, small streamed and large
    shapes in one plan)."""
    shapes = [(24, 3000), (96, 200), (600, 700), (2, 40, 520)]
    params, grads, moms = make_inputs(shapes, "bf16", 53, w_std=0.02, m_std=1e-3)
    kw = dict(mode=mode, lr=0.02, beta=0.95, ns_steps=5, coeffs=Q)
    w3, m3 = gpu_step(params, grads, moms, steps=3, **kw)
    w1, m1 = gpu_step(params, grads, moms, steps=1, **kw)
    w3b, m3b = gpu_step(w1, grads, m1, steps=2, **kw)
    for i in range(len(shapes)):
        assert np.array_equal(w3[i], w3b[i]) and np.array_equal(m3[i], m3b[i]), f"parameter {i}"


def test_skinny_long_rows():
    """Skinny slices of about 2M columns (8192 chunks of 256 per slice, one
    stored transposed): the polynomial kernel sums 8192 Gram partials per
    slice over many batches of loads, and the launches index tens of
    thousands of chunks.  Both modes against one oracle run."""
    shapes = [(24, (1 << 21) + 5), ((1 << 21) + 3, 20)]
    params, grads, moms = make_inputs(shapes, "bf16", 91, 1e-3, None, 0.0, 1e-3)
    w_ref, m_ref, o_ref = oracle_step(params, grads, moms, lr=1.0, beta=0.95, ns_steps=5, coeffs=Q)
    for mode in ("bf16", "fp32"):
        w_gpu, m_gpu = gpu_step(params, grads, moms, mode=mode, lr=1.0, beta=0.95, ns_steps=5, coeffs=Q)
        for i in range(len(shapes)):
            errs = update_errors(w_gpu[i], params[i], 1.0, o_ref[i], TOL[mode])
            print(f"{shapes[i]} {mode}: worst {max(errs):.3e}", flush=True)
            assert max(errs) <= TOL[mode], (shapes[i], mode, max(errs))
            assert max_ulp_diff(m_gpu[i], m_ref[i]) <= 1, (shapes[i], mode)


@pytest.mark.parametrize("mode", ["bf16", "fp32"])
def test_several_skinny_shapes_share_the_launches(mode):
    """Skinny shapes with different m and n (and ragged chunks) run in one
    launch per stage, each finding its bucket in the table."""
    check([(24, 3000), (16, 700), (7, 100), (32, 33), (3, 2, 500), (100, 8), (1, 300), (29, 257)], mode)


def test_shape_group_larger_than_one_bucket():
    """70000 slices of [8,16] fill two buckets (a launch indexes at most 65535
    slices); sampled slices of both, first and last included, match the
    oracle run on those slices alone."""
    shape = (70000, 8, 16)
    params, grads, moms = make_inputs([shape], "bf16", 77, w_std=0.02)
    w_gpu, m_gpu = gpu_step(params, grads, moms, mode="bf16", lr=0.02, beta=0.95, ns_steps=5, coeffs=Q)
    picks = [0, 1, 65534, 65535, 65536, 69999] + list(range(1000, 70000, 9973))
    sub = [a[0][picks] for a in (params, grads, moms)]
    w_ref, m_ref, o_ref = oracle_step([sub[0]], [sub[1]], [sub[2]], lr=0.02, beta=0.95, ns_steps=5, coeffs=Q)
    errs = update_errors(w_gpu[0][picks], sub[0], 0.02, o_ref[0], TOL["bf16"])
    print(f"{shape}: worst {max(errs):.3e} over {len(picks)} sampled slices", flush=True)
    assert max(errs) <= TOL["bf16"]
    assert max_ulp_diff(m_gpu[0][picks], m_ref[0]) <= 1


@pytest.mark.parametrize("mode", ["bf16", "fp32"])
def test_3d_equals_2d_slices(mode):
    shapes3 = [(3, 24, 900), (2, 80, 150)]
    params, grads, moms = make_inputs(shapes3, "bf16", 31)
    w3, m3 = gpu_step(params, grads, moms, mode=mode, lr=0.02, beta=0.95, ns_steps=5, coeffs=Q)
    p2 = [p[e] for p in params for e in range(p.shape[0])]
    g2 = [g[e] for g in grads for e in range(g.shape[0])]
    mm2 = [m[e] for m in moms for e in range(m.shape[0])]
    w2, m2 = gpu_step(p2, g2, mm2, mode=mode, lr=0.02, beta=0.95, ns_steps=5, coeffs=Q)
    k = 0
    for i, p in enumerate(params):
        for e in range(p.shape[0]):
            assert np.array_equal(w3[i][e], w2[k]) and np.array_equal(m3[i][e], m2[k])
            k += 1


@pytest.mark.parametrize("mode", ["bf16", "fp32"])
@pytest.mark.parametrize("shape", [(24, 1800), (96, 230), (600, 700)])
def test_transposed_input_gives_transposed_output(shape, mode):
    params, grads, moms = make_inputs([shape], "bf16", 41)
    w_a, _ = gpu_step(params, grads, moms, mode=mode, lr=0.02, beta=0.95, ns_steps=5, coeffs=Q)
    gt = [np.ascontiguousarray(grads[0].T)]
    w_b, _ = gpu_step([np.ascontiguousarray(params[0].T)], gt, [np.ascontiguousarray(moms[0].T)],
                      mode=mode, lr=0.02, beta=0.95, ns_steps=5, coeffs=Q)
    assert np.array_equal(w_a[0].T, w_b[0])


@pytest.mark.parametrize("mode", ["bf16", "fp32"])
def test_deterministic(mode):
    shapes = [(24, 4000), (256, 384)]
    params, grads, moms = make_inputs(shapes, "bf16", 51, w_std=0.02, m_std=1e-3)
    a = gpu_step(params, grads, moms, mode=mode, lr=0.02, beta=0.95, ns_steps=5, coeffs=Q, steps=2)
    b = gpu_step(params, grads, moms, mode=mode, lr=0.02, beta=0.95, ns_steps=5, coeffs=Q, steps=2)
    for x, y in zip(a[0] + a[1], b[0] + b[1]):
        assert np.array_equal(x, y)


def test_fused_74x24x10240_bf16():
    """The pages' fusion example: 74 parameters of [24, 10240], bf16 grads."""
    wl = workloads.WORKLOADS["fused_74x24x10240"]
    grads = [workloads.gradient(wl, i) for i in range(len(wl.params))]
    shapes = [p.shape for p in wl.params]
    params = [np.zeros(s, np.float32) for s in shapes]
    moms = [np.zeros(s, np.float32) for s in shapes]
    w_gpu, m_gpu = gpu_step(params, grads, moms, mode="bf16", lr=wl.lr, beta=wl.beta,
                            ns_steps=wl.ns_steps, coeffs=wl.coeffs)
    _, m_ref, o_ref = oracle_step(params, grads, moms, lr=wl.lr, beta=wl.beta, ns_steps=wl.ns_steps,
                                  coeffs=wl.coeffs)
    worst = max(max(update_errors(w_gpu[i], params[i], wl.lr, o_ref[i], TOL["bf16"])) for i in range(len(shapes)))
    print(f"74x[24,10240] bf16: worst {worst:.3e}")
    assert worst <= TOL["bf16"]
    for i in range(len(shapes)):
        assert max_ulp_diff(m_gpu[i], m_ref[i]) <= 1


def test_fused_74x24x10240_fp32():
    wl = workloads.WORKLOADS["fused_74x24x10240"]
    grads = [workloads.gradient(wl, i) for i in range(len(wl.params))]
    shapes = [p.shape for p in wl.params]
    params = [np.zeros(s, np.float32) for s in shapes]
    moms = [np.zeros(s, np.float32) for s in shapes]
    w_gpu, _ = gpu_step(params, grads, moms, mode="fp32", lr=1.0, beta=wl.beta, ns_steps=5,
                        coeffs=wl.coeffs)
    _, _, o_ref = oracle_step(params, grads, moms, lr=1.0, beta=wl.beta, ns_steps=5, coeffs=wl.coeffs)
    worst = max(max(update_errors(w_gpu[i], params[i], 1.0, o_ref[i], TOL["fp32"])) for i in range(len(shapes)))
    print(f"74x[24,10240] fp32: worst {worst:.3e}")
    assert worst <= TOL["fp32"]


def test_graph_replay_matches_eager():
    import torch

    from muon_newton_schulz_05_amd import MuonPlan
    shapes = [(96, 300), (300, 96), (24, 800)]
    params, grads, moms = make_inputs(shapes, "bf16", 61, w_std=0.02)
    dev = "cuda:0"
    outs = []
    for use_graph in (False, True):
        p = [to_device(x, dev) for x in params]
        g = [to_device(x, dev) for x in grads]
        m = [to_device(x, dev) for x in moms]
        plan = MuonPlan(p, grad_dtypes=[x.dtype for x in g], mode="bf16", use_graph=use_graph)
        s = torch.cuda.Stream()
        # lr, beta and the coefficients change between replays and must take effect.
        cubic = (1.5, -0.5, 0.0)
        with torch.cuda.stream(s):
            for lr, beta, co in [(0.02, 0.9, Q), (0.01, 0.95, Q), (0.03, 0.9, cubic), (0.03, 0.8, Q)]:
                plan.step(g, m, lr=lr, beta=beta, ns_steps=5, coeffs=co)
                s.synchronize()  # eager host work between replays
        torch.cuda.synchronize()
        outs.append([to_host(x) for x in p + m])
        plan.close()
    for x, y in zip(*outs):
        assert np.array_equal(x, y)


def test_steps_on_two_streams_are_ordered():
    """A step enqueued on another stream than the plan's previous step waits
    for it (both use the plan's workspace): three steps alternating between
    two streams, with no host synchronisation in between, give bitwise the W
    and M of three steps on one stream (skinny, small and large buckets)."""
    import torch

    from muon_newton_schulz_05_amd import MuonPlan
    shapes = [(24, 3000), (96, 300), (600, 700)]
    params, grads, moms = make_inputs(shapes, "bf16", 141, w_std=0.02, m_std=1e-3)
    outs = []
    for alternate in (False, True):
        p = [to_device(x, "cuda:0") for x in params]
        g = [to_device(x, "cuda:0") for x in grads]
        m = [to_device(x, "cuda:0") for x in moms]
        torch.cuda.synchronize()
        plan = MuonPlan(p, grad_dtypes=[x.dtype for x in g], mode="bf16")
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        for i in range(3):
            st = (s2 if i % 2 else s1) if alternate else s1
            plan.step(g, m, lr=0.02, beta=0.95, ns_steps=5, coeffs=Q, stream=st)
        plan.status()  # waits for the plan's last step
        outs.append([to_host(x) for x in p + m])
        plan.close()
    for x, y in zip(*outs):
        assert np.array_equal(x, y)


def test_step_rejects_bad_arguments_without_side_effects():
    import torch

    from muon_newton_schulz_05_amd import MuonError, MuonPlan, muon_step
    p = [torch.zeros(24, 100, device="cuda:0")]
    g = [torch.ones(24, 100, device="cuda:0")]
    m = [torch.zeros(24, 100, device="cuda:0")]
    plan = MuonPlan(p, mode="bf16")
    s = torch.cuda.current_stream().cuda_stream
    for bad in [dict(lr=float("nan")), dict(beta=float("inf")), dict(ns_steps=17), dict(ns_steps=-1)]:
        kw = dict(lr=0.02, beta=0.9, ns_steps=5)
        kw.update(bad)
        with pytest.raises(MuonError) as ei:
            muon_step(plan.handle, [p[0].data_ptr()], [g[0].data_ptr()], [m[0].data_ptr()],
                      kw["lr"], kw["beta"], kw["ns_steps"], *Q, s)
        assert ei.value.code == 1
    with pytest.raises(MuonError):
        muon_step(plan.handle, [0], [g[0].data_ptr()], [m[0].data_ptr()], 0.02, 0.9, 5, *Q, s)
    with pytest.raises(MuonError):
        muon_step(plan.handle, [p[0].data_ptr() + 4], [g[0].data_ptr()], [m[0].data_ptr()], 0.02, 0.9, 5,
                  *Q, s)
    torch.cuda.synchronize()
    assert not p[0].any() and not m[0].any()
    plan.close()


def _conditioned(shape, kind, seed):
    """Float32 gradients with controlled singular values (stored as given)."""
    rng = np.random.default_rng(seed)
    r, c = shape
    m = min(r, c)
    u, _ = np.linalg.qr(rng.standard_normal((r, m)))
    v, _ = np.linalg.qr(rng.standard_normal((c, m)))
    if kind == "logspaced":
        s = np.logspace(0, -4, m)
        g = (u * s) @ v.T
    else:  # rank one plus noise
        g = np.outer(rng.standard_normal(r), rng.standard_normal(c)) + 1e-4 * rng.standard_normal((r, c))
    return (g * 1e-2).astype(np.float32)


@pytest.mark.parametrize("mode", ["bf16", "fp32"])
@pytest.mark.parametrize("kind", ["logspaced", "rank1_noise"])
@pytest.mark.parametrize("shape", [(24, 3000), (3000, 24), (32, 700)])
def test_skinny_ill_conditioned(shape, kind, mode):
    """The Gram-space rounds keep float32 X0 (split hi/lo on the matrix cores
    in bf16 mode), so singular values spread over four decades still meet
    the bar."""
    g = _conditioned(shape, kind, 71)
    params, moms = [np.zeros(shape, np.float32)], [np.zeros(shape, np.float32)]
    w_gpu, _ = gpu_step(params, [g], moms, mode=mode, lr=1.0, beta=0.9, ns_steps=5, coeffs=Q)
    _, _, o_ref = oracle_step(params, [g], moms, lr=1.0, beta=0.9, ns_steps=5, coeffs=Q)
    err = max(update_errors(w_gpu[0], params[0], 1.0, o_ref[0], TOL[mode]))
    print(f"{shape} {kind} {mode}: {err:.3e}")
    assert err <= TOL[mode]


@pytest.mark.parametrize("kind", ["logspaced", "rank1_noise"])
def test_streamed_ill_conditioned_fp32(kind):
    shape = (96, 700)
    g = _conditioned(shape, kind, 72)
    params, moms = [np.zeros(shape, np.float32)], [np.zeros(shape, np.float32)]
    w_gpu, _ = gpu_step(params, [g], moms, mode="fp32", lr=1.0, beta=0.9, ns_steps=5, coeffs=Q)
    _, _, o_ref = oracle_step(params, [g], moms, lr=1.0, beta=0.9, ns_steps=5, coeffs=Q)
    err = max(update_errors(w_gpu[0], params[0], 1.0, o_ref[0], TOL["fp32"]))
    print(f"{shape} {kind} fp32: {err:.3e}")
    assert err <= TOL["fp32"]


@pytest.mark.parametrize("kind", ["logspaced", "rank1_noise"])
@pytest.mark.parametrize("shape,plan_kw", [((96, 700), None), ((200, 333), None), ((600, 700), None),
                                           ((300, 520), dict(large_min_m=-1))],
                         ids=["small", "large-mid", "large", "streamed-hilo"])
def test_bf16_ill_conditioned_resolved_directions(shape, plan_kw, kind):
    """bf16 mode stores X in bf16, whose 8-bit significand cannot hold a
    singular direction far below the largest one; the polynomial then
    amplifies what is left of it (by up to a^k), so over the whole matrix
    these inputs miss the bf16 bar (logspaced 4-10%, rank one plus noise
    about 117%, alike on every streamed path).  The directions that bf16
    resolves must still be right: O restricted to the singular vectors of G
    with sigma / sigma_1 > 2^-8 meets the bar."""
    g = _conditioned(shape, kind, 72)
    params, moms = [np.zeros(shape, np.float32)], [np.zeros(shape, np.float32)]
    w_gpu, _ = gpu_step(params, [g], moms, mode="bf16", lr=1.0, beta=0.9, ns_steps=5, coeffs=Q,
                        plan_kw=plan_kw)
    _, _, o_ref = oracle_step(params, [g], moms, lr=1.0, beta=0.9, ns_steps=5, coeffs=Q)
    o_gpu = -w_gpu[0].astype(np.float64)   # W0 = 0 and lr = 1
    u, s, vt = np.linalg.svd(g.astype(np.float64), full_matrices=False)
    k = int((s / s[0] > 2.0 ** -8).sum())
    a = u[:, :k].T @ o_gpu @ vt[:k].T
    b = u[:, :k].T @ o_ref[0] @ vt[:k].T
    err = float(np.linalg.norm(a - b) / np.linalg.norm(b))
    whole = float(np.linalg.norm(o_gpu - o_ref[0]) / np.linalg.norm(o_ref[0]))
    print(f"{shape} {kind} bf16: resolved ({k} directions) {err:.3e}, whole {whole:.3e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("mode", ["bf16", "fp32"])
def test_zero_gradient_slices(mode):
    """A zero momentum and gradient slice inside fused buckets (skinny,
    128-tile streamed and, in bf16 mode, the large products): eps keeps the
    normaliser finite, O = 0, so W stays bitwise unchanged; the neighbouring
    slices still match the oracle and the device error word stays clear."""
    shapes = [(3, 24, 900), (3, 96, 200), (3, 600, 700)]
    params, grads, moms = make_inputs(shapes, "bf16", 91, w_std=0.02)
    for g in grads:
        g[1] = 0
    w_gpu, m_gpu = gpu_step(params, grads, moms, mode=mode, lr=0.02, beta=0.95, ns_steps=5, coeffs=Q)
    _, _, o_ref = oracle_step(params, grads, moms, lr=0.02, beta=0.95, ns_steps=5, coeffs=Q)
    for i in range(len(shapes)):
        assert np.all(np.isfinite(w_gpu[i])), i
        assert np.array_equal(w_gpu[i][1], params[i][1]), f"parameter {i}: zero slice changed W"
        assert not m_gpu[i][1].any()
        assert not o_ref[i][1].any()
        for e in (0, 2):
            errs = update_errors(w_gpu[i][e], params[i][e], 0.02, o_ref[i][e], TOL[mode])
            assert max(errs) <= TOL[mode], (i, e, errs)


@pytest.mark.parametrize("shape,mode", [((96, 160), "fp32"), ((96, 160), "bf16"), ((600, 700), "bf16"),
                                        ((700, 600), "bf16"), ((600, 700), "fp32")])
def test_nonfinite_gradient_streamed_paths(shape, mode):
    """An infinite gradient entry in a slice of the streamed paths (the
    32-tile products, the tiled products of float32 mode and the large
    products of bf16 mode) sets bit 0 of the device error word, like the
    skinny path."""
    import torch

    from muon_newton_schulz_05_amd import MuonPlan
    p = [torch.zeros(shape, device="cuda:0"), torch.zeros(24, 300, device="cuda:0")]
    g = [torch.ones(shape, device="cuda:0"), torch.ones(24, 300, device="cuda:0")]
    g[0][5, 9] = float("inf")
    m = [torch.zeros_like(x) for x in p]
    plan = MuonPlan(p, mode=mode)
    plan.step(g, m, lr=0.02, beta=0.9, ns_steps=5)
    torch.cuda.synchronize()
    assert plan.status() & 1
    assert plan.status() == 0  # reading clears the word
    assert bool(torch.isfinite(p[1]).all())  # the other parameter is unaffected
    plan.close()


def test_step_checks_grad_dtype_and_device_before_launch():
    """The binding refuses gradients of another storage type than the plan
    was made for, and tensors on another device, before calling muon_step."""
    import torch

    from muon_newton_schulz_05_amd import MuonPlan
    p = [torch.zeros(24, 100, device="cuda:0")]
    m = [torch.zeros(24, 100, device="cuda:0")]
    plan = MuonPlan(p, grad_dtypes=[torch.bfloat16], mode="bf16")
    with pytest.raises(TypeError):
        plan.step([torch.ones(24, 100, device="cuda:0")], m)
    with pytest.raises(ValueError):
        plan.step([torch.ones(24, 100, dtype=torch.bfloat16)], m)
    with pytest.raises(ValueError):
        plan.step([torch.ones(24, 100, dtype=torch.bfloat16, device="cuda:0")], [torch.zeros(24, 100)])
    torch.cuda.synchronize()
    assert not p[0].any() and not m[0].any()
    plan.close()


def test_nonfinite_gradient_sets_device_error():
    import torch

    from muon_newton_schulz_05_amd import MuonPlan
    p = [torch.zeros(24, 600, device="cuda:0")]
    g = [torch.ones(24, 600, device="cuda:0")]
    g[0][3, 7] = float("inf")
    m = [torch.zeros(24, 600, device="cuda:0")]
    plan = MuonPlan(p, mode="bf16")
    plan.step(g, m, lr=0.02, beta=0.9, ns_steps=5)
    torch.cuda.synchronize()
    assert plan.status() & 1
    assert plan.status() == 0  # reading clears the word
    plan.close()

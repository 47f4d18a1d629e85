"""Parity at full workload sizes, in the launch configuration the benchmark
times (one fused plan over every parameter of the workload, eager), in bf16
mode and in fp32 mode.

The float64 oracle cannot run whole workloads in a test, so one slice of every
large oriented shape was run through it by tests/golden/make_golden.py; the
file holds 1024 sampled entries of that slice's O plus ||O||_F.  Here the
sampled parameter's gradient is the same seeded bf16 tensor, all other
parameters get device-generated Gaussian gradients, momentum and weights
start at zero and lr = 1, so the new weights are exactly -O.

Checked per case:
  * the sampled entries: ||O_gpu[s] - O_ref[s]|| / ||O_ref[s]|| <= 2e-2
    in bf16 mode, 1e-4 in fp32 mode;
  * ||O_gpu||_F of the sampled slice against the stored norm, same bar;
  * every other slice of the same oriented shape is finite and has a
    Frobenius norm within 5% of the sampled slice's (Gaussian matrices of one
    shape have near-identical singular-value spectra, so the Newton-Schulz
    output norm concentrates tightly).

The LAST slice of every large bucket also gets its seeded gradient, and its
contiguous bottom-right output tile (256 x 256, or the ragged remainder) is
compared entry by entry with the stored oracle tile
(tests/golden/large_last_tiles.*): relative error of the tile within the
bar, and every 64 x 64 block of it within 3 times its share of the slice's
allowed error (the block-local check of gpu_helpers).  The 32 skinny
[24,10240] expert slices of the MoE workload are compared whole against the
oracle, run here.
"""

from __future__ import annotations

import json
import os

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import TOL, block_ratios, to_device, to_host, update_errors

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "large_slices.json")
TILES = os.path.join(HERE, "golden", "large_last_tiles.json")
TILE_VALUES = os.path.join(HERE, "golden", "large_last_tiles.npz")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _tile_cases():
    with open(TILES) as f:
        return json.load(f)["cases"]


def _oriented(shape):
    r, c = shape[-2:]
    return (min(r, c), max(r, c))


@pytest.mark.gpu
@pytest.mark.parametrize("mode", ["bf16", "fp32"])
@pytest.mark.parametrize("workload", ["moe_experts", "dense_h4096_l8", "large_share"])
def test_full_workload_sampled(workload, mode):
    import torch

    from muon_newton_schulz_05_amd import MuonPlan

    cases = [c for c in _cases() if c["workload"] == workload]
    tiles = [c for c in _tile_cases() if c["workload"] == workload]
    assert cases and tiles
    wl = workloads.WORKLOADS[workload]
    dev = torch.device("cuda:0")
    print(f"full-size parity: {workload} ({mode} mode)", flush=True)

    skinny_params = [i for i, spec in enumerate(wl.params) if min(spec.shape[-2:]) <= 32]
    golden_params = {c["param"] for c in cases} | {c["param"] for c in tiles} | set(skinny_params)
    gen = torch.Generator(device=dev)
    grads, params, moms = [], [], []
    for i, spec in enumerate(wl.params):
        if i in golden_params:
            g = to_device(workloads.gradient(wl, i), dev)
        else:
            gen.manual_seed(77 + i)
            g = (torch.randn(spec.shape, generator=gen, device=dev) * wl.grad_std).to(torch.bfloat16)
        grads.append(g)
        params.append(torch.zeros(spec.shape, dtype=torch.float32, device=dev))
        moms.append(torch.zeros(spec.shape, dtype=torch.float32, device=dev))
    plan = MuonPlan(params, grad_dtypes=[g.dtype for g in grads], mode=mode)
    plan.step(grads, moms, lr=1.0, beta=wl.beta, ns_steps=wl.ns_steps, coeffs=wl.coeffs)
    torch.cuda.synchronize()
    assert plan.status() == 0, "device error word set"
    plan.close()
    del grads, moms

    def slice_of(t, s):
        return t[s] if t.dim() == 3 else t

    tol = TOL[mode]
    values = np.load(TILE_VALUES)
    for c in tiles:
        o_gpu = -slice_of(params[c["param"]], c["slice"])
        assert list(o_gpu.shape) == c["shape"]
        got = o_gpu[c["row0"]:, c["col0"]:].double().cpu().numpy()
        ref = values[c["array"]].astype(np.float64)
        assert got.shape == ref.shape
        err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        worst_block = float(block_ratios(got - ref, c["frobenius"], tol, full_shape=c["shape"]).max())
        print(f"  {workload} param {c['param']} slice {c['slice']} {c['shape']}: last tile "
              f"[{c['row0']}:, {c['col0']}:] rel err {err:.3e}, worst block {worst_block:.3f} of its bound",
              flush=True)
        assert err <= tol, (c["shape"], err)
        assert worst_block <= 1.0, (c["shape"], worst_block)

    for i in skinny_params:
        g = workloads.gradient(wl, i)
        zeros = np.zeros(wl.params[i].shape, np.float32)
        _, _, o_ref = oracle.muon_step([zeros], [g], [zeros], lr=1.0, beta=wl.beta, ns_steps=wl.ns_steps,
                                       a=wl.coeffs[0], b=wl.coeffs[1], c=wl.coeffs[2])
        errs = update_errors(to_host(params[i]), zeros, 1.0, o_ref[0], tol)
        print(f"  {workload} param {i} {wl.params[i].shape}: whole, worst slice {max(errs):.3e}", flush=True)
        assert max(errs) <= tol
    for c in cases:
        o_gpu = -slice_of(params[c["param"]], c["slice"])
        assert list(o_gpu.shape) == c["shape"]
        idx = torch.tensor(c["index"], dtype=torch.int64, device=dev)
        got = o_gpu.reshape(-1)[idx].double().cpu().numpy()
        ref = np.asarray(c["value"], np.float64)
        err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        fro = float(torch.linalg.vector_norm(o_gpu.double()))
        fro_err = abs(fro - c["frobenius"]) / c["frobenius"]
        print(f"  {workload} param {c['param']} slice {c['slice']} {c['shape']}: "
              f"sampled rel err {err:.3e}, ||O|| {fro:.6f} vs {c['frobenius']:.6f}", flush=True)
        assert err <= tol, (c["shape"], err)
        assert fro_err <= tol, (c["shape"], fro, c["frobenius"])

        key = _oriented(c["shape"])
        for i, spec in enumerate(wl.params):
            if _oriented(spec.shape) != key:
                continue
            t = params[i] if len(spec.shape) == 3 else params[i][None]
            norms = torch.linalg.vector_norm(t.double(), dim=(-2, -1))
            assert bool(torch.isfinite(t).all()), (i, spec.shape)
            rel = (norms - fro).abs() / fro
            assert float(rel.max()) <= 0.05, (i, spec.shape, float(rel.max()))

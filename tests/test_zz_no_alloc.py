"""muon_step_noalloc (the entry point that allocates nothing: the step runs in
the library's fixed device scratch array) against muon_step on a plan.

Both run the same kernels on the same arithmetic, so W and M must agree bit
for bit, which is within every parity bar.  Two calls in a row, the second
with a smaller input, show that the scratch left by one call does not leak
into the next (the streamed path relies on zero padding in its workspace)."""

from __future__ import annotations

import numpy as np
import pytest

import workloads
from gpu_helpers import make_inputs, to_device, to_host

pytestmark = pytest.mark.gpu

Q = workloads.QUINTIC


def _plan_step(params, grads, moms, mode, ns=5, lr=0.02, beta=0.95):
    import torch

    from muon_newton_schulz_05_amd import MuonPlan
    p = [to_device(x, "cuda:0") for x in params]
    g = [to_device(x, "cuda:0") for x in grads]
    m = [to_device(x, "cuda:0") for x in moms]
    plan = MuonPlan(p, grad_dtypes=[x.dtype for x in g], mode=mode)
    plan.step(g, m, lr=lr, beta=beta, ns_steps=ns, coeffs=Q)
    torch.cuda.synchronize()
    assert plan.status() == 0
    plan.close()
    return [to_host(x) for x in p], [to_host(x) for x in m]


def _noalloc_step(params, grads, moms, mode, ns=5, lr=0.02, beta=0.95, err=None):
    import torch

    from muon_newton_schulz_05_amd import binding as b
    p = [to_device(x, "cuda:0") for x in params]
    g = [to_device(x, "cuda:0") for x in grads]
    m = [to_device(x, "cuda:0") for x in moms]
    descs = b.make_descs([tuple(x.shape) for x in p],
                         [b.MUON_BF16 if x.dtype == torch.bfloat16 else b.MUON_F32 for x in p],
                         [b.MUON_BF16 if x.dtype == torch.bfloat16 else b.MUON_F32 for x in g])
    opts = b.make_opts(mode=mode)
    s = torch.cuda.current_stream().cuda_stream
    b.muon_step_noalloc(descs, opts, [x.data_ptr() for x in p], [x.data_ptr() for x in g],
                        [x.data_ptr() for x in m], lr, beta, ns, *Q, err.data_ptr() if err is not None else 0, s)
    torch.cuda.synchronize()
    return [to_host(x) for x in p], [to_host(x) for x in m]


def _same(a, b):
    for i, (x, y) in enumerate(zip(a[0] + a[1], b[0] + b[1])):
        assert x.dtype == y.dtype and np.array_equal(x, y), f"tensor {i}"


@pytest.mark.parametrize("mode", ["bf16", "fp32"])
def test_noalloc_matches_plan_step_twice(mode):
    # First call: skinny, 128-tile streamed and (bf16 mode) large-tile buckets,
    # a 3-D stack and a transposed slice; nonzero W and M.
    big = [(3, 24, 900), (1000, 24), (2, 96, 200), (300, 130), (600, 700), (700, 600)]
    params, grads, moms = make_inputs(big, "bf16", 131, w_std=0.02, m_std=1e-3)
    print(f"noalloc {mode}: first call {big}", flush=True)
    _same(_noalloc_step(params, grads, moms, mode), _plan_step(params, grads, moms, mode))
    # Second call, smaller input on the same scratch (what the first left
    # behind must not matter).
    small = [(24, 300), (100, 130)]
    params, grads, moms = make_inputs(small, "bf16", 137, w_std=0.02)
    print(f"noalloc {mode}: second call {small}", flush=True)
    _same(_noalloc_step(params, grads, moms, mode, ns=3), _plan_step(params, grads, moms, mode, ns=3))


def test_noalloc_reports_nonfinite_into_the_callers_word():
    import torch
    params, grads, moms = make_inputs([(24, 500), (600, 700)], "f32", 139)
    grads[1][3, 4] = np.inf
    err = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    _noalloc_step(params, grads, moms, "bf16", err=err)
    assert int(err.item()) & 1
    err.zero_()
    _noalloc_step(params[:1], grads[:1], moms[:1], "bf16", err=err)
    assert int(err.item()) == 0


def test_noalloc_refuses_steps_larger_than_the_scratch():
    import torch

    from muon_newton_schulz_05_amd import MuonError
    from muon_newton_schulz_05_amd import binding as b
    descs = b.make_descs([(4096, 4096)], [b.MUON_F32], [b.MUON_BF16])
    t = torch.zeros(16, device="cuda:0")
    with pytest.raises(MuonError) as ei:
        b.muon_step_noalloc(descs, b.make_opts(mode="bf16"), [t.data_ptr()], [t.data_ptr()], [t.data_ptr()],
                            0.02, 0.95, 5, *Q, 0, torch.cuda.current_stream().cuda_stream)
    assert ei.value.code == b.MUON_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert not t.any()

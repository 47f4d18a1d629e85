"""Benchmark of the fused Muon step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--mode bf16|fp32]

Prints ONE JSON line.  A step is one full Muon update of every parameter of
the workload (momentum, normalisation, k Newton-Schulz rounds, weight update)
with inputs already resident in HBM.  The headline workload (default: the
h = 4096 transformer, 8 layers, the largest single-GPU configuration) gives
``value``, matrices (2-D slices) per second; the line also carries the
effective TFLOP/s twice (the dense count of the method and the flops this
library actually computes), graph-replay timing, the roofline of the dominant
kernel (timed with HIP events on the launch stream), the other large and the
skinny workloads as extra keys, and the CPU oracle's throughput on a bounded
sample of the headline workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}
DEFAULT_WORKLOAD = "dense_h4096_l8"
# Measured after the headline workload and reported as extra keys: the
# large-matrix share and the fused skinny batch.
EXTRA_WORKLOADS = ("large_share", "fused_74x24x10240")


def elem_bytes(dt: str) -> int:
    return 2 if dt == "bf16" else 4


def compulsory_bytes(wl: workloads.Workload) -> float:
    """Bytes a step must move: read G, read+write M (f32), read+write W."""
    tot = 0.0
    for p in wl.params:
        e = 1
        for d in p.shape:
            e *= d
        tot += e * (elem_bytes(p.grad_dtype) + 8 + 2 * elem_bytes(p.param_dtype))
    return tot


def stream_model(wl: workloads.Workload, mode: str):
    """The streaming cost model of a step: B_stream, the bytes a design moves
    when X leaves the chip between the Gram and the apply of every round,
    m n (s_G + 8 + 2 s_W + (3k + 2) s_X) + k m^2 (8 + 2 s_X) per oriented
    slice; and T_roof, the sum over same-shape buckets of
    max(F / matrix-core peak, B_stream / 8 TB/s), F = k (4 m^2 n + 2 m^3).
    The skinny path's Gram-space rounds skip the per-round X passes, so
    B_stream / t can exceed the HBM peak there."""
    k = wl.ns_steps
    s_x = 2 if mode == "bf16" else 4
    buckets = {}
    for p in wl.params:
        r, c = p.shape[-2:]
        e = p.shape[0] if len(p.shape) == 3 else 1
        m, n = min(r, c), max(r, c)
        b = m * n * (elem_bytes(p.grad_dtype) + 8 + 2 * elem_bytes(p.param_dtype) + (3 * k + 2) * s_x) \
            + k * m * m * (8 + 2 * s_x)
        f = k * (4.0 * m * m * n + 2.0 * m ** 3)
        key = (m, n, p.grad_dtype, p.param_dtype)
        fb = buckets.setdefault(key, [0.0, 0.0])
        fb[0] += e * f
        fb[1] += e * b
    b_stream = sum(v[1] for v in buckets.values())
    t_roof = sum(max(f / (MFMA_PEAK_TFLOPS[mode] * 1e12), b / (HBM_PEAK_GBS * 1e9)) for f, b in buckets.values())
    return b_stream, t_roof


def make_gpu_inputs(wl: workloads.Workload, dev):
    """Seeded synthetic inputs generated on the device (same recipe as the
    host generator: Gaussian gradients of the workload's std, stored in the
    workload's types; momentum from a prior step; weights N(0, 0.02^2))."""
    import torch
    gen = torch.Generator(device=dev)
    params, grads, moms = [], [], []
    for i, p in enumerate(wl.params):
        gen.manual_seed(workloads.seed(wl, i))
        g = torch.randn(p.shape, generator=gen, device=dev, dtype=torch.float32) * wl.grad_std
        grads.append(g.to(torch.bfloat16) if p.grad_dtype == "bf16" else g)
        m = torch.randn(p.shape, generator=gen, device=dev, dtype=torch.float32) * wl.grad_std
        moms.append(m)
        w = torch.randn(p.shape, generator=gen, device=dev, dtype=torch.float32) * 0.02
        params.append(w.to(torch.bfloat16) if p.param_dtype == "bf16" else w)
    return params, grads, moms


KERNEL_SOURCES = {
    "k_skinny_gram": ("skinny.hip", "device_common.h", "kernels.h", "layout.h"),
    "k_skinny_apply": ("skinny.hip", "device_common.h", "kernels.h", "layout.h"),
    # apply and final launches of the large-tile products (the "apply" timing class);
    # the planner's tile order decides their operand reuse in the L2
    "apply": ("stream_big.hip", "device_common.h", "kernels.h", "layout.h", "planner.cpp"),
}


def source_hash(files) -> str:
    """sha256 of the `sha256sum` listing of a kernel's source files (the form
    recorded beside the counter figures in profiles/)."""
    import hashlib
    csrc = os.path.join(ROOT, "muon_newton_schulz_05_amd", "csrc")
    lines = []
    for f in files:
        with open(os.path.join(csrc, f), "rb") as fh:
            lines.append(f"{hashlib.sha256(fh.read()).hexdigest()}  muon_newton_schulz_05_amd/csrc/{f}\n")
    return hashlib.sha256("".join(lines).encode()).hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the rocprofv3 FETCH_SIZE/WRITE_SIZE summaries
    under profiles/, or None when none was taken on the current source."""
    files = KERNEL_SOURCES.get(kernel)
    pdir = os.path.join(ROOT, "profiles")
    if not files or not os.path.isdir(pdir):
        return None
    want = source_hash(files)
    for name in sorted(os.listdir(pdir)):
        with open(os.path.join(pdir, name)) as fh:
            for line in fh:
                f = line.split()
                if len(f) == 5 and f[0] == "traffic" and f[1] == kernel and f[2] == workload and f[3] == want:
                    return float(f[4])
    return None


def big_apply_bytes(wl: workloads.Workload) -> float:
    """Compulsory HBM bytes per launch of the large-tile apply class (k - 1
    apply launches and one final launch per step), over the slices with
    m >= 129 in their padded workspace layout (multiples of 256): an apply
    reads R (2 mp^2) and X^T and writes X' and X'^T (2 mp np each; the X term
    comes from the X^T operand already on chip); the final launch reads R and
    X^T and reads and writes W (float32, 8 m n)."""
    k = wl.ns_steps
    apply = final = 0.0
    for m, n in wl.oriented_matrices():
        if path_of(m, "bf16") != "large":
            continue
        mp, np_ = -(-m // 256) * 256, -(-n // 256) * 256
        apply += 2 * mp * mp + 6 * mp * np_
        final += 2 * mp * mp + 2 * mp * np_ + 8 * m * n
    return ((k - 1) * apply + final) / k if k > 0 else 0.0


def measure_ceilings(dev, copy_mib: int = 1024, reps: int = 20, gemm: bool = True):
    """Measured ceilings on this GPU: a plain device-to-device copy (torch's
    copy kernel, read + write bytes counted) and a library bf16 GEMM
    (torch.matmul, 8192^3, hipBLASLt)."""
    import torch
    n = copy_mib * (1 << 20) // 4
    src = torch.empty(n, dtype=torch.float32, device=dev).uniform_()
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2.0 * n * 4 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    out = {"copy_gbs": round(copy_gbs, 1), "copy_bytes_per_launch": 2 * n * 4}
    if not gemm:
        return out
    k = 8192
    a = torch.randn(k, k, device=dev, dtype=torch.bfloat16)
    b = torch.randn(k, k, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        c = a @ b
    e0.record()
    for _ in range(10):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    gemm_tf = 2.0 * k ** 3 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b, c
    out.update(library_bf16_gemm_tflops=round(gemm_tf, 1), library_gemm_shape=[k, k, k])
    return out


def cpu_baseline(wl: workloads.Workload, budget_s: float, budget32_s: float):
    """The oracle, as it stands, timed on the host on a bounded sample of the
    workload: whole parameters in workload order until the budget is spent,
    in float64 (the oracle's own arithmetic), then the same steps in float32
    storage (the GPU path's precision class) on a second budget."""
    import numpy as np

    import oracle
    cores = len(os.sched_getaffinity(0))
    try:
        blas = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas_name = f"{blas.get('name', '?')} {blas.get('version', '')}".strip()
    except Exception:
        blas_name = "unknown"

    def run(budget, dtype):
        mats, t_total, idx, reps = 0, 0.0, 0, 0
        while t_total < budget:
            i = idx % len(wl.params)
            spec = wl.params[i]
            g = workloads.gradient(wl, i)
            w = np.zeros(spec.shape, np.float32)
            m = np.zeros(spec.shape, np.float32)
            t0 = time.perf_counter()
            oracle.muon_step([w], [g], [m], lr=wl.lr, beta=wl.beta, ns_steps=wl.ns_steps,
                             a=wl.coeffs[0], b=wl.coeffs[1], c=wl.coeffs[2], dtype=dtype)
            t_total += time.perf_counter() - t0
            mats += spec.shape[0] if len(spec.shape) == 3 else 1
            idx += 1
            if idx % len(wl.params) == 0:
                reps += 1
        desc = (f"{reps} full pass(es) + {idx % len(wl.params)} of {len(wl.params)} parameters"
                if reps else f"first {idx} of {len(wl.params)} parameters")
        return mats / t_total, f"{desc} ({mats} matrices, {t_total:.1f} s)"

    v64, s64 = run(budget_s, np.float64)
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([d.get("num_threads", 0) for d in threadpool_info()
                            if d.get("user_api") == "blas"] or [0]) or None
    except Exception:
        blas_threads = None
    out = {"value": round(v64, 4), "unit": "matrices/s", "cores": int(cores), "kind": "oracle",
           "sample": f"{s64}, float64 numpy", "blas": blas_name, "blas_threads": blas_threads,
           "cores_from": "os.sched_getaffinity(0)"}
    if budget32_s > 0:
        v32, s32 = run(budget32_s, np.float32)
        out["value_fp32"] = round(v32, 4)
        out["sample_fp32"] = f"{s32}, the same steps in float32 numpy"
    return out


def path_of(m: int, mode: str) -> str:
    """Kernel path the planner gives an oriented slice with m rows."""
    if m <= 32:
        return "skinny"
    return "large" if mode == "bf16" and m >= 129 else "stream"


def own_work_flops(wl: workloads.Workload, mode: str):
    """Flops of the products as this library computes them, per timing class
    and step (k rounds):
      skinny (Gram-space rounds): the first Gram matrix once (symmetric,
        m(m+1) n), per round A^2 and P^2 (symmetric, m^2 (m+1) each) and
        P Q, S A (2 m^3 each), then one apply Q X0 (2 m^2 n);
      large tiles: per round Gram m(m+1) n and A^2 m^2 (m+1) (one
        triangle each), apply 2 m^2 n;
      other streamed: per round Gram 2 m^2 n, A^2 2 m^3 (full squares), apply 2 m^2 n.
    The dense count of the method, k (4 m^2 n + 2 m^3), is Workload.flops()."""
    k = wl.ns_steps
    cls = {"skinny_gram": 0.0, "skinny_poly": 0.0, "skinny_apply": 0.0, "gram": 0.0, "poly": 0.0, "apply": 0.0}
    for m, n in wl.oriented_matrices():
        path = path_of(m, mode)
        if path == "skinny":
            cls["skinny_gram"] += m * (m + 1) * n
            cls["skinny_poly"] += k * (2 * m * m * (m + 1) + 4 * m ** 3)
            cls["skinny_apply"] += 2 * m * m * n
        elif path == "large":
            cls["gram"] += k * m * (m + 1) * n
            cls["poly"] += k * m * m * (m + 1)
            cls["apply"] += k * 2 * m * m * n
        else:
            cls["gram"] += k * 2 * m * m * n
            cls["poly"] += k * 2 * m ** 3
            cls["apply"] += k * 2 * m * m * n
    return sum(cls.values()), cls


def skinny_bytes(wl: workloads.Workload):
    """Algorithmic bytes of the skinny kernels per step: skinny_gram reads G
    and M and writes M; skinny_apply reads M and W and writes W."""
    gram_b = apply_b = 0.0
    for p in wl.params:
        r, c = p.shape[-2:]
        if min(r, c) <= 32:
            e = 1
            for dd in p.shape:
                e *= dd
            gram_b += e * (elem_bytes(p.grad_dtype) + 8)
            apply_b += e * (4 + 2 * elem_bytes(p.param_dtype))
    return gram_b, apply_b


def measure(wl: workloads.Workload, mode: str, steps: int, warmup: int, dev, graph: bool):
    """Time `steps` eager steps of one fused plan over the workload (inputs
    resident in HBM), then single steps for percentiles, graph replays, and
    per-launch kernel times on a timing plan.  Returns a dict of results."""
    import torch

    from muon_newton_schulz_05_amd import MuonPlan

    params, grads, moms = make_gpu_inputs(wl, dev)
    torch.cuda.synchronize()
    plan = MuonPlan(params, grad_dtypes=[g.dtype for g in grads], mode=mode)
    info = plan.info()
    stream = torch.cuda.current_stream(dev)
    kw = dict(lr=wl.lr, beta=wl.beta, ns_steps=wl.ns_steps, coeffs=wl.coeffs)

    for _ in range(warmup):
        plan.step(grads, moms, **kw)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        plan.step(grads, moms, **kw)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / steps
    # Distribution of single steps: a separate pass, each step between its
    # own pair of events on the launch stream (kept out of the timed region).
    n_dist = max(1, min(steps, 100))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_dist)]
    for e0, e1 in evs:
        e0.record(stream)
        plan.step(grads, moms, **kw)
        e1.record(stream)
    torch.cuda.synchronize()
    per_step = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    pct = lambda q: per_step[min(len(per_step) - 1, int(round(q * (len(per_step) - 1))))]
    step_pct = {"p10": round(pct(0.1), 5), "p50": round(pct(0.5), 5), "p90": round(pct(0.9), 5),
                "steps": n_dist}
    status = plan.status()
    plan.close()

    graph_ms = None
    if graph:
        # The same steps replayed from a HIP graph (a prologue kernel writes
        # the scalars, the graph holds every other launch of the step).
        gs = torch.cuda.Stream(dev)
        gplan = MuonPlan(params, grad_dtypes=[g.dtype for g in grads], mode=mode, use_graph=True)
        with torch.cuda.stream(gs):
            for _ in range(max(1, warmup)):
                gplan.step(grads, moms, **kw)
            gs.synchronize()
            g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            g0.record(gs)
            for _ in range(steps):
                gplan.step(grads, moms, **kw)
            g1.record(gs)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / steps
        status |= gplan.status()
        gplan.close()

    # Per-kernel timing: the same steps again on a plan that brackets every
    # launch with HIP events on the launch stream.
    tplan = MuonPlan(params, grad_dtypes=[g.dtype for g in grads], mode=mode, timing=True)
    tsteps = max(1, min(steps, 20))
    for _ in range(tsteps):
        tplan.step(grads, moms, **kw)
    torch.cuda.synchronize()
    tplan.timings()  # discard the first pass (warm caches)
    for _ in range(tsteps):
        tplan.step(grads, moms, **kw)
    tim = tplan.timings()
    tplan.close()
    del params, grads, moms
    torch.cuda.empty_cache()

    kernel_ms = {k: (v[0] / tsteps, v[1] // tsteps) for k, v in tim.items() if v[1]}
    dominant = max(kernel_ms, key=lambda k: kernel_ms[k][0])
    dom_ms_per_launch = kernel_ms[dominant][0] / max(1, kernel_ms[dominant][1])
    own_total, own_cls = own_work_flops(wl, mode)
    gram_b, apply_b = skinny_bytes(wl)

    if dominant in ("skinny_gram", "skinny_apply"):
        nbytes = gram_b if dominant == "skinny_gram" else apply_b
        per_launch = nbytes / max(1, kernel_ms[dominant][1])
        achieved = per_launch / (dom_ms_per_launch * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": "k_" + dominant, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic("k_" + dominant, wl.name), "algorithmic_bytes_per_launch": per_launch,
                "avg_launch_ms": round(dom_ms_per_launch, 5)}
    else:
        # Own-work flops of the dominant matrix-core class per launch.
        per_launch = own_cls.get(dominant, 0.0) / max(1, kernel_ms[dominant][1])
        achieved = per_launch / (dom_ms_per_launch * 1e-3) / 1e12
        peak = MFMA_PEAK_TFLOPS[mode]
        name = {"gram": "k_gemm_big<GramPhase>", "poly": "k_gemm_big<PolyPhase>",
                "apply": "k_gemm_big<ApplyPhase> + k_gemm_big<FinalPhase>"}.get(dominant, dominant)
        if mode != "bf16" or any(path_of(m, mode) == "stream" for m, _ in wl.oriented_matrices()):
            name = dominant
        roof = {"bound": "mfma", "kernel": name, "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None,
                "algorithmic_flops_per_launch": per_launch, "avg_launch_ms": round(dom_ms_per_launch, 5),
                "flops_counted": "own work: symmetric products counted once (one triangle)"}
        if dominant == "apply" and mode == "bf16":
            roof["traffic"] = measured_traffic("apply", wl.name)
            roof["algorithmic_bytes_per_launch"] = big_apply_bytes(wl)
    if gram_b and "skinny_gram" in kernel_ms and "skinny_apply" in kernel_ms:
        sk_ms = kernel_ms["skinny_gram"][0] + kernel_ms["skinny_apply"][0]
        roof["skinny_pair_gbs"] = round((gram_b + apply_b) / (sk_ms * 1e-3) / 1e9, 1)

    dense = wl.flops()
    comp = compulsory_bytes(wl)
    b_stream, t_roof = stream_model(wl, mode)
    return {
        "ms": ms, "wall_ms": wall * 1e3 / steps, "pct": step_pct, "graph_ms": graph_ms,
        "value": wl.n_matrices / (ms * 1e-3), "dense_tflops": dense / (ms * 1e-3) / 1e12,
        "own_tflops": own_total / (ms * 1e-3) / 1e12, "own_flops": own_total, "dense_flops": dense,
        "compulsory_gbs": comp / (ms * 1e-3) / 1e9, "roofline": roof,
        "stream_model_gbs": b_stream / (ms * 1e-3) / 1e9, "stream_model_bytes": b_stream,
        "t_roof_ms": t_roof * 1e3,
        "kernels_ms_per_step": {k: round(v[0], 5) for k, v in kernel_ms.items()},
        "launches_per_step": info["launches_fixed"] + info["launches_per_ns"] * wl.ns_steps,
        "device_error": status,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=list(workloads.WORKLOADS))
    ap.add_argument("--mode", default=None, choices=["bf16", "fp32"])
    ap.add_argument("--also", default=",".join(EXTRA_WORKLOADS),
                    help="comma-separated workloads measured after the headline one and reported as "
                         "extra keys ('none': skip)")
    ap.add_argument("--cpu-budget", type=float, default=8.0, help="seconds of float64 oracle time (0: skip)")
    ap.add_argument("--cpu-budget-fp32", type=float, default=3.0, help="seconds of float32 oracle time")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replay timing")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the copy/GEMM ceiling measurement")
    ap.add_argument("--copy-only", action="store_true",
                    help="only run the copy ceiling (calibrates the byte counters of a profiler)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU; --gpus must be 1"}))
        sys.exit(2)

    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_only:
        print(json.dumps(measure_ceilings(dev, gemm=False)), flush=True)
        return

    def defaults(wl):
        big = wl.flops() > 1e13
        return (10, 3) if big else (200, 10)

    wl = workloads.WORKLOADS[args.workload]
    mode = args.mode or wl.mode
    d_steps, d_warm = defaults(wl)
    steps = args.steps if args.steps is not None else d_steps
    warmup = args.warmup if args.warmup is not None else d_warm
    r = measure(wl, mode, steps, warmup, dev, graph=not args.no_graph)

    extras = {}
    for name in [x for x in args.also.split(",") if x and x != "none" and x != wl.name]:
        xw = workloads.WORKLOADS[name]
        xs, xwu = defaults(xw)
        xr = measure(xw, xw.mode, xs, xwu, dev, graph=not args.no_graph)
        roof = xr["roofline"]
        extras[name] = {
            "ms_per_step": round(xr["ms"], 5), "matrices_per_s": round(xr["value"], 3), "steps": xs,
            "graph_ms_per_step": None if xr["graph_ms"] is None else round(xr["graph_ms"], 5),
            "dense_tflops": round(xr["dense_tflops"], 2), "own_work_tflops": round(xr["own_tflops"], 2),
            "own_work_frac": round(xr["own_tflops"] / MFMA_PEAK_TFLOPS[xw.mode], 4),
            "compulsory_gbs": round(xr["compulsory_gbs"], 1),
            "compulsory_frac": round(xr["compulsory_gbs"] / HBM_PEAK_GBS, 4),
            "stream_model_gbs": round(xr["stream_model_gbs"], 1),
            "stream_model_frac": round(xr["stream_model_gbs"] / HBM_PEAK_GBS, 4),
            "t_roof_ms": round(xr["t_roof_ms"], 5), "t_roof_frac": round(xr["t_roof_ms"] / xr["ms"], 4),
            "roofline": {k: roof[k] for k in ("bound", "kernel", "achieved", "unit", "frac", "traffic")},
            "kernels_ms_per_step": xr["kernels_ms_per_step"], "device_error": xr["device_error"],
        }

    peak = MFMA_PEAK_TFLOPS[mode]
    out = {
        "metric": "Muon step matrices/s + effective TFLOP/s (frac of MFMA/HBM roofline), 1 GPU",
        "value": round(r["value"], 3),
        "unit": "matrices/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(r["ms"], 5),
        "wall_ms_per_step": round(r["wall_ms"], 5),
        "step_ms_percentiles": r["pct"],
        "graph_ms_per_step": None if r["graph_ms"] is None else round(r["graph_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if mode == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "matrices": wl.n_matrices, "ns_steps": wl.ns_steps, "mode": mode,
                   "shapes": sorted({tuple(p.shape) for p in wl.params}), "graph": False},
        "effective_tflops": round(r["dense_tflops"], 3),
        "effective_tflops_frac": round(r["dense_tflops"] / peak, 4),
        "dense_flops_per_step": r["dense_flops"],
        "own_work_tflops": round(r["own_tflops"], 3),
        "own_work_frac": round(r["own_tflops"] / peak, 4),
        "own_work_flops_per_step": r["own_flops"],
        "compulsory_gbs": round(r["compulsory_gbs"], 1),
        "compulsory_frac": round(r["compulsory_gbs"] / HBM_PEAK_GBS, 4),
        # the streaming cost model: X written and read back every round
        "stream_model_bytes_per_step": r["stream_model_bytes"],
        "stream_model_gbs": round(r["stream_model_gbs"], 1),
        "stream_model_frac": round(r["stream_model_gbs"] / HBM_PEAK_GBS, 4),
        "t_roof_ms": round(r["t_roof_ms"], 5),
        "t_roof_frac": round(r["t_roof_ms"] / r["ms"], 4),
        "roofline": r["roofline"],
        "kernels_ms_per_step": r["kernels_ms_per_step"],
        "launches_per_step": r["launches_per_step"],
        "device_error": r["device_error"],
        "extra_workloads": extras,
    }
    if not args.no_ceilings:
        out["ceilings"] = ceil = measure_ceilings(dev)
        # The same achieved rates against what this machine measured: the
        # library bf16 GEMM for matrix-core classes, the device copy for
        # HBM-bound ones.
        def vs_ceiling(roof, mode_):
            if roof.get("bound") == "mfma" and mode_ == "bf16":
                roof["frac_of_library_gemm"] = round(roof["achieved"] / ceil["library_bf16_gemm_tflops"], 4)
            elif roof.get("bound") == "hbm":
                roof["frac_of_copy"] = round(roof["achieved"] / ceil["copy_gbs"], 4)
        vs_ceiling(out["roofline"], mode)
        for name, x in extras.items():
            vs_ceiling(x["roofline"], workloads.WORKLOADS[name].mode)
    if args.cpu_budget > 0:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget, args.cpu_budget_fp32)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""ctypes binding of libmuon.so (include/muon.h).

Argument marshalling only: every step of the Muon update runs in the HIP
kernels behind the C ABI.  PyTorch is used for device memory and streams.
The functions keep the C names; ``MuonPlan`` wraps a plan for torch tensors.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmuon.so")

MUON_OK = 0
MUON_ERR_INVALID_ARGUMENT = 1
MUON_ERR_UNSUPPORTED = 2
MUON_ERR_HIP = 3
MUON_ERR_OOM = 4
MUON_ERR_DEVICE_MISMATCH = 5
MUON_ERR_DEVICE = 6

MUON_F32 = 0
MUON_BF16 = 1
MUON_MODE_FP32 = 0
MUON_MODE_BF16_MFMA = 1
MUON_PATH_SKINNY = 0
MUON_PATH_STREAM = 1
MUON_MAX_BUCKETS = 64

KERNEL_CLASSES = ("skinny_gram", "skinny_poly", "skinny_apply", "momentum", "norm", "gram", "poly", "apply",
                  "update")
EXPORTED = ("muon_default_opts", "muon_plan_create", "muon_plan_describe", "muon_plan_query",
            "muon_step", "muon_plan_status", "muon_plan_timings", "muon_plan_destroy",
            "muon_step_noalloc", "muon_last_error")
MUON_NOALLOC_SCRATCH_BYTES = 64 << 20


class ParamDesc(ctypes.Structure):
    _fields_ = [("ndim", ctypes.c_int32), ("param_dtype", ctypes.c_int32),
                ("grad_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 3)]


class PlanOpts(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("use_graph", ctypes.c_int32), ("eps", ctypes.c_float),
                ("max_ns_steps", ctypes.c_int32), ("workspace_limit", ctypes.c_uint64),
                ("skinny_max_m", ctypes.c_int32), ("timing", ctypes.c_int32),
                ("n_cu", ctypes.c_int32), ("nesterov", ctypes.c_int32), ("update_scale", ctypes.c_int32),
                ("weight_decay", ctypes.c_float), ("large_min_m", ctypes.c_int32)]


MUON_SCALE_NONE, MUON_SCALE_ASPECT, MUON_SCALE_RMS = 0, 1, 2
UPDATE_SCALES = {"none": MUON_SCALE_NONE, "aspect": MUON_SCALE_ASPECT, "rms": MUON_SCALE_RMS}


class BucketInfo(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int64), ("n", ctypes.c_int64), ("count", ctypes.c_int32),
                ("n_transposed", ctypes.c_int32), ("path", ctypes.c_int32),
                ("chunks", ctypes.c_int32), ("reserved", ctypes.c_int32 * 2),
                ("workspace_bytes", ctypes.c_uint64)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("n_params", ctypes.c_int32), ("n_matrices", ctypes.c_int32),
                ("n_buckets", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_uint64), ("launches_fixed", ctypes.c_int32),
                ("launches_per_ns", ctypes.c_int32),
                ("buckets", BucketInfo * MUON_MAX_BUCKETS)]


class MuonError(RuntimeError):
    def __init__(self, code: int, where: str, message: str):
        super().__init__(f"{where} failed ({code}): {message}")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libmuon.so (built by ``python -m muon_newton_schulz_05_amd.build``).

    Raises if it is missing: there is no fallback implementation."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing; build it with `python -m muon_newton_schulz_05_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.muon_default_opts.argtypes = [ctypes.POINTER(PlanOpts)]
    lib.muon_default_opts.restype = None
    lib.muon_plan_create.argtypes = [ctypes.POINTER(ParamDesc), ctypes.c_int32, ctypes.POINTER(PlanOpts),
                                     ctypes.POINTER(P)]
    lib.muon_plan_describe.argtypes = [ctypes.POINTER(ParamDesc), ctypes.c_int32, ctypes.POINTER(PlanOpts),
                                       ctypes.POINTER(PlanInfo)]
    lib.muon_plan_query.argtypes = [P, ctypes.POINTER(PlanInfo)]
    lib.muon_step.argtypes = [P, ctypes.POINTER(P), ctypes.POINTER(P), ctypes.POINTER(P),
                              ctypes.c_float, ctypes.c_float, ctypes.c_int32,
                              ctypes.c_float, ctypes.c_float, ctypes.c_float, P]
    lib.muon_plan_status.argtypes = [P, ctypes.POINTER(ctypes.c_uint32)]
    lib.muon_plan_timings.argtypes = [P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64),
                                      ctypes.c_int32]
    lib.muon_plan_destroy.argtypes = [P]
    lib.muon_step_noalloc.argtypes = [ctypes.POINTER(ParamDesc), ctypes.c_int32, ctypes.POINTER(PlanOpts),
                                      ctypes.POINTER(P), ctypes.POINTER(P), ctypes.POINTER(P),
                                      ctypes.c_float, ctypes.c_float, ctypes.c_int32,
                                      ctypes.c_float, ctypes.c_float, ctypes.c_float, P, P]
    lib.muon_last_error.argtypes = []
    lib.muon_last_error.restype = ctypes.c_char_p
    for name in ("muon_plan_create", "muon_plan_describe", "muon_plan_query", "muon_step",
                 "muon_plan_status", "muon_plan_timings", "muon_plan_destroy", "muon_step_noalloc"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def muon_last_error() -> str:
    return load_library().muon_last_error().decode()


def _check(rc: int, where: str):
    if rc != MUON_OK:
        raise MuonError(rc, where, muon_last_error())


def muon_default_opts() -> PlanOpts:
    o = PlanOpts()
    load_library().muon_default_opts(ctypes.byref(o))
    return o


def make_descs(shapes, param_dtypes=None, grad_dtypes=None):
    """Build the C descriptor array.  dtypes are "f32"/"bf16" strings or ints."""
    n = len(shapes)
    arr = (ParamDesc * n)()
    to_code = {"f32": MUON_F32, "bf16": MUON_BF16, MUON_F32: MUON_F32, MUON_BF16: MUON_BF16}
    for i, shp in enumerate(shapes):
        arr[i].ndim = len(shp)
        for k, v in enumerate(shp[:3]):
            arr[i].shape[k] = int(v)
        arr[i].param_dtype = to_code.get(param_dtypes[i] if param_dtypes else "f32", 99)
        arr[i].grad_dtype = to_code.get(grad_dtypes[i] if grad_dtypes else "f32", 99)
    return arr


def make_opts(mode="bf16", use_graph=False, eps=1e-7, max_ns_steps=16, workspace_limit=0,
              skinny_max_m=0, timing=False, n_cu=0, nesterov=False, update_scale="none",
              weight_decay=0.0, large_min_m=0) -> PlanOpts:
    o = muon_default_opts()
    o.mode = {"fp32": MUON_MODE_FP32, "bf16": MUON_MODE_BF16_MFMA}.get(mode, mode)
    o.use_graph = int(bool(use_graph))
    o.eps = eps
    o.max_ns_steps = max_ns_steps
    o.workspace_limit = workspace_limit
    o.skinny_max_m = skinny_max_m
    o.timing = int(bool(timing))
    o.n_cu = n_cu
    o.nesterov = int(nesterov)
    o.update_scale = UPDATE_SCALES.get(update_scale, update_scale)
    o.weight_decay = weight_decay
    o.large_min_m = large_min_m
    return o


def muon_plan_describe(descs, opts: PlanOpts | None = None) -> PlanInfo:
    info = PlanInfo()
    _check(load_library().muon_plan_describe(descs, len(descs), ctypes.byref(opts) if opts else None,
                                             ctypes.byref(info)), "muon_plan_describe")
    return info


def muon_plan_create(descs, opts: PlanOpts | None = None) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(load_library().muon_plan_create(descs, len(descs), ctypes.byref(opts) if opts else None,
                                           ctypes.byref(h)), "muon_plan_create")
    return h


def muon_plan_query(plan) -> PlanInfo:
    info = PlanInfo()
    _check(load_library().muon_plan_query(plan, ctypes.byref(info)), "muon_plan_query")
    return info


def muon_step(plan, params, grads, momentum, lr, beta, ns_steps, a, b, c, stream) -> None:
    """params/grads/momentum: sequences of device addresses (ints)."""
    n = len(params)
    P = ctypes.c_void_p * n
    _check(load_library().muon_step(plan, P(*params), P(*grads), P(*momentum), lr, beta, ns_steps,
                                    a, b, c, ctypes.c_void_p(stream)), "muon_step")


def muon_step_noalloc(descs, opts, params, grads, momentum, lr, beta, ns_steps, a, b, c,
                      device_error, stream) -> None:
    """One step in the library's fixed device scratch (no plan, no allocation).
    params/grads/momentum: sequences of device addresses (ints); device_error:
    a device address of a uint32 word, or 0."""
    n = len(params)
    P = ctypes.c_void_p * n
    _check(load_library().muon_step_noalloc(descs, len(descs), ctypes.byref(opts) if opts else None,
                                            P(*params), P(*grads), P(*momentum), lr, beta, ns_steps, a, b, c,
                                            ctypes.c_void_p(device_error or None), ctypes.c_void_p(stream)),
           "muon_step_noalloc")


def muon_plan_status(plan) -> int:
    word = ctypes.c_uint32(0)
    rc = load_library().muon_plan_status(plan, ctypes.byref(word))
    if rc not in (MUON_OK, MUON_ERR_DEVICE):
        _check(rc, "muon_plan_status")
    return int(word.value)


def muon_plan_timings(plan) -> dict:
    n = len(KERNEL_CLASSES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    rc = load_library().muon_plan_timings(plan, ms, cnt, n)
    if rc < 0 or rc > 100:
        _check(rc, "muon_plan_timings")
    return {k: (ms[i], int(cnt[i])) for i, k in enumerate(KERNEL_CLASSES)}


def muon_plan_destroy(plan) -> None:
    _check(load_library().muon_plan_destroy(plan), "muon_plan_destroy")


def info_dict(info: PlanInfo) -> dict:
    return {
        "n_params": info.n_params, "n_matrices": info.n_matrices, "n_buckets": info.n_buckets,
        "mode": info.mode, "workspace_bytes": int(info.workspace_bytes),
        "launches_fixed": info.launches_fixed, "launches_per_ns": info.launches_per_ns,
        "buckets": [
            {"m": b.m, "n": b.n, "count": b.count, "n_transposed": b.n_transposed,
             "path": "skinny" if b.path == MUON_PATH_SKINNY else "stream",
             "chunks": b.chunks, "workspace_bytes": int(b.workspace_bytes)}
            for b in info.buckets[: info.n_buckets]],
    }


# --------------------------------------------------------------------- torch


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return MUON_F32
    if t.dtype == torch.bfloat16:
        return MUON_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


@dataclass
class StepArgs:
    lr: float = 0.02
    beta: float = 0.95
    ns_steps: int = 5
    coeffs: tuple = (3.4445, -4.7750, 2.0315)


class MuonPlan:
    """A plan over a fixed list of parameter tensors (2-D or 3-D, on one GPU).

    ``step(grads, momentum, ...)`` enqueues one fused Muon step on the current
    torch stream; params and momentum are updated in place.
    """

    def __init__(self, params, grad_dtypes=None, mode: str = "bf16", use_graph=False, eps=1e-7,
                 timing=False, skinny_max_m=0, workspace_limit=0, max_ns_steps=16, nesterov=False,
                 update_scale="none", weight_decay=0.0, large_min_m=0):
        import torch
        self.params = list(params)
        if not self.params:
            raise ValueError("no parameters")
        dev = self.params[0].device
        if dev.type != "cuda":
            raise ValueError("parameters must live on a GPU")
        for p in self.params:
            if p.device != dev or not p.is_contiguous():
                raise ValueError("parameters must be contiguous and on one device")
        gd = grad_dtypes or [p.dtype for p in self.params]
        if len(gd) != len(self.params):
            raise ValueError("grad_dtypes must match the parameter list")
        codes = {torch.bfloat16: MUON_BF16, "bf16": MUON_BF16, MUON_BF16: MUON_BF16,
                 torch.float32: MUON_F32, "f32": MUON_F32, MUON_F32: MUON_F32}
        if any(g not in codes for g in gd):
            raise TypeError("grad dtypes must be float32 or bfloat16")
        # The kernels read gradients in the storage type given here, so
        # step() checks every gradient against it.
        self.grad_torch_dtypes = [torch.bfloat16 if codes[g] == MUON_BF16 else torch.float32 for g in gd]
        self.descs = make_descs([tuple(p.shape) for p in self.params],
                                [_dtype_code(p) for p in self.params], [codes[g] for g in gd])
        self.opts = make_opts(mode=mode, use_graph=use_graph, eps=eps, timing=timing,
                              skinny_max_m=skinny_max_m, workspace_limit=workspace_limit,
                              max_ns_steps=max_ns_steps, nesterov=nesterov, update_scale=update_scale,
                              weight_decay=weight_decay, large_min_m=large_min_m)
        self.device = dev
        with torch.cuda.device(dev):
            self.handle = muon_plan_create(self.descs, self.opts)

    def info(self) -> dict:
        return info_dict(muon_plan_query(self.handle))

    def step(self, grads, momentum, lr=0.02, beta=0.95, ns_steps=5, coeffs=(3.4445, -4.7750, 2.0315),
             stream=None):
        import torch
        if len(grads) != len(self.params) or len(momentum) != len(self.params):
            raise ValueError("grads/momentum must match the parameter list")
        for i, (p, g, m) in enumerate(zip(self.params, grads, momentum)):
            if g.shape != p.shape or m.shape != p.shape:
                raise ValueError(f"parameter {i}: shape mismatch")
            if g.device != self.device or m.device != self.device:
                raise ValueError(f"parameter {i}: grads and momentum must be on {self.device}")
            if g.dtype != self.grad_torch_dtypes[i]:
                raise TypeError(f"parameter {i}: gradient is {g.dtype}, the plan expects "
                                f"{self.grad_torch_dtypes[i]}")
            if m.dtype != torch.float32:
                raise TypeError(f"parameter {i}: momentum must be float32")
            if not (g.is_contiguous() and m.is_contiguous()):
                raise ValueError(f"parameter {i}: grads and momentum must be contiguous")
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        muon_step(self.handle, [p.data_ptr() for p in self.params], [g.data_ptr() for g in grads],
                  [m.data_ptr() for m in momentum], lr, beta, ns_steps, *coeffs, s.cuda_stream)

    def status(self) -> int:
        return muon_plan_status(self.handle)

    def timings(self) -> dict:
        return muon_plan_timings(self.handle)

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            muon_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

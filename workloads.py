"""Seeded synthetic inputs for the Muon step (shared by tests and the benchmark).

This module holds no part of the method's arithmetic: it only names the
workloads (shapes, storage types, hyper-parameters) and draws their inputs.
Both the oracle side and the GPU side take their inputs from here.

Shapes follow the sources: 74 parameters of [24, 10240] fused into one batch
("MindSpore HyperParallel X 盘古,Muon优化器实现6倍性能跃升", 矩阵融合优化 /
matrix fusion, Fig. 6-7); 3-D expert tensors whose slices are independent
(same page, 专家切分 / expert split); the transformer matrices h x 3h, h x h,
h x 4h and 4h x h ("关于分布式Muon的想法整合及讨论", §3) at h = 4096.

Gradient recipe: ``numpy.random.default_rng(1000 * config_index + param_index)``
draws float32 N(0, 1) values in C order over the whole parameter, scaled by
the workload's standard deviation and stored either as float32 or rounded to
nearest-even bfloat16 (kept as uint16 bit patterns).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

QUINTIC = (3.4445, -4.7750, 2.0315)
CUBIC = (1.5, -0.5, 0.0)


@dataclass(frozen=True)
class ParamSpec:
    shape: tuple
    param_dtype: str = "f32"   # storage of the weight: "f32" or "bf16"
    grad_dtype: str = "bf16"   # storage of the gradient


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    params: tuple
    grad_std: float
    mode: str                  # "fp32" or "bf16" (the NS arithmetic)
    beta: float = 0.95
    lr: float = 0.02
    ns_steps: int = 5
    coeffs: tuple = QUINTIC
    note: str = field(default="", compare=False)

    @property
    def n_matrices(self) -> int:
        return sum(int(np.prod(p.shape[:-2])) if len(p.shape) == 3 else 1 for p in self.params)

    def oriented_matrices(self):
        """(m, n) of every 2-D slice after orientation, in parameter order."""
        out = []
        for p in self.params:
            r, c = p.shape[-2:]
            e = p.shape[0] if len(p.shape) == 3 else 1
            out += [(min(r, c), max(r, c))] * e
        return out

    def flops(self) -> float:
        """Dense algorithmic flops of one step: k (4 m^2 n + 2 m^3) per slice
        (Gram 2m^2n, A^2 2m^3, B X 2m^2n)."""
        k = self.ns_steps
        return float(sum(k * (4.0 * m * m * n + 2.0 * m ** 3) for m, n in self.oriented_matrices()))


def _transformer(h: int, layers: int):
    out = []
    for _ in range(layers):
        out += [ParamSpec((h, 3 * h)), ParamSpec((h, h)), ParamSpec((h, 4 * h)), ParamSpec((4 * h, h))]
    return tuple(out)


WORKLOADS = {
    "single_128x256": Workload(
        0, "single_128x256", (ParamSpec((128, 256), "f32", "f32"),), grad_std=1.0, mode="fp32",
        note="one float32 matrix, N(0,1) gradient, zero momentum"),
    "fused_74x24x10240": Workload(
        1, "fused_74x24x10240", tuple(ParamSpec((24, 10240)) for _ in range(74)), grad_std=1e-3,
        mode="bf16", note="74 parameters of [24,10240] fused into one [74,24,10240] batch"),
    "moe_experts": Workload(
        2, "moe_experts", (ParamSpec((32, 24, 10240)), ParamSpec((64, 1408, 2048))), grad_std=1e-3,
        mode="bf16", note="3-D expert tensors, Newton-Schulz per expert slice"),
    "dense_h4096_l8": Workload(
        3, "dense_h4096_l8", _transformer(4096, 8), grad_std=1e-3, mode="bf16",
        note="QKV [h,3h], out [h,h], up [h,4h], down [4h,h] (transposed) x 8 layers, h=4096"),
    "large_share": Workload(
        4, "large_share",
        tuple([ParamSpec((8192, 8192))] * 4 + [ParamSpec((16384, 4096))] * 4), grad_std=1e-3,
        mode="bf16", note="4 x [8192,8192] + 4 x [16384,4096] (transposed)"),
}
ORDER = list(WORKLOADS)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16 (ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def seed(workload: Workload, param_index: int) -> int:
    return 1000 * workload.index + param_index


def gradient(workload: Workload, param_index: int, std: float | None = None) -> np.ndarray:
    """Seeded Gaussian gradient of parameter ``param_index`` in its storage type."""
    spec = workload.params[param_index]
    rng = np.random.default_rng(seed(workload, param_index))
    g = rng.standard_normal(spec.shape, dtype=np.float32)
    g *= np.float32(workload.grad_std if std is None else std)
    return f32_to_bf16_bits(g) if spec.grad_dtype == "bf16" else g


def gaussian(shape, seed_value: int, std: float = 1.0, dtype: str = "f32") -> np.ndarray:
    """A generic seeded Gaussian array (float32, or bf16 bits when dtype='bf16')."""
    rng = np.random.default_rng(seed_value)
    g = rng.standard_normal(tuple(shape), dtype=np.float32) * np.float32(std)
    return f32_to_bf16_bits(g) if dtype == "bf16" else g


def zeros_param(spec: ParamSpec) -> np.ndarray:
    return np.zeros(spec.shape, dtype=np.uint16 if spec.param_dtype == "bf16" else np.float32)


def zeros_momentum(spec: ParamSpec) -> np.ndarray:
    return np.zeros(spec.shape, dtype=np.float32)

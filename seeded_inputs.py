"""Seeded synthetic attention inputs, shared by the tests, the benchmark and smoke().

This module draws random tensors and names workloads. It holds none of the attention
arithmetic, so both the HIP path and the CPU oracle can take their inputs from it without
sharing any of the method.

Recipe: Q, K, V and dO are iid N(0, 1), drawn in float32 from NumPy's
``Generator(PCG64(seed))`` with ``seed = 1000 * config + t`` and t = 0, 1, 2, 3 for
Q, K, V, dO. For bf16 workloads the float32 draw is rounded to bfloat16 (round to nearest
even) on the CPU; the rounded values are the canonical inputs for both sides. Layout is
contiguous [B, H, N, d]. The shapes stand in for the benchmark sweeps whose tables were
stripped from "Systems and Parallelism" (CS336 field map, A2), problems pytorch_attention
and flash_benchmarking, and the leaderboard of section 1.3.3.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

TENSOR_INDEX = {"q": 0, "k": 1, "v": 2, "do": 3}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int  # seeds are 1000 * index + t
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str  # "f32" or "bf16"
    causal: bool

    @property
    def scale(self) -> float:
        """1/sqrt(d) rounded to float32: the value both sides receive."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def counted_flops(self) -> dict:
        """Counted work: forward 4*B*H*N^2*d (halved when causal), backward 2.5x forward."""
        fwd = 4.0 * self.B * self.H * self.Nq * self.Nk * self.d
        if self.causal:
            fwd /= 2.0
        return {"fwd": fwd, "bwd": 2.5 * fwd, "total": 3.5 * fwd}


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 1, 1, 128, 128, 16, "f32", True),
    "b8_n4096_d64": Workload("b8_n4096_d64", 2, 8, 1, 4096, 4096, 64, "bf16", True),
    "gpt_small": Workload("gpt_small", 3, 4, 12, 1024, 1024, 64, "bf16", True),
    "long_n16384_d128": Workload("long_n16384_d128", 4, 8, 1, 16384, 16384, 128, "bf16", True),
    "xl_causal": Workload("xl_causal", 5, 4, 25, 2048, 2048, 64, "bf16", True),
    "xl_noncausal": Workload("xl_noncausal", 5, 4, 25, 2048, 2048, 64, "bf16", False),
}


def draw(shape, seed: int) -> np.ndarray:
    """iid N(0,1) in float32 from PCG64(seed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal(size=tuple(shape), dtype=np.float32)


def torch_dtype(dtype: str) -> torch.dtype:
    if dtype == "f32":
        return torch.float32
    if dtype == "bf16":
        return torch.bfloat16
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(B: int, H: int, Nq: int, Nk: int, d: int, dtype: str, index: int) -> dict:
    """CPU tensors q, k, v, do in the canonical dtype (bf16 values already rounded)."""
    shapes = {"q": (B, H, Nq, d), "k": (B, H, Nk, d), "v": (B, H, Nk, d), "do": (B, H, Nq, d)}
    out = {}
    for name, t in TENSOR_INDEX.items():
        x = torch.from_numpy(draw(shapes[name], 1000 * index + t))
        out[name] = x.to(torch_dtype(dtype)).contiguous()
    return out


def workload_inputs(w: Workload) -> dict:
    return make_inputs(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.index)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a CPU tensor (bf16 or f32) to a float64 NumPy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()

"""Seeded synthetic inputs for the MoE layer forward.

This module only draws numbers: it holds none of the layer's arithmetic, so
both the HIP path (through its tests and the bench) and the CPU oracle can
take their inputs from it without sharing any of the method.

Recipe (same for every workload): a CPU ``torch.Generator`` seeded with
``seed`` draws, in this order, X[T,d], W_r[d,E], W_gate[E,d,n], W_up[E,d,n],
W_down[E,n,d], each as ``randn * (1/sqrt(fan_in))`` in float32, with
fan_in = 1 for X (so X ~ N(0,1)), d for W_r / W_gate / W_up and n for W_down.
bf16 workloads then cast each tensor to bfloat16 (round to nearest even).
The skewed workload adds a per-expert router bias b_e = 1.5 * ln(1/(e+1))
(float64, stored as float32); the decode workload reuses the fine-grained
layer's weights and takes the first 64 rows of its X.

Output gradients for the backward: dY[T,d] = randn (N(0,1)) from a CPU
generator seeded with ``seed + 7919`` (a stream of its own, so the layer's
tensors are the same with or without it), cast like the layer's tensors.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int
    K: int
    n: int
    dtype: str                 # "fp32" or "bf16"
    capacity_factor: float = 0.0
    bias: str | None = None    # None or "zipf"
    parent: str | None = None  # decode workloads reuse a parent's weights
    note: str = field(default="", compare=False)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_fp32", 256, 128, 8, 2, 256, "fp32",
                 note="tiny correctness layer, fp32, no capacity limit"),
        Workload("mixtral_bf16", 4096, 4096, 8, 2, 14336, "bf16",
                 note="coarse experts, Mixtral-8x7B-shaped"),
        Workload("qwen3_bf16", 16384, 2048, 128, 8, 768, "bf16",
                 note="fine-grained experts, Qwen3-30B-A3B-shaped"),
        Workload("skewed_cap_bf16", 8192, 2048, 64, 4, 1024, "bf16",
                 capacity_factor=1.25, bias="zipf",
                 note="Zipf-like router bias, capacity factor 1.25"),
        Workload("granular_bf16", 32768, 4096, 256, 8, 512, "bf16",
                 note="G=8, rho=1/32"),
        Workload("granular_decode_bf16", 64, 4096, 256, 8, 512, "bf16",
                 parent="granular_bf16",
                 note="decode size, same weights as granular_bf16"),
    ]
}


def _randn(g, shape, fan_in):
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if fan_in != 1:
        x.mul_(1.0 / math.sqrt(fan_in))
    return x


def zipf_bias(E: int) -> torch.Tensor:
    """b_e = 1.5 * ln(1/(e+1)), computed in float64, stored as float32."""
    return torch.tensor([1.5 * math.log(1.0 / (e + 1)) for e in range(E)],
                        dtype=torch.float64).to(torch.float32)


def draw(T, d, E, n, dtype=torch.bfloat16, seed=0, bias=None):
    """Draw one layer's tensors with the recipe above (CPU tensors)."""
    g = torch.Generator("cpu").manual_seed(seed)
    out = {}
    out["X"] = _randn(g, (T, d), 1).to(dtype)
    out["W_r"] = _randn(g, (d, E), d).to(dtype)
    out["W_gate"] = _randn(g, (E, d, n), d).to(dtype)
    out["W_up"] = _randn(g, (E, d, n), d).to(dtype)
    out["W_down"] = _randn(g, (E, n, d), n).to(dtype)
    if bias == "zipf":
        out["bias"] = zipf_bias(E)
    else:
        out["bias"] = None
    return out


def make_inputs(name: str, seed: int = 0) -> dict:
    """Inputs of a named workload as CPU tensors (plus the workload record)."""
    w = WORKLOADS[name]
    if w.parent is not None:
        p = WORKLOADS[w.parent]
        out = draw(p.T, p.d, p.E, p.n, p.torch_dtype, seed, p.bias)
        out["X"] = out["X"][: w.T].clone()
    else:
        out = draw(w.T, w.d, w.E, w.n, w.torch_dtype, seed, w.bias)
    out["workload"] = w
    return out


def draw_grad_output(T: int, d: int, dtype=torch.bfloat16, seed: int = 0) -> torch.Tensor:
    """dY for the backward (recipe above; CPU tensor)."""
    g = torch.Generator("cpu").manual_seed(seed + 7919)
    return _randn(g, (T, d), 1).to(dtype)


# ---------------------------------------------------------------- atomic experts
# Layers of N = Nr*Nc rank-1 experts with a Cartesian router (the OmniMoE
# design).  Recipe: a CPU generator seeded with ``seed`` draws, in this order,
# X[T,d] ~ N(0,1), W_r[d,Nr] and W_c[d,Nc] ~ N(0,1/d), W_in[N,d] ~ N(0,1/d)
# and W_out[N,d] ~ N(0,1/K) (each output sums K expert rows); then bf16.


@dataclass(frozen=True)
class OmniWorkload:
    name: str
    T: int
    d: int
    Nr: int
    Nc: int
    K: int
    note: str = field(default="", compare=False)


OMNI_WORKLOADS = {
    w.name: w for w in [
        OmniWorkload("omni_small_bf16", 300, 128, 16, 16, 8, note="parity-sized atomic-expert layer"),
        OmniWorkload("omni_bf16", 4096, 1024, 256, 256, 64,
                     note="N = 65536 atomic experts, K = 64, reuse L*K/N = 4"),
    ]
}


def draw_omni(T, d, Nr, Nc, K, seed=0, dtype=torch.bfloat16):
    g = torch.Generator("cpu").manual_seed(seed)
    N = Nr * Nc
    return {
        "X": _randn(g, (T, d), 1).to(dtype),
        "W_r": _randn(g, (d, Nr), d).to(dtype),
        "W_c": _randn(g, (d, Nc), d).to(dtype),
        "W_in": _randn(g, (N, d), d).to(dtype),
        "W_out": _randn(g, (N, d), K).to(dtype),
    }


def make_omni_inputs(name: str, seed: int = 0) -> dict:
    w = OMNI_WORKLOADS[name]
    out = draw_omni(w.T, w.d, w.Nr, w.Nc, w.K, seed)
    out["workload"] = w
    return out


def to_numpy_f32(t: torch.Tensor):
    """Exact float32 numpy copy of a bf16/fp32 tensor (for the oracle)."""
    return t.detach().to("cpu", torch.float32).numpy()

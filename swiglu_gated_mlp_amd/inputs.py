"""Seeded synthetic inputs for the SwiGLU gated-MLP workloads.

This module is the one piece both the GPU library's tests and the CPU oracle's
tests draw from.  It holds none of the method's arithmetic: it only draws random
numbers and rounds them to the bf16 storage type.

Workloads stand in for the Qwen-2.5 MLP gate/up projections the pages measure
on ("Tile-Level Activation Overlap for Efficient LLM Inference", gist.science
technical summary, "Results": Qwen-2.5 0.5B to 72B); no checkpoint is used.
The activation A ~ N(0, 1) and the weights W1, W2 ~ N(0, 1/K) are drawn in fp32
and rounded to bf16, so Gate and Up come out near unit variance.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Tuple

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    """One Qwen-2.5-shaped gate/up projection: Y[M,N] from A[M,K], W1/W2[K,N].

    ``ms`` lists every batch height the workload is run at; the activation is
    drawn once at ``max(ms)`` rows and smaller heights take its first rows, so
    the decode points share a prefix."""
    index: int
    name: str
    K: int
    N: int
    ms: Tuple[int, ...]
    note: str = ""

    @property
    def m_max(self) -> int:
        return max(self.ms)

    def seeds(self) -> Dict[str, int]:
        return {"A": 1000 * self.index + 1, "W1": 1000 * self.index + 2,
                "W2": 1000 * self.index + 3, "W3": 1000 * self.index + 4}


#: The five workloads, indexed 0..4.
WORKLOADS: List[Workload] = [
    Workload(0, "tiny-0.5B", 896, 4864, (64,), "tiny fused SwiGLU, Qwen-2.5-0.5B gate/up shape"),
    Workload(1, "qwen2.5-0.5B-prefill", 896, 4864, (4096,), "short-K prefill"),
    Workload(2, "qwen2.5-7B-decode", 3584, 18944, (1, 16, 128), "weight-bandwidth-bound decode"),
    Workload(3, "qwen2.5-7B-prefill", 3584, 18944, (8192,), "compute-bound prefill"),
    Workload(4, "qwen2.5-72B", 8192, 29568, (32, 4096), "largest single-GPU shape"),
]

BY_NAME = {w.name: w for w in WORKLOADS}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def activation(M: int, K: int, seed: int) -> torch.Tensor:
    """A ~ N(0,1), [M,K], drawn in fp32 then rounded to bf16 (CPU tensor)."""
    return torch.randn(M, K, generator=_gen(seed), dtype=torch.float32).to(torch.bfloat16)


def weight(K: int, N: int, seed: int) -> torch.Tensor:
    """W ~ N(0, 1/K), [K,N] row-major, drawn in fp32 then rounded to bf16."""
    w = torch.randn(K, N, generator=_gen(seed), dtype=torch.float32)
    return (w * (float(max(K, 1)) ** -0.5)).to(torch.bfloat16)


def workload_tensors(w: Workload, m: int | None = None):
    """(A[m,K], W1, W2) for a workload, CPU bf16.  ``m`` defaults to max(ms)."""
    s = w.seeds()
    A = activation(w.m_max, w.K, s["A"])
    if m is not None:
        if m > w.m_max:
            raise ValueError("m=%d exceeds the workload's largest height %d" % (m, w.m_max))
        A = A[:m].contiguous()
    return A, weight(w.K, w.N, s["W1"]), weight(w.K, w.N, s["W2"])


def down_weight(w: Workload) -> torch.Tensor:
    """W3[N,K] ~ N(0, 1/N): the workload's down projection (CPU bf16)."""
    return weight(w.N, w.K, w.seeds()["W3"])


def gaussian_case(M: int, K: int, N: int, seed: int):
    """Small ad-hoc case with the workloads' value distributions."""
    return activation(M, K, 7919 * seed + 11), weight(K, N, 7919 * seed + 12), \
        weight(K, N, 7919 * seed + 13)


def integer_case(M: int, K: int, N: int, seed: int, a_vals=(1, 2, 3), w1_vals=(1, 2, 3),
                 w2_vals=tuple(range(-4, 5))):
    """Integer-valued bf16 inputs drawn uniformly from the given value sets.

    With small integers every partial sum is an integer well below 2^24, so the
    fp32 accumulators are exact in any summation order."""
    g = _gen(104729 * seed + 17)

    def pick(shape, vals):
        v = torch.tensor(vals, dtype=torch.float32)
        idx = torch.randint(0, len(vals), shape, generator=g)
        return v[idx].to(torch.bfloat16)

    return pick((M, K), a_vals), pick((K, N), w1_vals), pick((K, N), w2_vals)


def quantize_e4m3(t: torch.Tensor):
    """Per-tensor FP8 E4M3 quantisation: scale = amax / 448 (the largest finite
    E4M3 value), bytes = E4M3(t / scale) with torch's round-to-nearest-even
    conversion.  Returns (uint8 tensor of E4M3 bytes, scale as a Python float
    that is exactly an fp32 value)."""
    amax = float(t.float().abs().max()) if t.numel() else 0.0
    scale = float(np.float32(amax / 448.0)) if amax > 0 else 1.0
    q = (t.float() / scale).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).contiguous(), scale


def fp8_case(M: int, K: int, N: int, seed: int):
    """The seeded Gaussian case quantised per tensor: (A8, W1_8, W2_8, sg, su)
    with sg = fp32(sA * s1) and su = fp32(sA * s2), the scale products both
    sides apply to the fp32 Gate and Up sums."""
    A, W1, W2 = gaussian_case(M, K, N, seed)
    A8, sa = quantize_e4m3(A)
    W18, s1 = quantize_e4m3(W1)
    W28, s2 = quantize_e4m3(W2)
    sg = float(np.float32(sa) * np.float32(s1))
    su = float(np.float32(sa) * np.float32(s2))
    return A8, W18, W28, sg, su


def as_bits(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (CPU copy)."""
    import numpy as np
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(bits) -> torch.Tensor:
    """numpy uint16 bit patterns -> bf16 CPU tensor."""
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)

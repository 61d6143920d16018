"""Seeded synthetic inputs for the NVFP4 MoE workloads.

This module is shared by the HIP path's tests/bench and by the oracle's
tests. It holds NONE of the method's arithmetic (no quantization, routing,
GEMM or rounding rule): it only draws the FP32 / bf16 tensors that both sides
consume, with the shapes and value distributions of the workloads measured
on the pages:

  * tiny    -- 8 experts, top-2, 16 tokens, H=256, F=512 (W4A16).
  * dense   -- one M=512, N=2048, K=6144 GEMM ("The 2x Gap", section
               "The Pivot: Comparing FP4 Against BF16").
  * decode  -- 256 experts, top-8, H=6144, F=2048, tokens in {1,8,16,64,512}
               ("The 2x Gap", section "The Investigation So Far": 512
               concurrent requests, 8 of 256 experts, ~16 tokens/expert).
  * many_small -- 512 experts, top-22, H=4096, F=1024, tokens in {1,4,16,64},
               FP8 activations ("Native FP4 Is Slower Than Emulated FP4",
               section 1).
  * prefill -- 8192 tokens, 256 experts, top-8, H=7168, F=2048, W4A4, with a
               Zipf(1.1) expert bias added to the router logits.

Distributions: weights FP32 N(0, 0.02); activations FP32 N(0, 1) cast to bf16;
router logits FP32 N(0, 1); the prefill bias is b_e = -1.1 * ln(r_e) with
r a seeded permutation of 1..E (a Zipf(1.1) law on expert popularity, added
in log space). Every tensor has its own seed derived from
(workload, tensor kind, expert), so experts can be generated one at a time
on any device and regenerated identically on the same device.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens (rows for the dense GEMM)
    E: int            # experts (1 for the dense GEMM)
    k: int            # top-k
    H: int            # hidden size (K of up/gate, N of down); K for dense
    F: int            # expert FFN width; N for dense
    mode: str         # "w4a16" | "w4a4"
    act: str = "bf16"  # "bf16" | "fp8" (FP8 E4M3 activations dequantized to bf16)
    zipf: float = 0.0
    sweep: tuple = field(default_factory=tuple)


WORKLOADS = {
    "tiny": Workload("tiny", T=16, E=8, k=2, H=256, F=512, mode="w4a16"),
    "dense": Workload("dense", T=512, E=1, k=1, H=6144, F=2048, mode="w4a16"),
    "decode": Workload("decode", T=512, E=256, k=8, H=6144, F=2048, mode="w4a16",
                       sweep=(1, 8, 16, 64, 512)),
    "many_small": Workload("many_small", T=64, E=512, k=22, H=4096, F=1024, mode="w4a16",
                           act="fp8", sweep=(1, 4, 16, 64)),
    "prefill": Workload("prefill", T=8192, E=256, k=8, H=7168, F=2048, mode="w4a4", zipf=1.1),
}

WEIGHT_STD = 0.02


def seed_of(workload: str, kind: str, index: int = 0) -> int:
    """Stable 63-bit seed for (workload, tensor kind, index)."""
    return (zlib.crc32(f"{workload}/{kind}".encode()) << 20) + int(index)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def expert_weight_fp32(wl: Workload, which: str, e: int, device="cpu") -> torch.Tensor:
    """FP32 N(0, 0.02) weight of expert e.

    ``which`` = "w13" -> [2F, H] (rows 0..F-1 gate, F..2F-1 up),
    ``which`` = "w2"  -> [H, F],
    ``which`` = "dense" -> [F, H] (the dense GEMM's [N, K] weight).
    """
    shape = {"w13": (2 * wl.F, wl.H), "w2": (wl.H, wl.F), "dense": (wl.F, wl.H)}[which]
    g = _gen(device, seed_of(wl.name, which, e))
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * WEIGHT_STD


def activations_fp32(wl: Workload, T: int | None = None, device="cpu") -> torch.Tensor:
    """FP32 N(0, 1) activations [T, H]."""
    T = wl.T if T is None else T
    g = _gen(device, seed_of(wl.name, f"x{T}"))
    return torch.randn((T, wl.H), generator=g, device=device, dtype=torch.float32)


def activations_bf16(wl: Workload, T: int | None = None, device="cpu") -> torch.Tensor:
    """The activations as bf16 (a plain dtype cast of :func:`activations_fp32`)."""
    return activations_fp32(wl, T, device).to(torch.bfloat16)


def router_logits(wl: Workload, T: int | None = None, device="cpu") -> torch.Tensor:
    """FP32 router logits [T, E]: N(0, 1), plus the Zipf bias when the workload has one."""
    T = wl.T if T is None else T
    g = _gen(device, seed_of(wl.name, f"logits{T}"))
    lg = torch.randn((T, wl.E), generator=g, device=device, dtype=torch.float32)
    if wl.zipf:
        gp = _gen("cpu", seed_of(wl.name, "zipf_rank"))
        rank = torch.randperm(wl.E, generator=gp).to(torch.float64) + 1.0
        bias = (-wl.zipf * torch.log(rank)).to(torch.float32).to(device)
        lg = lg + bias[None, :]
    return lg


def random_fp32(shape, seed: int, std: float = 1.0, device="cpu") -> torch.Tensor:
    """Generic seeded N(0, std) FP32 tensor for unit tests."""
    return torch.randn(shape, generator=_gen(device, seed), device=device,
                       dtype=torch.float32) * std

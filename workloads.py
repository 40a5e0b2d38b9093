"""Seeded synthetic inputs for the attention workloads.

This module only draws inputs and names workload shapes; it holds none of
the attention arithmetic. The GPU path and the CPU oracle both consume the
same bfloat16 tensors drawn here.

Recipe: for a workload with seed s, a CPU torch.Generator seeded with s
draws q, then k, then v with torch.randn(B, H, N, d) in float32, and each is
rounded to bfloat16 (round to nearest even). Values are N(0, 1), which
stands in for the Stable Diffusion 2.1 UNet activations of the NKI tutorial
("Fused Self Attention", seqlen 4096 and d_head 64 at 512x512; the 96x96
latent at 768x768), for the causal decoder of "Profiling in PyTorch", and for
the MR-image neighbourhood attention of NATTEN issue 142; none of those
activations, weights or datasets are available, so only the shapes are kept.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    mask: str               # "none" | "causal" | "na2d"
    scale: float            # float32-representable value passed to both sides
    seed: int
    na2d: dict = field(default_factory=dict)   # grid_h, grid_w, kernel_h, kernel_w, wrap_h, wrap_w
    note: str = ""


def f32(x: float) -> float:
    """Round a Python float to the nearest float32 value."""
    return float(torch.tensor(x, dtype=torch.float32).item())


WORKLOADS = {
    w.name: w
    for w in [
        Workload("single_head_n256", 1, 1, 256, 64, "none", f32(1 / math.sqrt(64)), 6801,
                 note="single-head self-attention, B1 H1 N256 d64"),
        Workload("sd21_512_selfattn", 2, 5, 4096, 64, "none", f32(1 / 8), 6802,
                 note="SD2.1 512x512 UNet self-attention, 64x64 latent, B2 H5 N4096 d64"),
        Workload("causal_n2048", 4, 16, 2048, 64, "causal", f32(1 / 8), 6803,
                 note="causal decoder attention, B4 H16 N2048 d64"),
        Workload("na2d_wrap_64x64_k7", 2, 4, 4096, 32, "na2d", f32(1 / math.sqrt(32)), 6804,
                 na2d=dict(grid_h=64, grid_w=64, kernel_h=7, kernel_w=7, wrap_h=1, wrap_w=1),
                 note="2D neighbourhood attention, 64x64 grid, 7x7 window wrapping both axes, d32"),
        Workload("sd21_768_selfattn", 2, 5, 9216, 64, "none", f32(1 / 8), 6805,
                 note="SD2.1 768x768 UNet self-attention, 96x96 latent, B2 H5 N9216 d64"),
    ]
}

# the workload the headline metric is quoted on
HEADLINE = "sd21_512_selfattn"


def make_qkv(B: int, H: int, N: int, d: int, seed: int, q_gain: float = 1.0):
    """Draw bfloat16 q, k, v of shape [B, H, N, d] on the CPU (see the module recipe).

    q_gain multiplies q before rounding (a "peaky" variant with sharper rows).
    """
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn(B, H, N, d, generator=g, dtype=torch.float32)
    k = torch.randn(B, H, N, d, generator=g, dtype=torch.float32)
    v = torch.randn(B, H, N, d, generator=g, dtype=torch.float32)
    return (q * q_gain).to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def workload_qkv(w: Workload):
    return make_qkv(w.B, w.H, w.N, w.d, w.seed)

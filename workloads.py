"""Seeded synthetic inputs for the attention workloads.

This module only draws inputs and names workload shapes; it holds none of
the attention arithmetic. The GPU path and the CPU oracle both consume the
same bfloat16 tensors drawn here.

Recipe: for a workload with seed s, a CPU torch.Generator seeded with s
draws q, then k, then v with torch.randn in float32 (q of shape [B, H, N, d],
k and v of shape [B, H, Nkv, d], Nkv = N unless stated), and each is rounded
to bfloat16 (round to nearest even). Values are N(0, 1), which
stands in for the Stable Diffusion 2.1 UNet activations of the NKI tutorial
("Fused Self Attention", seqlen 4096 and d_head 64 at 512x512; the 96x96
latent at 768x768), for the causal decoder of "Profiling in PyTorch", and for
the MR-image neighbourhood attention of NATTEN issue 142; none of those
activations, weights or datasets are available, so only the shapes are kept.

Shapes the pages leave open are readings: the SD2.1 cross-attention takes 77
context tokens (the text encoder's sequence length) against the 4096 latent
tokens; the d = 128 workload keeps the SD2.1 512x512 token count; the 3D
volume is 20 x 20 x 20 patches with a 5 x 5 x 5 window wrapping in two of its
three axes (the issue's "~15-20 patches in each dim", "window size 5" and
wrapping "in at least 1-2 dimensions").
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
    mask: str               # "none" | "causal" | "na2d" | "na3d"
    scale: float            # float32-representable value passed to both sides
    seed: int
    na: dict = field(default_factory=dict)     # window: grid_*, kernel_*, wrap_*, dil_* per axis
    note: str = ""
    Nkv: int = 0            # keys per head (0: N, self-attention)

    @property
    def n_kv(self) -> int:
        return self.Nkv or self.N


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
                 na=dict(grid_h=64, grid_w=64, kernel_h=7, kernel_w=7, wrap_h=1, wrap_w=1),
                 note="2D neighbourhood attention, 64x64 grid, 7x7 window wrapping both axes, d32"),
        Workload("sd21_768_selfattn", 2, 5, 9216, 64, "none", f32(1 / 8), 6805,
                 note="SD2.1 768x768 UNet self-attention, 96x96 latent, B2 H5 N9216 d64"),
        Workload("sd21_512_crossattn", 2, 5, 4096, 64, "none", f32(1 / 8), 6806, Nkv=77,
                 note="SD2.1 512x512 UNet cross-attention, 4096 latent queries against 77 context keys, d64"),
        Workload("selfattn_n4096_d128", 2, 5, 4096, 128, "none", f32(1 / math.sqrt(128)), 6807,
                 note="self-attention at the SD2.1 512x512 token count with 128-wide heads"),
        Workload("na3d_wrap_20x20x20_k5", 2, 4, 8000, 32, "na3d", f32(1 / math.sqrt(32)), 6808,
                 na=dict(grid_d=20, grid_h=20, grid_w=20, kernel_d=5, kernel_h=5, kernel_w=5,
                         wrap_d=1, wrap_h=1, wrap_w=0),
                 note="3D neighbourhood attention, 20x20x20 volume, 5x5x5 window wrapping depth and rows, d32"),
        Workload("na2d_wrap_64x64_k7_dil2", 2, 4, 4096, 32, "na2d", f32(1 / math.sqrt(32)), 6809,
                 na=dict(grid_h=64, grid_w=64, kernel_h=7, kernel_w=7, wrap_h=1, wrap_w=1, dil_h=2, dil_w=2),
                 note="2D neighbourhood attention, 64x64 grid, 7x7 window dilated by 2, wrapping both axes, d32"),
        Workload("na3d_wrap_20x20x20_k5_dil2", 2, 4, 8000, 32, "na3d", f32(1 / math.sqrt(32)), 6810,
                 na=dict(grid_d=20, grid_h=20, grid_w=20, kernel_d=5, kernel_h=5, kernel_w=5,
                         wrap_d=1, wrap_h=1, wrap_w=0, dil_d=2, dil_h=2, dil_w=2),
                 note="3D neighbourhood attention, 20x20x20 volume, 5x5x5 window dilated by 2 on every axis, "
                      "wrapping depth and rows, d32"),
        Workload("na2d_clamp_64x64_k7", 2, 4, 4096, 32, "na2d", f32(1 / math.sqrt(32)), 6811,
                 na=dict(grid_h=64, grid_w=64, kernel_h=7, kernel_w=7, wrap_h=0, wrap_w=0),
                 note="2D neighbourhood attention, 64x64 grid, 7x7 window clamped at the borders on both axes, d32"),
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


def make_qkv_cross(B: int, H: int, Nq: int, Nkv: int, d: int, seed: int, q_gain: float = 1.0):
    """Like make_qkv with Nq queries and Nkv keys: q [B, H, Nq, d], then k and v [B, H, Nkv, d]."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn(B, H, Nq, d, generator=g, dtype=torch.float32)
    k = torch.randn(B, H, Nkv, d, generator=g, dtype=torch.float32)
    v = torch.randn(B, H, Nkv, d, generator=g, dtype=torch.float32)
    return (q * q_gain).to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def workload_qkv(w: Workload):
    if w.n_kv != w.N:
        return make_qkv_cross(w.B, w.H, w.N, w.n_kv, w.d, w.seed)
    return make_qkv(w.B, w.H, w.N, w.d, w.seed)

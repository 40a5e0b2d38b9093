"""Parity of attn_bwd (the backward pass: gradients of Q, K and V) against the float64 CPU oracle on an
MI355X. attn_bwd gets the oracle's output (bf16) and logsumexp (fp32), so the per-element tolerance
(parity.bwd_reference, derived from the backward's arithmetic) covers the backward alone; the
pipeline cases feed it the GPU forward's output and logsumexp instead."""
import math

import numpy as np
import pytest
import torch

import workloads
from parity import check_bwd_case, run_gpu_bwd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    from exact_attention_68_amd.build import ensure_built

    ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"


def _inputs(B, H, Nq, Nkv, d, seed, q_gain=1.0):
    q, k, v = workloads.make_qkv_cross(B, H, Nq, Nkv, d, seed, q_gain)
    g = torch.Generator(device="cpu").manual_seed(seed + 1)
    do = torch.randn(B, H, Nq, d, generator=g, dtype=torch.float32).to(torch.bfloat16)
    return q, k, v, do


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("mask", ["none", "causal"])
@pytest.mark.parametrize("N", [1, 17, 100, 128, 255, 257, 320])
def test_bwd_edge_shapes(N, mask, d):
    q, k, v, do = _inputs(1, 2, N, N, d, 11000 + N + d)
    check_bwd_case(q, k, v, do, 1 / math.sqrt(d), mask, what=f"bwd N{N}")


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("mask", ["none", "causal"])
@pytest.mark.parametrize("Nq,Nkv", [(300, 77), (77, 300), (1, 500), (500, 1), (129, 384)])
def test_bwd_cross_shapes(Nq, Nkv, mask, d):
    q, k, v, do = _inputs(1, 2, Nq, Nkv, d, 11100 + Nq + Nkv + d)
    check_bwd_case(q, k, v, do, 1 / math.sqrt(d), mask, what=f"bwd cross {Nq}x{Nkv}")


@pytest.mark.parametrize("scale,q_gain", [(0.0, 1.0), (-0.2, 1.0), (0.125, 2.0), (1e-3, 1.0)])
@pytest.mark.parametrize("mask", ["none", "causal"])
def test_bwd_scales(scale, q_gain, mask):
    q, k, v, do = _inputs(2, 3, 300, 300, 64, 11200, q_gain)
    check_bwd_case(q, k, v, do, scale, mask, what=f"bwd scale {scale} gain {q_gain}")


@pytest.mark.parametrize("mask", ["none", "causal"])
def test_bwd_sd21_head_shape(mask):
    """Two heads at the SD2.1 512x512 token count (N4096, d64)."""
    q, k, v, do = _inputs(1, 2, 4096, 4096, 64, 11300)
    check_bwd_case(q, k, v, do, 0.125, mask, what="bwd N4096")


@pytest.mark.parametrize("mask", ["none", "causal"])
def test_bwd_d128_head_shape(mask):
    """One head of the d = 128 workload's size (N4096, d128)."""
    q, k, v, do = _inputs(1, 1, 4096, 4096, 128, 11320)
    check_bwd_case(q, k, v, do, 1 / math.sqrt(128), mask, what="bwd N4096 d128")


@pytest.mark.parametrize("mask", ["none", "causal"])
@pytest.mark.parametrize("N,Nkv,d", [(300, 300, 64), (257, 100, 32), (1000, 1000, 64), (700, 700, 128)])
def test_bwd_after_gpu_forward(N, Nkv, d, mask):
    """attn_fwd_ex then attn_bwd, both on the GPU (bound with the forward's errors as inputs)."""
    q, k, v, do = _inputs(1, 2, N, Nkv, d, 11350 + N + Nkv)
    check_bwd_case(q, k, v, do, 1 / math.sqrt(d), mask, what=f"bwd pipeline {N}x{Nkv}", pipeline=True)


# ---------------------------------------------------------------- neighbourhood windows
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("mode,geo", [
    ("na2d", (5, 5, 3, 3, 1, 1, 1, 1)),       # the issue's 5x5 wrap example geometry
    ("na2d", (8, 9, 5, 5, 1, 1, 1, 1)),
    ("na2d", (7, 13, 3, 5, 0, 0, 1, 1)),      # clamped windows: not symmetric between queries and keys
    ("na2d", (10, 6, 5, 3, 1, 0, 1, 1)),
    ("na2d", (33, 17, 9, 3, 1, 1, 1, 1)),     # band crosses tiles and wraps
    ("na2d", (16, 20, 3, 5, 1, 1, 2, 3)),     # dilated, wrapped
    ("na2d", (17, 9, 5, 3, 0, 0, 3, 2)),      # dilated, clamped
    ("na3d", (3, 5, 4, 3, 3, 3, 1, 1, 1, 1, 1, 1)),
    ("na3d", (6, 6, 6, 3, 3, 3, 1, 0, 1, 2, 2, 2)),
    ("na2d", (40, 3, 5, 3, 1, 1, 2, 1)),      # width 3 and 200: the element test instead of the window masks
    ("na2d", (2, 200, 1, 7, 0, 1, 1, 3)),
    ("na3d", (2, 130, 4, 1, 5, 3, 0, 1, 1, 1, 2, 1)),   # more than 128 rows
    # at d = 32 these take the row kernels (grids at most 32 wide): dQ by query rows, dK/dV by key
    # rows over the queries whose windows reach them
    ("na3d", (8, 8, 8, 5, 5, 5, 1, 1, 0, 1, 1, 1)),     # the 3D workload's window: wrapped planes and rows
    ("na3d", (5, 9, 20, 3, 5, 5, 0, 1, 1, 1, 1, 1)),    # clamped planes, 9 rows (a partial group)
    ("na3d", (4, 6, 32, 3, 3, 7, 1, 0, 0, 1, 1, 1)),    # 32 wide, clamped rows and columns
    ("na2d", (12, 31, 3, 7, 0, 0, 1, 1)),               # clamped both ways: reverse bands near the borders
    ("na2d", (20, 32, 5, 5, 0, 1, 1, 1)),               # clamped 5-row windows: dK/dV on the patch kernel (reverse row bands past 8)
    ("na2d", (16, 20, 3, 5, 1, 0, 2, 2)),               # dilated rows and columns
    ("na2d", (9, 1, 3, 1, 1, 0, 1, 1)),                 # one column
    # wider single-plane grids at d = 32 and 64: the patch kernels (8 x 16 patches over LDS rectangles)
    ("na2d", (20, 40, 5, 5, 1, 1, 1, 1)),
    ("na2d", (17, 48, 7, 3, 0, 0, 1, 1)),               # clamped: reverse rectangles near the borders
    ("na2d", (24, 36, 3, 7, 1, 0, 2, 1)),               # dilated rows, clamped columns
    ("na2d", (33, 64, 5, 9, 0, 1, 1, 2)),               # a 32-column band: dilated, wrapped columns
    ("na2d", (40, 64, 7, 7, 0, 0, 2, 2)),               # clamped and dilated (tight clamped bands)
    ("na2d", (30, 50, 5, 5, 0, 0, 3, 3)),               # dilation 3, clamped
    ("na2d", (32, 48, 5, 7, 1, 1, 2, 2)),               # patches of rows of one parity (also at d = 64)
    ("na2d", (33, 48, 5, 5, 1, 1, 2, 2)),               # 33 wrapped rows: patches of consecutive rows
    ("na2d", (48, 64, 7, 7, 1, 1, 4, 4)),               # dilation 4: patches of one residue per axis
    ("na2d", (40, 48, 5, 9, 0, 0, 3, 3)),               # clamped, dilation 3: residue sub-grids of unequal lengths
    ("na3d", (10, 12, 14, 3, 3, 3, 0, 0, 0, 2, 2, 3)),  # clamped, dilated (d = 128: the tile kernels' query runs)
    # row groups of one residue mod the dilation (8-row bands), and the wide 12-row stages, at d = 32
    ("na3d", (10, 16, 12, 5, 5, 5, 1, 1, 0, 2, 2, 1)),  # 16 wrapped rows, dilation 2: groups of one residue
    ("na3d", (10, 15, 12, 5, 5, 5, 1, 1, 0, 2, 2, 1)),  # 15 wrapped rows: consecutive groups, all three wide
    ("na3d", (6, 20, 12, 3, 5, 5, 0, 0, 0, 1, 1, 1)),   # clamped: dK/dV's 10-row reverse bands near the borders
    ("na3d", (7, 13, 9, 3, 5, 3, 0, 0, 1, 2, 2, 1)),    # clamped and dilated: residue groups of 7 and 6 rows
])
def test_bwd_neighbourhood(mode, geo, d):
    import exact_attention_68_amd as A

    params = A.na2d_params(*geo) if mode == "na2d" else A.na3d_params(*geo)
    N = geo[0] * geo[1] * (geo[2] if mode == "na3d" else 1)
    q, k, v, do = _inputs(1, 2, N, N, d, 11600 + N + d)
    check_bwd_case(q, k, v, do, 1 / math.sqrt(d), mode, what=f"bwd {mode} {geo}", params=params)


@pytest.mark.parametrize("scale", [0.0, -0.3, 1e-3])
@pytest.mark.parametrize("mode,geo", [
    ("na3d", (6, 7, 9, 3, 5, 3, 1, 1, 0, 1, 1, 1)),   # the row kernels
    ("na3d", (5, 13, 9, 3, 5, 3, 1, 1, 0, 2, 2, 1)),  # their wide 12-row stages (13 rows, dilation 2)
    ("na3d", (5, 12, 9, 3, 5, 3, 1, 1, 0, 2, 2, 1)),  # row groups of one residue (12 rows, dilation 2)
    ("na2d", (20, 40, 5, 7, 1, 0, 1, 1)),             # the patch kernels
])
def test_bwd_neighbourhood_scales(mode, geo, scale):
    """Scale 0 (every visible key weighs the same), a negative scale (the flipped sign bits of K in the
    dK/dV kernels, of Q in the dQ kernels) and a tiny one, through the row and patch kernels at d = 32."""
    import exact_attention_68_amd as A

    params = A.na2d_params(*geo) if mode == "na2d" else A.na3d_params(*geo)
    N = geo[0] * geo[1] * (geo[2] if mode == "na3d" else 1)
    q, k, v, do = _inputs(1, 2, N, N, 32, 11700 + N)
    check_bwd_case(q, k, v, do, scale, mode, what=f"bwd {mode} {geo} scale {scale}", params=params)


def test_bwd_neighbourhood_workload_shape():
    """The 64x64 7x7 wrapped window of the 2D workload (B2 H4 d32), through the GPU forward."""
    import exact_attention_68_amd as A

    w = workloads.WORKLOADS["na2d_wrap_64x64_k7"]
    q, k, v = workloads.workload_qkv(w)
    g = torch.Generator(device="cpu").manual_seed(w.seed + 1)
    do = torch.randn(w.B, w.H, w.N, w.d, generator=g, dtype=torch.float32).to(torch.bfloat16)
    check_bwd_case(q, k, v, do, w.scale, "na2d", what="bwd na2d 64x64 k7", pipeline=True, params=A.na2d_params(**w.na))


def test_bwd_deterministic_and_workspace_content_free():
    """Every gradient element is written by one lane in a fixed order: repeated calls agree bit for bit,
    whatever the workspace held."""
    q, k, v, do = _inputs(2, 3, 700, 700, 64, 11400)
    a = run_gpu_bwd(q, k, v, do, 0.125, 1)
    b = run_gpu_bwd(q, k, v, do, 0.125, 1)
    assert all(torch.equal(x, y) for x, y in zip(a[:3], b[:3]))


def test_bwd_rejects_unsupported_and_leaves_outputs():
    import exact_attention_68_amd as A

    q, k, v, do = (t.cuda() for t in _inputs(1, 1, 64, 64, 96, 11500))
    o = torch.zeros_like(q)
    lse = torch.zeros(1, 1, 64, dtype=torch.float32, device="cuda")
    gq, gk, gv = (torch.full_like(t, 3.0) for t in (q, k, v))
    ws = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(A.AttnError) as e:
        A.attn_bwd(q, k, v, o, do, lse, gq, gk, gv, 0.1, A.ATTN_MASK_NONE, None, ws)
    assert e.value.status == A.ATTN_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert all(torch.all(t == 3.0) for t in (gq, gk, gv))

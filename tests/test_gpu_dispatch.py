"""How many GPU dispatches one call of each entry point makes, counted in-process with
torch.profiler (no relaunch, no second process).

The fused forward is one kernel: the score matrix never reaches memory and nothing
is copied or cleared on the device ("Profiling in PyTorch", the efficient SDPA
backend: one fused kernel per forward; and the in-place masked_fill_ section: an
out-of-place mask costs an extra Memcpy kernel). attn_fwd_ws / attn_fwd_ex queue a
one-work-group kernel that zeroes the split tiles' arrival counters before the
attention kernel only when they split key ranges (the parts are merged inside the
attention kernel); attn_bwd is two kernels (dQ, then dK and dV).
"""
import pytest
import torch

import workloads
from parity import split_workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    from exact_attention_68_amd.build import ensure_built

    ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"


def _dispatches(fn):
    """Names of the device activities (kernels, copies, fills) recorded while fn runs."""
    from torch.autograd import DeviceType
    from torch.profiler import ProfilerActivity, profile

    fn()  # warm: module loading and first-launch work stay outside the recording
    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        fn()
        torch.cuda.synchronize()
    return [e.name for e in prof.events() if e.device_type == DeviceType.CUDA]


def _split(names):
    kernels = [n for n in names if "attn" in n]
    others = [n for n in names if "attn" not in n]
    return kernels, others


def _inputs(B, H, N, d, seed):
    return [t.cuda() for t in workloads.make_qkv(B, H, N, d, seed)]


@pytest.mark.parametrize("mask", ["none", "causal"])
def test_attn_fwd_is_one_kernel(mask):
    import exact_attention_68_amd as A

    q, k, v = _inputs(2, 5, 4096, 64, 1)
    o = torch.empty_like(q)
    mode = A.ATTN_MASK_CAUSAL if mask == "causal" else A.ATTN_MASK_NONE
    kernels, others = _split(_dispatches(lambda: A.attn_fwd(q, k, v, o, 0.125, mode)))
    assert len(kernels) == 1 and "attn_fwd_kernel" in kernels[0], kernels
    assert others == [], others  # no memcpy, no memset


@pytest.mark.parametrize("N,expect", [(4096, 2), (1000, 2), (9216, 1)])
def test_attn_fwd_ws_dispatches(N, expect):
    """SD2.1-512 (320 query tiles) and a 1000-token problem split (counter clear + attention);
    SD2.1-768 (720 tiles, more than two per CU) does not."""
    import exact_attention_68_amd as A

    B, H, d = (2, 5, 64) if N != 1000 else (1, 2, 64)
    q, k, v = _inputs(B, H, N, d, 2)
    o = torch.empty_like(q)
    ws = split_workspace(B, H, N, d, A.ATTN_MASK_NONE)
    kernels, others = _split(_dispatches(lambda: A.attn_fwd_ws(q, k, v, o, 0.125, A.ATTN_MASK_NONE, None, ws)))
    assert len(kernels) == expect, kernels
    if expect == 2:
        assert "attn_split_clear_kernel" in kernels[0] and "attn_fwd_kernel" in kernels[1], kernels
    else:
        assert "attn_fwd_kernel" in kernels[0], kernels
    assert others == [], others


def test_attn_fwd_ex_na2d_is_one_kernel():
    import exact_attention_68_amd as A

    w = workloads.WORKLOADS["na2d_wrap_64x64_k7"]
    q, k, v = (t.cuda() for t in workloads.workload_qkv(w))
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device="cuda")
    params = A.na2d_params(**w.na)
    kernels, others = _split(_dispatches(
        lambda: A.attn_fwd_ex(q, k, v, o, lse, w.scale, A.ATTN_MASK_NA2D, params, None)))
    assert len(kernels) == 1, kernels
    assert others == [], others


def test_attn_bwd_is_two_kernels():
    import exact_attention_68_amd as A

    B, H, N, d = 1, 4, 1024, 64
    q, k, v = _inputs(B, H, N, d, 3)
    do = torch.randn(B, H, N, d, device="cuda").to(torch.bfloat16)
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, dtype=torch.float32, device="cuda")
    A.attn_fwd_ex(q, k, v, o, lse, 0.125, A.ATTN_MASK_CAUSAL)
    ws = torch.empty(A.attn_bwd_workspace_size(B, H, N, N, d, A.ATTN_MASK_CAUSAL), dtype=torch.uint8, device="cuda")
    grads = [torch.empty_like(t) for t in (q, k, v)]
    kernels, others = _split(_dispatches(
        lambda: A.attn_bwd(q, k, v, o, do, lse, *grads, 0.125, A.ATTN_MASK_CAUSAL, None, ws)))
    assert len(kernels) == 2, kernels
    assert "attn_bwd_dq_kernel" in kernels[0] and "attn_bwd_dkv_kernel" in kernels[1], kernels
    assert others == [], others


@pytest.mark.parametrize("name,dq,dkv", [
    ("na3d_wrap_20x20x20_k5", "attn_bwd_dq_rows_kernel", "attn_bwd_dkv_rows_kernel"),
    ("na2d_wrap_64x64_k7", "attn_bwd_dq_patch_kernel", "attn_bwd_dkv_patch_kernel"),
])
def test_attn_bwd_neighbourhood_kernels(name, dq, dkv):
    """Grids at most 32 wide take the row kernels (dQ by query rows, dK/dV by key rows); wider grids of
    one plane the patch kernels (8 x 16 patches over LDS rectangles)."""
    import exact_attention_68_amd as A

    w = workloads.WORKLOADS[name]
    q, k, v = (t.cuda() for t in workloads.workload_qkv(w))
    mode = A.ATTN_MASK_NA3D if w.mask == "na3d" else A.ATTN_MASK_NA2D
    params = A.na3d_params(**w.na) if w.mask == "na3d" else A.na2d_params(**w.na)
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device="cuda")
    A.attn_fwd_ex(q, k, v, o, lse, w.scale, mode, params)
    do = torch.randn_like(q, dtype=torch.float32).to(torch.bfloat16)
    ws = torch.empty(A.attn_bwd_workspace_size(w.B, w.H, w.N, w.N, w.d, mode, params), dtype=torch.uint8,
                     device="cuda")
    grads = [torch.empty_like(t) for t in (q, k, v)]
    kernels, others = _split(_dispatches(lambda: A.attn_bwd(q, k, v, o, do, lse, *grads, w.scale, mode, params, ws)))
    assert len(kernels) == 2 and dq in kernels[0] and dkv in kernels[1], kernels
    assert others == [], others


def test_clamped_dilated_na2d_takes_patch_kernels():
    """Clamped windows are pushed inwards at the borders but otherwise span rad * dil either side of
    their query, so a clamped 7x7 window of dilation 2 on a 64x64 grid has the same 20-row bands as
    the wrapped one and takes the patch kernels forward and backward."""
    import exact_attention_68_amd as A

    B, H, N, d = 1, 2, 64 * 64, 32
    q, k, v = _inputs(B, H, N, d, 4)
    params = A.na2d_params(64, 64, 7, 7, 0, 0, 2, 2)
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, dtype=torch.float32, device="cuda")
    kernels, others = _split(_dispatches(
        lambda: A.attn_fwd_ex(q, k, v, o, lse, d ** -0.5, A.ATTN_MASK_NA2D, params, None)))
    assert len(kernels) == 1 and "attn_fwd_na_patch_kernel" in kernels[0], kernels
    assert others == [], others
    do = torch.randn_like(q, dtype=torch.float32).to(torch.bfloat16)
    ws = torch.empty(A.attn_bwd_workspace_size(B, H, N, N, d, A.ATTN_MASK_NA2D, params), dtype=torch.uint8,
                     device="cuda")
    grads = [torch.empty_like(t) for t in (q, k, v)]
    kernels, others = _split(_dispatches(
        lambda: A.attn_bwd(q, k, v, o, do, lse, *grads, d ** -0.5, A.ATTN_MASK_NA2D, params, ws)))
    assert len(kernels) == 2 and "attn_bwd_dq_patch_kernel" in kernels[0] and "attn_bwd_dkv_patch_kernel" in kernels[1], \
        kernels
    assert others == [], others


@pytest.mark.parametrize("gh,fwd,dq,dkv", [(15, 12, 12, 12), (16, 10, 10, 8)])
def test_na3d_dilated_row_kernel_stages(gh, fwd, dq, dkv):
    """A 5x5x5 window of dilation 2 on planes and rows. On 16 wrapped rows a work-group takes rows of one
    residue mod 2 (8-row bands): the narrow stages (10 rows, 8 for dK/dV). On 15 the dilation does not
    divide the cycle, groups stay consecutive and reach 12-row bands: the wide (12-row) stages."""
    import re

    import exact_attention_68_amd as A

    B, H, N, d = 1, 2, 10 * gh * 12, 32
    q, k, v = _inputs(B, H, N, d, 5)
    params = A.na3d_params(10, gh, 12, 5, 5, 5, 1, 1, 0, 2, 2, 1)
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, dtype=torch.float32, device="cuda")
    stage = lambda rows: re.compile(r"<32,\s*%d>" % rows)
    kernels, others = _split(_dispatches(
        lambda: A.attn_fwd_ex(q, k, v, o, lse, d ** -0.5, A.ATTN_MASK_NA3D, params, None)))
    assert len(kernels) == 1 and "attn_fwd_na_rows_kernel" in kernels[0] and stage(fwd).search(kernels[0]), kernels
    assert others == [], others
    do = torch.randn_like(q, dtype=torch.float32).to(torch.bfloat16)
    ws = torch.empty(A.attn_bwd_workspace_size(B, H, N, N, d, A.ATTN_MASK_NA3D, params), dtype=torch.uint8,
                     device="cuda")
    grads = [torch.empty_like(t) for t in (q, k, v)]
    kernels, others = _split(_dispatches(
        lambda: A.attn_bwd(q, k, v, o, do, lse, *grads, d ** -0.5, A.ATTN_MASK_NA3D, params, ws)))
    assert len(kernels) == 2, kernels
    assert "attn_bwd_dq_rows_kernel" in kernels[0] and stage(dq).search(kernels[0]), kernels
    assert "attn_bwd_dkv_rows_kernel" in kernels[1] and stage(dkv).search(kernels[1]), kernels
    assert others == [], others


@pytest.mark.parametrize("d,dil", [(64, 2), (32, 4)])
def test_na2d_dilated_takes_patch_kernels(d, dil):
    """A 7x7 window of dilation 2 or 4 on a 64x64 wrapped grid: each patch takes 8 rows and 16 columns of
    one residue per axis, whose windows reach 14 rows and 22 columns of those residues, so the d = 64
    rectangles (17 rows) and the 32-column blocks hold them."""
    import exact_attention_68_amd as A

    B, H, N = 1, 2, 64 * 64
    q, k, v = _inputs(B, H, N, d, 6)
    params = A.na2d_params(64, 64, 7, 7, 1, 1, dil, dil)
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, dtype=torch.float32, device="cuda")
    kernels, others = _split(_dispatches(
        lambda: A.attn_fwd_ex(q, k, v, o, lse, d ** -0.5, A.ATTN_MASK_NA2D, params, None)))
    assert len(kernels) == 1 and "attn_fwd_na_patch_kernel" in kernels[0], kernels
    assert others == [], others
    do = torch.randn_like(q, dtype=torch.float32).to(torch.bfloat16)
    ws = torch.empty(A.attn_bwd_workspace_size(B, H, N, N, d, A.ATTN_MASK_NA2D, params), dtype=torch.uint8,
                     device="cuda")
    grads = [torch.empty_like(t) for t in (q, k, v)]
    kernels, others = _split(_dispatches(
        lambda: A.attn_bwd(q, k, v, o, do, lse, *grads, d ** -0.5, A.ATTN_MASK_NA2D, params, ws)))
    assert len(kernels) == 2 and "attn_bwd_dq_patch_kernel" in kernels[0] and "attn_bwd_dkv_patch_kernel" in kernels[1], \
        kernels
    assert others == [], others


def test_na3d_d64_takes_row_kernel():
    """At d = 64 the forward row kernel runs with 8-row stages (one work-group per CU)."""
    import re

    import exact_attention_68_amd as A

    B, H, N, d = 1, 2, 8 * 8 * 8, 64
    q, k, v = _inputs(B, H, N, d, 7)
    params = A.na3d_params(8, 8, 8, 5, 5, 5, 1, 1, 0)
    o = torch.empty_like(q)
    kernels, others = _split(_dispatches(
        lambda: A.attn_fwd_ex(q, k, v, o, None, d ** -0.5, A.ATTN_MASK_NA3D, params, None)))
    assert len(kernels) == 1 and "attn_fwd_na_rows_kernel" in kernels[0] and re.search(r"<64,\s*8>", kernels[0]), \
        kernels
    assert others == [], others

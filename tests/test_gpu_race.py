"""Race check of the hand-managed tile rings: the pipelined library against the serial one, bit
for bit.

Key and value tiles stream through LDS rings (PhotoRoom's xformers post, the running-softmax
paragraph: K and V are read tile by tile). The kernels issue each tile's global -> LDS copy one
or more steps before the step that reads it and wait for it with hand-set vmcnt counts, outside
the compiler's tracking. libattn_serial.so is the same source built with ATTN_SERIAL_TILES=1:
every load is issued after its step's computation and awaited in full before the barrier that
publishes it, so no tile is read while any load is in flight. The arithmetic is identical, so
every output must match bit for bit; a wait count or barrier that let a step read a tile before
it landed would show as a mismatch (and, being timing-dependent, would vary between the repeated
calls of the pipelined library).

Cases: SD2.1-512 through the remainder split and without it, causal, the 64x64 wrapped window
(with its logsumexp), d = 32 (four-stage rings), d = 128, and the backward (both kernels).
"""
import ctypes

import pytest
import torch

import workloads
from parity import split_workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    from exact_attention_68_amd.build import LIB_SERIAL, ensure_built

    import exact_attention_68_amd as A

    ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return A.lib(), A._load(LIB_SERIAL)


def _p(t):
    return None if t is None else t.data_ptr()


def _fwd(lib, q, k, v, mode, scale, params, entry, want_lse):
    import exact_attention_68_amd as A

    B, H, Nq, d = q.shape
    Nkv = k.shape[2]
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device="cuda") if want_lse else None
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    pp = A._params_ptr(params)
    if entry == "attn_fwd":
        rc = lib.attn_fwd(_p(q), _p(k), _p(v), _p(o), B, H, Nq, d, scale, mode, pp, stream)
    else:
        ws = split_workspace(B, H, Nq, d, mode, params, n_kv=Nkv)
        nb = 0 if ws is None else ws.numel()
        rc = lib.attn_fwd_ex(_p(q), _p(k), _p(v), _p(o), _p(lse), B, H, Nq, Nkv, d, scale, mode, pp, _p(ws), nb,
                             stream)
    assert rc == 0, rc
    torch.cuda.synchronize()
    return o, lse


CASES = [
    ("sd21_512_selfattn", "attn_fwd_ex", False),  # remainder split: whole tiles + key-range parts + merge
    ("sd21_512_selfattn", "attn_fwd", False),     # one work-group per query tile
    ("causal_n2048", "attn_fwd", False),
    ("na2d_wrap_64x64_k7", "attn_fwd_ex", True),
    ("selfattn_n4096_d128", "attn_fwd_ex", False),
]


@pytest.mark.parametrize("name,entry,want_lse", CASES)
def test_forward_pipelined_equals_serial(libs, name, entry, want_lse):
    import exact_attention_68_amd as A

    piped, serial = libs
    w = workloads.WORKLOADS[name]
    q, k, v = (t.cuda() for t in workloads.workload_qkv(w))
    mode = {"none": A.ATTN_MASK_NONE, "causal": A.ATTN_MASK_CAUSAL, "na2d": A.ATTN_MASK_NA2D}[w.mask]
    params = A.na2d_params(**w.na) if w.mask == "na2d" else None
    print(f"[race] {name} {entry}", flush=True)
    ref_o, ref_l = _fwd(serial, q, k, v, mode, w.scale, params, entry, want_lse)
    for _ in range(3):
        o, lse = _fwd(piped, q, k, v, mode, w.scale, params, entry, want_lse)
        assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16)), f"{name}: output differs from the serial build"
        if want_lse:
            assert torch.equal(lse.view(torch.int32), ref_l.view(torch.int32)), f"{name}: logsumexp differs"


@pytest.mark.parametrize("mask", ["none", "causal"])
def test_d32_four_stage_rings_equal_serial(libs, mask):
    import exact_attention_68_amd as A

    piped, serial = libs
    q, k, v = (t.cuda() for t in workloads.make_qkv(2, 4, 3000, 32, 77))
    mode = A.ATTN_MASK_CAUSAL if mask == "causal" else A.ATTN_MASK_NONE
    ref_o, _ = _fwd(serial, q, k, v, mode, 32 ** -0.5, None, "attn_fwd", False)
    for _ in range(3):
        o, _ = _fwd(piped, q, k, v, mode, 32 ** -0.5, None, "attn_fwd", False)
        assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16))


@pytest.mark.parametrize("gh,d", [(15, 32), (16, 32), (16, 64)])
def test_na3d_dilated_rows_forward_equals_serial(libs, gh, d):
    """The forward row kernel on a 10 x gh x 12 volume, 5x5x5 window dilated by 2 on planes and rows, with its
    logsumexp: 15 wrapped rows take the wide 12-row stages, 16 the row groups of one residue (at d = 64 the
    8-row stages)."""
    import exact_attention_68_amd as A

    piped, serial = libs
    q, k, v = (t.cuda() for t in workloads.make_qkv(1, 2, 10 * gh * 12, d, 90))
    params = A.na3d_params(10, gh, 12, 5, 5, 5, 1, 1, 0, 2, 2, 1)
    ref_o, ref_l = _fwd(serial, q, k, v, A.ATTN_MASK_NA3D, d ** -0.5, params, "attn_fwd_ex", True)
    for _ in range(3):
        o, lse = _fwd(piped, q, k, v, A.ATTN_MASK_NA3D, d ** -0.5, params, "attn_fwd_ex", True)
        assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), ref_l.view(torch.int32))


@pytest.mark.parametrize("mask,d", [("none", 64), ("causal", 64), ("none", 128), ("na3d", 32), ("na3d_wide", 32),
                                   ("na3d_residue", 32)])
def test_backward_pipelined_equals_serial(libs, mask, d):
    """The tile kernels; at "na3d" (a 10x10x10 volume, 5x5x5 window) the row kernels' two-stage rings, at
    "na3d_wide" (10x15x12, dilation 2 on planes and 15 wrapped rows: 12-row bands) their wide stages, at
    "na3d_residue" (10x16x12, the same window: row groups of one residue) their strided stages."""
    import exact_attention_68_amd as A

    piped, serial = libs
    B, H, N = {"na3d": (2, 2, 1000), "na3d_wide": (1, 2, 1800), "na3d_residue": (1, 2, 1920)}.get(mask, (1, 4, 2000))
    q, k, v = (t.cuda() for t in workloads.make_qkv(B, H, N, d, 88))
    g = torch.Generator(device="cpu").manual_seed(89)
    do = torch.randn(B, H, N, d, generator=g).to(torch.bfloat16).cuda()
    mode = {"none": A.ATTN_MASK_NONE, "causal": A.ATTN_MASK_CAUSAL}.get(mask, A.ATTN_MASK_NA3D)
    params = {"na3d": A.na3d_params(10, 10, 10, 5, 5, 5, 1, 1, 0),
              "na3d_wide": A.na3d_params(10, 15, 12, 5, 5, 5, 1, 1, 0, 2, 2, 1),
              "na3d_residue": A.na3d_params(10, 16, 12, 5, 5, 5, 1, 1, 0, 2, 2, 1)}.get(mask)
    pp = A._params_ptr(params)
    o, lse = _fwd(piped, q, k, v, mode, d ** -0.5, params, "attn_fwd_ex", True)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nws = A.attn_bwd_workspace_size(B, H, N, N, d, mode, params)

    def grads(lib):
        ws = torch.full((nws,), 255, dtype=torch.uint8, device="cuda")
        out = [torch.full_like(t, float("nan")) for t in (q, k, v)]
        rc = lib.attn_bwd(_p(q), _p(k), _p(v), _p(o), _p(do), _p(lse), *[_p(t) for t in out], B, H, N, N, d,
                          d ** -0.5, mode, pp, _p(ws), nws, stream)
        assert rc == 0, rc
        torch.cuda.synchronize()
        return out

    ref = grads(serial)
    for _ in range(3):
        for name, a, b in zip(("dq", "dk", "dv"), grads(piped), ref):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{name} differs from the serial build"

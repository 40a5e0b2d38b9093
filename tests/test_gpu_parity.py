"""Parity of the HIP path against the CPU oracle, element by element, on an MI355X.

Inputs are the seeded bfloat16 tensors of workloads.py. Small cases span
several query and key tiles plus a ragged tail; the workload sizes are
compared in full where the oracle finishes in seconds and on sampled query
rows otherwise. Tolerance: |gpu - ref| <= 4e-3 * max(1, |ref|) + 2e-3.

Both C entry points are covered: attn_fwd (one work-group per query tile) and
attn_fwd_ws (unmasked problems of less than two tiles per CU: a round of whole
tiles plus the remaining tiles cut into key-range parts, merged by a second
kernel through the workspace).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check_case, compare, run_gpu, split_workspace, to_f64, workload_params

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    from exact_attention_68_amd.build import ensure_built

    ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"


def _qkv(B, H, N, d, seed, q_gain=1.0):
    return workloads.make_qkv(B, H, N, d, seed, q_gain)


# ---------------------------------------------------------------- workloads
ENTRIES = ["attn_fwd", "attn_fwd_ws"]


@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("name", ["single_head_n256", "sd21_512_selfattn", "causal_n2048", "na2d_wrap_64x64_k7"])
def test_workload_full(name, entry):
    w = workloads.WORKLOADS[name]
    q, k, v = workloads.workload_qkv(w)
    check_case(q, k, v, w.scale, w.mask, workload_params(w), what=name, entry=entry)


@pytest.mark.parametrize("entry", ENTRIES)
def test_sd21_768_sampled_rows(entry):
    w = workloads.WORKLOADS["sd21_768_selfattn"]
    q, k, v = workloads.workload_qkv(w)
    rng = np.random.default_rng(7)
    rows = sorted({0, 1, 63, 64, 127, 128, w.N - 1, w.N - 2, *rng.choice(w.N, 250, replace=False).tolist()})
    check_case(q, k, v, w.scale, w.mask, rows=rows, what=w.name, entry=entry)



# ---------------------------------------------------------------- remainder split (attn_fwd_ws)
def _splits(B, H, N, d):
    import exact_attention_68_amd as A

    return A.attn_fwd_workspace_size(B, H, N, d, A.ATTN_MASK_NONE) > 0


@pytest.mark.parametrize("B,H,N,d", [
    (1, 2, 1000, 64),    # 16 tiles of 8 key tiles: every tile in parts
    (2, 3, 1500, 32),    # ragged query and key tails
    (1, 3, 777, 64),     # parts of 2 and 3 key tiles
    (3, 1, 2048, 32),
    (1, 1, 4096 + 77, 64),
    (2, 5, 4096, 64),    # the SD2.1 512x512 shape: 256 whole tiles, 64 tiles in 4 parts; every row
])
def test_split_shapes(B, H, N, d):
    assert _splits(B, H, N, d), "shape expected to run split on this device"
    q, k, v = _qkv(B, H, N, d, 8000 + N + d)
    check_case(q, k, v, 1 / math.sqrt(d), "none", what=f"split B{B}H{H}N{N}d{d}", entry="attn_fwd_ws")


@pytest.mark.parametrize("scale,q_gain", [(0.0, 1.0), (-0.2, 1.0), (0.125, 2.0), (1e-3, 1.0)])
def test_split_scales_and_peaky_rows(scale, q_gain):
    q, k, v = _qkv(1, 2, 1000, 64, 8100, q_gain)
    assert _splits(1, 2, 1000, 64)
    check_case(q, k, v, scale, "none", what=f"split scale {scale} gain {q_gain}", entry="attn_fwd_ws")


def test_split_deterministic():
    """Parts are merged in a fixed order: repeated calls on one workspace agree bit for bit."""
    import exact_attention_68_amd as A

    B, H, N, d = 2, 5, 4096, 64
    q, k, v = (t.cuda() for t in _qkv(B, H, N, d, 8200))
    ws = split_workspace(B, H, N, d, A.ATTN_MASK_NONE)
    assert ws is not None
    outs = []
    for _ in range(3):
        o = torch.empty_like(q)
        A.attn_fwd_ws(q, k, v, o, 0.125, A.ATTN_MASK_NONE, None, ws)
        torch.cuda.synchronize()
        outs.append(o)
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_split_concurrent_streams_own_workspaces():
    """Two streams, each with its own workspace, run split launches at the same time: a split tile's
    parts meet through the arrival counters of their own workspace only, so both streams' outputs equal
    the serial ones bit for bit (a counter shared across calls would merge a tile early or never)."""
    import exact_attention_68_amd as A

    B, H, N, d = 2, 5, 4096, 64
    ins = [[t.cuda() for t in _qkv(B, H, N, d, 8250 + i)] for i in range(2)]
    wss = [split_workspace(B, H, N, d, A.ATTN_MASK_NONE) for _ in range(2)]
    assert all(ws is not None for ws in wss)
    ref = []
    for (q, k, v), ws in zip(ins, wss):
        o = torch.empty_like(q)
        A.attn_fwd_ws(q, k, v, o, 0.125, A.ATTN_MASK_NONE, None, ws)
        ref.append(o)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.empty_like(ins[i][0]) for _ in range(8)] for i in range(2)]
    for it in range(8):  # interleaved launches: the two streams' kernels overlap on the device
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                q, k, v = ins[i]
                A.attn_fwd_ws(q, k, v, outs[i][it], 0.125, A.ATTN_MASK_NONE, None, wss[i])
    torch.cuda.synchronize()
    for i in range(2):
        for it in range(8):
            assert torch.equal(outs[i][it], ref[i]), f"stream {i}, call {it} differs from the serial output"


def test_split_workspace_reused_across_shapes():
    """One workspace, sized for the largest problem, serves other sizes and head sizes in turn."""
    import exact_attention_68_amd as A

    shapes = [(2, 5, 4096, 64), (1, 2, 1000, 64), (2, 3, 1500, 32), (2, 5, 4096, 64)]
    need = max(A.attn_fwd_workspace_size(*s, A.ATTN_MASK_NONE) for s in shapes)
    ws = torch.full((need,), 255, dtype=torch.uint8, device="cuda")
    for i, (B, H, N, d) in enumerate(shapes):
        q, k, v = _qkv(B, H, N, d, 8300 + i)
        o = torch.empty(B, H, N, d, dtype=torch.bfloat16, device="cuda")
        print(f"[parity] reuse B{B} H{H} N{N} d{d}", flush=True)
        A.attn_fwd_ws(q.cuda(), k.cuda(), v.cuda(), o, 1 / math.sqrt(d), A.ATTN_MASK_NONE, None, ws)
        torch.cuda.synchronize()
        rows = list(range(0, N, max(1, N // 300)))
        ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), 1 / math.sqrt(d), rows=rows)
        compare(to_f64(o)[:, :, rows], ref, f"reuse {i}")


def test_split_rejects_bad_workspace():
    import exact_attention_68_amd as A

    B, H, N, d = 1, 2, 1000, 64
    q, k, v = (t.cuda() for t in _qkv(B, H, N, d, 8400))
    o = torch.full_like(q, 3.0)
    need = A.attn_fwd_workspace_size(B, H, N, d)
    assert need > 0
    big = torch.zeros(need + 512, dtype=torch.uint8, device="cuda")
    lib = A.lib()
    p = [t.data_ptr() for t in (q, k, v, o)]
    assert lib.attn_fwd_ws(*p, B, H, N, d, 0.125, 0, None, None, 0, None) == A.ATTN_ERR_WORKSPACE
    assert lib.attn_fwd_ws(*p, B, H, N, d, 0.125, 0, None, big.data_ptr(), need - 1, None) == A.ATTN_ERR_WORKSPACE
    assert lib.attn_fwd_ws(*p, B, H, N, d, 0.125, 0, None, big.data_ptr() + 16, need, None) == A.ATTN_ERR_WORKSPACE
    assert lib.attn_fwd_ws(*p, B, H, N, d, 0.125, 0, None, p[3], need, None) == A.ATTN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(o == 3.0)
    assert int(big.count_nonzero()) == 0


def test_split_not_used_where_it_cannot_help():
    import exact_attention_68_amd as A

    assert A.attn_fwd_workspace_size(2, 5, 9216, 64) == 0          # two and more rounds of tiles
    assert A.attn_fwd_workspace_size(4, 16, 2048, 64, A.ATTN_MASK_CAUSAL) == 0
    assert A.attn_fwd_workspace_size(1, 1, 256, 64) == 0           # 2 tiles of 2 key tiles
    assert A.attn_fwd_workspace_size(2, 4, 4096, 32, A.ATTN_MASK_NA2D, A.na2d_params(64, 64, 7, 7)) == 0


# ---------------------------------------------------------------- edge shapes
@pytest.mark.parametrize("d", [32, 64])
@pytest.mark.parametrize("mask", ["none", "causal"])
@pytest.mark.parametrize("N", [1, 17, 64, 100, 128, 255, 257, 320])
def test_edge_shapes(N, mask, d):
    q, k, v = _qkv(1, 2, N, d, 1000 + N + d)
    check_case(q, k, v, 1 / math.sqrt(d), mask, what=f"edge N{N}")


# Rows up to score std 2 (scale 0.125 with Q doubled, or scale 0.25) meet the parity bound.
@pytest.mark.parametrize("scale,q_gain", [(0.0, 1.0), (-0.2, 1.0), (0.125, 2.0), (0.25, 1.0), (1e-3, 1.0)])
@pytest.mark.parametrize("mask", ["none", "causal"])
def test_scales_and_peaky_rows(scale, q_gain, mask):
    q, k, v = _qkv(2, 3, 300, 64, 2000, q_gain)
    check_case(q, k, v, scale, mask, what=f"scale {scale} gain {q_gain}")


# Sharper rows: score std 4 (Q x 4 at scale 1/8) and 8 (scale 1 at d = 64). With so much of a row's
# weight on few keys, rounding the probabilities to bfloat16 can move single outputs past the
# parity bound (tests/test_kernel_model.py: the modelled arithmetic reaches 1.16 of it on seed
# 2003 and 1.07 on seed 2000 at scale 1). These rows are held to the bound derived from that
# arithmetic (parity.derived_tolerance), element by element.
@pytest.mark.parametrize("scale,q_gain,seed", [(0.125, 4.0, 2000), (0.125, 4.0, 2003), (1.0, 1.0, 2000),
                                               (1.0, 1.0, 2001), (-1.0, 1.0, 2002)])
@pytest.mark.parametrize("mask", ["none", "causal"])
@pytest.mark.parametrize("entry", ENTRIES)
def test_sharp_rows_derived_bound(scale, q_gain, seed, mask, entry):
    q, k, v = _qkv(2, 3, 300, 64, seed, q_gain)
    check_case(q, k, v, scale, mask, what=f"sharp rows scale {scale} gain {q_gain} seed {seed}", entry=entry,
               derived=True)


@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("mask", ["none", "causal"])
def test_rescale_path_planted_keys(mask, entry):
    """Keys whose scores climb by 30 to 60 (base 2) from one key tile to the next, far past
    the 2^20 row-sum guard: every row's reference maximum has to move several times (the
    rare slow path of a step), for both the unmasked and the causal loop."""
    B, H, N, d = 1, 2, 1000, 64
    q, k, v = _qkv(B, H, N, d, 8500)
    q = q.float().abs() + 0.5                                # positive queries
    grow = (1.0 + 2.0 * (torch.arange(N) // 128)).view(1, 1, N, 1)
    k = (k.float().abs() + 0.25) * grow                      # scores grow tile by tile
    check_case(q.to(torch.bfloat16), k.to(torch.bfloat16), v, 0.25, mask, what="planted keys", entry=entry)


@pytest.mark.parametrize("mode,geo", [
    ("na3d", (8, 8, 8, 5, 5, 5, 1, 0, 1, 1, 1, 1)),   # the row kernel (a grid 8 wide)
    ("na2d", (24, 48, 7, 7, 0, 1, 1, 1)),             # the patch kernel
])
def test_rescale_path_planted_keys_windows(mode, geo):
    """Keys whose scores climb by about 30 (base 2) from one grid row to the next (rows clamped, so
    a walk meets them in rising order): the row kernel's walk and the patch kernel's steps move the
    reference maximum past the 2^20 row-sum guard again and again."""
    import exact_attention_68_amd as A

    params = A.na3d_params(*geo) if mode == "na3d" else A.na2d_params(*geo)
    H, W = (geo[1], geo[2]) if mode == "na3d" else (geo[0], geo[1])
    N = geo[0] * geo[1] * (geo[2] if mode == "na3d" else 1)
    q, k, v = _qkv(1, 2, N, 32, 8600)
    q = q.float().abs() + 0.5                                # positive queries
    y = (torch.arange(N) // W) % H                           # each key's grid row
    k = (k.float().abs() + 0.25) * (1.0 + 2.0 * y).view(1, 1, N, 1)
    check_case(q.to(torch.bfloat16), k.to(torch.bfloat16), v, 0.25, mode, params, what=f"planted keys {mode}",
               entry="attn_fwd_ex")


# ---------------------------------------------------------------- 2D neighbourhood
def test_na2d_issue_example_5x5():
    """NATTEN issue 142: q = k = 1, v one-hot at the top-left pixel, 5x5 grid, kernel 3, wrap."""
    import exact_attention_68_amd as A

    d = 32
    q = torch.ones(1, 1, 25, d, dtype=torch.bfloat16)
    k = torch.ones(1, 1, 25, d, dtype=torch.bfloat16)
    v = torch.zeros(1, 1, 25, d, dtype=torch.bfloat16)
    v[0, 0, 0, :] = 1
    o = run_gpu(q, k, v, 1 / math.sqrt(d), A.ATTN_MASK_NA2D, A.na2d_params(5, 5, 3, 3, 1, 1))
    got = to_f64(o)[0, 0, :, 0].reshape(5, 5)
    printed = np.loadtxt(__import__("pathlib").Path(__file__).parent / "golden" / "na2d_wrap_5x5_k3.txt")
    exact = np.where(printed > 0, 1 / 9, 0.0)
    compare(got, exact, "5x5 wrap example")
    assert np.all(got[printed == 0] == 0.0)


@pytest.mark.parametrize("d", [32, 64])
@pytest.mark.parametrize("gh,gw,kh,kw,wh,ww", [
    (8, 9, 5, 5, 1, 1),
    (5, 5, 3, 3, 1, 1),
    (7, 13, 3, 5, 0, 0),
    (10, 6, 5, 3, 1, 0),
    (6, 10, 3, 7, 0, 1),
    (5, 7, 5, 7, 1, 1),     # window = grid: full attention
    (33, 17, 9, 3, 1, 1),   # band crosses tiles and wraps
    (20, 20, 1, 1, 1, 1),   # self only
    (3, 200, 3, 11, 1, 1),  # short, wide grid: band is the whole sequence
    (64, 64, 7, 7, 0, 0),
    (16, 32, 5, 5, 0, 1),   # width 32: one 32-column phase per grid row (bit-mask path)
    (8, 96, 5, 7, 1, 1),    # width 96: three phases
    (6, 128, 3, 9, 1, 0),   # width 128: four phases, clamped columns
    (5, 128, 5, 127, 0, 1), # window almost the whole row
])
def test_na2d_shapes(gh, gw, kh, kw, wh, ww, d):
    import exact_attention_68_amd as A

    N = gh * gw
    q, k, v = _qkv(1, 2, N, d, 3000 + N + kh)
    check_case(q, k, v, 1 / math.sqrt(d), "na2d", A.na2d_params(gh, gw, kh, kw, wh, ww),
               what=f"na2d {gh}x{gw} k{kh}x{kw} wrap{wh}{ww}")


# ---------------------------------------------------------------- properties
def test_causal_first_row_is_exact():
    q, k, v = _qkv(2, 2, 200, 64, 4000)
    import exact_attention_68_amd as A

    o = run_gpu(q, k, v, 0.125, A.ATTN_MASK_CAUSAL)
    assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])


def test_deterministic_bitwise():
    import exact_attention_68_amd as A

    q, k, v = _qkv(2, 5, 1000, 64, 5000)
    a = run_gpu(q, k, v, 0.125, A.ATTN_MASK_NONE)
    b = run_gpu(q, k, v, 0.125, A.ATTN_MASK_NONE)
    assert torch.equal(a, b)


@pytest.mark.parametrize("entry", ENTRIES)
def test_no_device_allocation_and_side_stream(entry):
    import exact_attention_68_amd as A

    B, H, N, d = 1, 2, 1000, 64
    q, k, v = (t.cuda() for t in _qkv(B, H, N, d, 6000))
    o = torch.empty_like(q)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ws = split_workspace(B, H, N, d, A.ATTN_MASK_NONE) if entry == "attn_fwd_ws" else None
    s.synchronize()
    before = torch.cuda.memory_allocated()
    with torch.cuda.stream(s):
        if entry == "attn_fwd":
            A.attn_fwd(q, k, v, o, 0.125, A.ATTN_MASK_NONE)
        else:
            A.attn_fwd_ws(q, k, v, o, 0.125, A.ATTN_MASK_NONE, None, ws)
    s.synchronize()
    assert torch.cuda.memory_allocated() == before
    ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), 0.125)
    compare(to_f64(o), ref, f"side stream {entry}")


def test_attention_convenience_uses_split_path():
    import exact_attention_68_amd as A

    q, k, v = (t.cuda() for t in _qkv(1, 2, 1000, 64, 6100))
    o = A.attention(q, k, v)
    torch.cuda.synchronize()
    ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), 1 / 8)
    compare(to_f64(o), ref, "attention()")


def test_rejected_arguments_leave_output_untouched():
    import exact_attention_68_amd as A

    q, k, v = (t.cuda() for t in _qkv(1, 1, 64, 64, 7000))
    o = torch.full_like(q, 3.0)
    lib = A.lib()
    p = [t.data_ptr() for t in (q, k, v, o)]
    assert lib.attn_fwd(*p, 1, 1, 64, 64, 0.1, 9, None, None) == A.ATTN_ERR_INVALID_ARG
    assert lib.attn_fwd(*p, 1, 1, 64, 48, 0.1, 0, None, None) == A.ATTN_ERR_UNSUPPORTED
    assert lib.attn_fwd(*p, 1, 1, 64, 64, float("nan"), 0, None, None) == A.ATTN_ERR_INVALID_ARG
    bad = A.na2d_params(8, 8, 4, 3)
    import ctypes
    assert lib.attn_fwd(*p, 1, 1, 64, 64, 0.1, 2, ctypes.cast(ctypes.pointer(bad), ctypes.c_void_p),
                        None) == A.ATTN_ERR_PARAMS
    assert lib.attn_fwd(p[0], p[1], p[2], p[0], 1, 1, 64, 64, 0.1, 0, None, None) == A.ATTN_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.all(o == 3.0)

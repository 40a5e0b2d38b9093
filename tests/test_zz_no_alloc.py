"""attn_fwd_ex_static, the entry point that allocates nothing, against attn_fwd_ex.

attn_fwd_ex_static runs attn_fwd_ex's kernels with the split workspace in the library's
static device array instead of a caller buffer. Two calls in a row on one stream (the
second smaller, so it reuses a prefix of the array the first call left filled) must give
exactly attn_fwd_ex's output and logsumexp, and the oracle's within the parity bound.
"""
import ctypes

import pytest
import torch

import oracle
import workloads
from parity import compare, split_workspace, to_f64

pytestmark = pytest.mark.gpu


def _run_ex(A, q, k, v, scale, static):
    B, H, Nq, d = q.shape
    Nkv = k.shape[2]
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    lib = A.lib()
    if static:
        before = torch.cuda.memory_allocated()
        rc = lib.attn_fwd_ex_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Nq,
                                    Nkv, d, scale, A.ATTN_MASK_NONE, None, stream)
        assert torch.cuda.memory_allocated() == before
    else:
        ws = split_workspace(B, H, Nq, d, A.ATTN_MASK_NONE, n_kv=Nkv)
        nb = 0 if ws is None else ws.numel()
        rc = lib.attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Nq, Nkv,
                             d, scale, A.ATTN_MASK_NONE, None, None if ws is None else ws.data_ptr(), nb, stream)
    assert rc == A.ATTN_OK, A.attn_status_string(rc)
    torch.cuda.synchronize()
    return o, lse


def test_static_scratch_matches_attn_fwd_ex_twice():
    from exact_attention_68_amd.build import ensure_built

    ensure_built()
    import exact_attention_68_amd as A

    # SD2.1-512 (320 query tiles: 64 of them split into key-range parts), then a smaller
    # cross-attention problem at d = 128 that also splits
    shapes = [(2, 5, 4096, 4096, 64, 0.125), (1, 3, 1000, 700, 128, 128 ** -0.5)]
    for i, (B, H, Nq, Nkv, d, scale) in enumerate(shapes):
        print(f"[no-alloc] call {i}: B{B} H{H} Nq{Nq} Nkv{Nkv} d{d}", flush=True)
        assert A.attn_fwd_ex_workspace_size(B, H, Nq, Nkv, d, A.ATTN_MASK_NONE) > 0, "the case must split"
        q, k, v = (t.cuda() for t in workloads.make_qkv_cross(B, H, Nq, Nkv, d, 12000 + i))
        o_s, l_s = _run_ex(A, q, k, v, scale, static=True)
        o_e, l_e = _run_ex(A, q, k, v, scale, static=False)
        assert torch.equal(o_s.view(torch.int16), o_e.view(torch.int16)), "output differs from attn_fwd_ex"
        assert torch.equal(l_s.view(torch.int32), l_e.view(torch.int32)), "logsumexp differs from attn_fwd_ex"
        rows = list(range(0, Nq, max(1, Nq // 97))) + [Nq - 1]
        ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), scale, rows=rows)
        compare(to_f64(o_s)[:, :, rows], ref, f"attn_fwd_ex_static call {i}")

"""Shared helpers for the GPU parity tests: run the HIP path, run the oracle, compare."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads

# Per-element bound for a bfloat16 output with float32 accumulation against the
# unrounded float64 oracle: |gpu - ref| <= 4e-3 * max(1, |ref|) + 2e-3.
REL_TOL = 4e-3
ABS_TOL = 2e-3


def tolerance(ref: np.ndarray) -> np.ndarray:
    return REL_TOL * np.maximum(1.0, np.abs(ref)) + ABS_TOL


def compare(got: np.ndarray, ref: np.ndarray, what: str) -> float:
    """Assert got is within tolerance of ref everywhere; returns the worst err/tol ratio."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    ratio = np.abs(got - ref) / tolerance(ref)
    worst = float(ratio.max()) if ratio.size else 0.0
    if worst > 1.0:
        idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        raise AssertionError(f"{what}: {int((ratio > 1).sum())} of {ratio.size} elements out of tolerance; "
                             f"worst err/tol {worst:.3f} at {idx}: got {got[idx]}, ref {ref[idx]}")
    return worst


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def oracle_na2d(p) -> "oracle.NA2D | None":
    if p is None:
        return None
    return oracle.NA2D(p.grid_h, p.grid_w, p.kernel_h, p.kernel_w, bool(p.wrap_h), bool(p.wrap_w))


def split_workspace(B, H, N, d, mask_mode, params=None):
    """A fresh workspace for attn_fwd_ws (None when the problem needs none), filled with 0xff bytes
    (NaN bit patterns): the library must not depend on its initial content."""
    import exact_attention_68_amd as A

    n = A.attn_fwd_workspace_size(B, H, N, d, mask_mode, params)
    return torch.full((n,), 255, dtype=torch.uint8, device="cuda") if n else None


def run_gpu(q, k, v, scale, mask_mode, params=None, entry="attn_fwd"):
    """Output of the HIP path through the C ABI entry point `entry` (attn_fwd or attn_fwd_ws)."""
    import exact_attention_68_amd as A

    dq, dk, dv = (t.to("cuda") for t in (q, k, v))
    o = torch.empty_like(dq)
    if entry == "attn_fwd":
        A.attn_fwd(dq, dk, dv, o, scale, mask_mode, params)
    else:
        ws = split_workspace(*dq.shape, mask_mode, params)
        A.attn_fwd_ws(dq, dk, dv, o, scale, mask_mode, params, ws)
    torch.cuda.synchronize()
    return o


def check_case(q, k, v, scale, mask: str, params=None, rows=None, what="", entry="attn_fwd") -> float:
    """Run the HIP path and the oracle on the same bf16 inputs and compare (all rows or `rows`)."""
    import exact_attention_68_amd as A

    mode = {"none": A.ATTN_MASK_NONE, "causal": A.ATTN_MASK_CAUSAL, "na2d": A.ATTN_MASK_NA2D}[mask]
    print(f"[parity] {entry} {what} B{q.shape[0]} H{q.shape[1]} N{q.shape[2]} d{q.shape[3]} mask={mask} "
          f"scale={scale}", flush=True)
    o = run_gpu(q, k, v, scale, mode, params, entry)
    got = to_f64(o)
    ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), scale, mask, oracle_na2d(params), rows=rows)
    if rows is not None:
        got = got[:, :, rows]
    return compare(got, ref, what or mask)


def workload_params(w: workloads.Workload):
    import exact_attention_68_amd as A

    return A.na2d_params(**w.na2d) if w.mask == "na2d" else None

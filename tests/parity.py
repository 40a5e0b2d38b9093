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


def compare(got: np.ndarray, ref: np.ndarray, what: str, tol: np.ndarray | None = None) -> float:
    """Assert got is within tolerance of ref everywhere (the parity bound unless `tol` is
    given); returns the worst err/tol ratio."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    ratio = np.abs(got - ref) / (tolerance(ref) if tol is None else tol)
    worst = float(ratio.max()) if ratio.size else 0.0
    if worst > 1.0:
        idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        raise AssertionError(f"{what}: {int((ratio > 1).sum())} of {ratio.size} elements out of tolerance; "
                             f"worst err/tol {worst:.3f} at {idx}: got {got[idx]}, ref {ref[idx]}")
    return worst


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def oracle_na(p):
    """The oracle's window for an attn_na2d_params_t / attn_na3d_params_t (None for no window)."""
    if p is None:
        return None
    if hasattr(p, "grid_d"):
        return oracle.NA3D(p.grid_d, p.grid_h, p.grid_w, p.kernel_d, p.kernel_h, p.kernel_w,
                           bool(p.wrap_d), bool(p.wrap_h), bool(p.wrap_w), p.dil_d, p.dil_h, p.dil_w)
    return oracle.NA2D(p.grid_h, p.grid_w, p.kernel_h, p.kernel_w, bool(p.wrap_h), bool(p.wrap_w), p.dil_h, p.dil_w)


def split_workspace(B, H, N, d, mask_mode, params=None, n_kv=None):
    """A fresh workspace for attn_fwd_ws / attn_fwd_ex (None when the problem needs none), filled
    with 0xff bytes (NaN bit patterns): the library must not depend on its initial content."""
    import exact_attention_68_amd as A

    n = A.attn_fwd_ex_workspace_size(B, H, N, N if n_kv is None else n_kv, d, mask_mode, params)
    return torch.full((n,), 255, dtype=torch.uint8, device="cuda") if n else None


def run_gpu(q, k, v, scale, mask_mode, params=None, entry="attn_fwd", want_lse=False):
    """Output (and, for attn_fwd_ex with want_lse, the logsumexp) of the HIP path through the C ABI
    entry point `entry` (attn_fwd, attn_fwd_ws or attn_fwd_ex)."""
    import exact_attention_68_amd as A

    dq, dk, dv = (t.to("cuda") for t in (q, k, v))
    o = torch.empty_like(dq)
    lse = None
    if entry == "attn_fwd":
        A.attn_fwd(dq, dk, dv, o, scale, mask_mode, params)
    elif entry == "attn_fwd_ws":
        ws = split_workspace(*dq.shape, mask_mode, params)
        A.attn_fwd_ws(dq, dk, dv, o, scale, mask_mode, params, ws)
    else:
        B, H, Nq, d = dq.shape
        ws = split_workspace(B, H, Nq, d, mask_mode, params, n_kv=dk.shape[2])
        if want_lse:
            lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device="cuda")
        A.attn_fwd_ex(dq, dk, dv, o, lse, scale, mask_mode, params, ws)
    torch.cuda.synchronize()
    return (o, lse) if want_lse else o


MASK_MODES = {"none": 0, "causal": 1, "na2d": 2, "na3d": 3}

# logsumexp: the row sum of bfloat16-rounded probabilities is within 2^-8 (relative) of the
# exact sum, so log l is within log(1 + 2^-8) = 3.9e-3; the float32 scores, exp2 and log2
# add far less. Bound: |gpu - ref| <= 6e-3 + 1e-5 * |ref|.
def lse_tolerance(ref: np.ndarray) -> np.ndarray:
    return 6e-3 + 1e-5 * np.abs(ref)


def derived_tolerance(q, k, v, scale, mask, na, ref) -> np.ndarray:
    """Per-element tolerance for rows sharper than the benchmark's: the larger of the parity
    bound and the bound derived from the kernel's arithmetic (bfloat16 probabilities whose row sum
    is taken of the rounded values, bfloat16 output; kernel_model.derived_bound)."""
    from kernel_model import derived_bound

    p = oracle.probs(q, k, scale, mask, na)
    tol = np.empty_like(ref)
    for b in range(ref.shape[0]):
        for h in range(ref.shape[1]):
            tol[b, h] = np.maximum(tolerance(ref[b, h]), derived_bound(p[b, h], v[b, h], ref[b, h]))
    return tol


def check_case(q, k, v, scale, mask: str, params=None, rows=None, what="", entry="attn_fwd",
               want_lse=None, derived=False) -> float:
    """Run the HIP path and the oracle on the same bf16 inputs and compare (all rows or `rows`).
    With attn_fwd_ex the logsumexp is compared too (unless want_lse is False). With derived=True
    the output bound is derived_tolerance (all rows only); the worst ratio against the parity
    bound is printed as well."""
    mode = MASK_MODES[mask]
    want_lse = entry == "attn_fwd_ex" if want_lse is None else want_lse
    print(f"[parity] {entry} {what} B{q.shape[0]} H{q.shape[1]} Nq{q.shape[2]} Nkv{k.shape[2]} d{q.shape[3]} "
          f"mask={mask} scale={scale}", flush=True)
    res = run_gpu(q, k, v, scale, mode, params, entry, want_lse)
    o, lse = res if want_lse else (res, None)
    got = to_f64(o)
    ref, ref_lse = oracle.attention(to_f64(q), to_f64(k), to_f64(v), scale, mask, oracle_na(params), rows=rows,
                                    return_lse=True)
    if rows is not None:
        got = got[:, :, rows]
    tol = None
    if derived:
        assert rows is None, "the derived bound is computed for whole heads"
        tol = derived_tolerance(to_f64(q), to_f64(k), to_f64(v), scale, mask, oracle_na(params), ref)
        ns = float((np.abs(got - ref) / tolerance(ref)).max())
        print(f"[parity] {what}: worst err / parity bound {ns:.3f}", flush=True)
    worst = compare(got, ref, what or mask, tol)
    if want_lse:
        g = lse.cpu().numpy().astype(np.float64)
        if rows is not None:
            g = g[:, :, rows]
        assert np.all(np.isfinite(g)), f"{what}: non-finite logsumexp"
        ratio = np.abs(g - ref_lse) / lse_tolerance(ref_lse)
        if ratio.max() > 1.0:
            idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
            raise AssertionError(f"{what}: logsumexp {int((ratio > 1).sum())} of {ratio.size} out of tolerance; "
                                 f"worst err/tol {ratio.max():.3f} at {idx}: got {g[idx]}, ref {ref_lse[idx]}")
        worst = max(worst, float(ratio.max()))
    return worst


def workload_params(w: workloads.Workload):
    import exact_attention_68_amd as A

    if w.mask == "na2d":
        return A.na2d_params(**w.na)
    if w.mask == "na3d":
        return A.na3d_params(**w.na)
    return None


# ---------------------------------------------------------------- backward
# Per-element bound of the GPU gradients, derived from the arithmetic of attn_bwd (first order).
# The backward recomputes P = exp(scale s - LSE) from the logsumexp it is given (off by eL, so P is
# off by that factor per row), takes D = rowsum(dO * O) from the bf16 O it is given (off by dD_i,
# computed exactly below), rounds dS (and P for dV) to bf16 as MFMA operands (2^-8 relative) and
# rounds the gradients to bf16 (2^-8 relative):
#   |d(dS)_ij| <= P_ij (eL |dP_ij - D_i| + |dD_i|) + 2^-8 |dS_ij|
#   |d(dQ)|    <= |scale| |d(dS)| |K| + 2^-8 |dQ|,   |d(dK)| <= |scale| |d(dS)|^T |Q| + 2^-8 |dK|
#   |d(dV)|    <= (eL + 2^-8) P^T |dO| + 2^-8 |dV|
# The tests allow 1.25 x this bound plus 1e-4 (fp32 sums and exp2).
BF16_U = 2.0 ** -8


def bf16_round(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)


def bwd_reference(q, k, v, do, scale, mask="none", na=None, o_used=None, lse_err=2.0 ** -22):
    """Oracle gradients and per-element tolerances (float64 arrays shaped like q, k, v) for a backward
    given the output o_used (default: the exact output rounded to bf16) and a logsumexp within lse_err."""
    grads = oracle.attention_backward(q, k, v, do, scale, mask, na)
    p = oracle.probs(q, k, scale, mask, na)
    o = oracle.attention(q, k, v, scale, mask, na)
    o_used = bf16_round(o) if o_used is None else o_used
    dp = do @ np.swapaxes(v, -1, -2)
    dd = np.sum(p * dp, axis=-1, keepdims=True)
    ds = p * (dp - dd)
    d_delta = np.abs(np.sum(do * (o_used - o), axis=-1, keepdims=True))
    dds = p * (lse_err * np.abs(dp - dd) + d_delta) + BF16_U * np.abs(ds)
    tq = abs(scale) * (dds @ np.abs(k)) + BF16_U * np.abs(grads[0])
    tk = abs(scale) * (np.swapaxes(dds, -1, -2) @ np.abs(q)) + BF16_U * np.abs(grads[1])
    tv = (lse_err + BF16_U) * (np.swapaxes(p, -1, -2) @ np.abs(do)) + BF16_U * np.abs(grads[2])
    return grads, tuple(1.25 * t + 1e-4 for t in (tq, tk, tv))


def run_gpu_bwd(q, k, v, do, scale, mask_mode, o=None, lse=None, params=None):
    """attn_bwd on the device; o and lse default to the GPU forward's (attn_fwd_ex). Returns
    (dq, dk, dv, o, lse) on the device."""
    import exact_attention_68_amd as A

    dq_, dk_, dv_, do_ = (t.to("cuda") for t in (q, k, v, do))
    B, H, Nq, d = dq_.shape
    Nkv = dk_.shape[2]
    if o is None:
        o = torch.empty_like(dq_)
        lse = torch.empty(B, H, Nq, dtype=torch.float32, device="cuda")
        ws = split_workspace(B, H, Nq, d, mask_mode, params, n_kv=Nkv)
        A.attn_fwd_ex(dq_, dk_, dv_, o, lse, scale, mask_mode, params, ws)
    else:
        o, lse = o.to("cuda"), lse.to("cuda")
    wsb = torch.full((A.attn_bwd_workspace_size(B, H, Nq, Nkv, d, mask_mode, params),), 255, dtype=torch.uint8,
                     device="cuda")
    gq, gk, gv = torch.empty_like(dq_), torch.empty_like(dk_), torch.empty_like(dv_)
    A.attn_bwd(dq_, dk_, dv_, o, do_, lse, gq, gk, gv, scale, mask_mode, params, wsb)
    torch.cuda.synchronize()
    return gq, gk, gv, o, lse


def check_bwd_case(q, k, v, do, scale, mask: str, what="", pipeline=False, params=None) -> float:
    """GPU gradients against the oracle. By default attn_bwd gets the oracle's output (rounded to bf16)
    and logsumexp (fp32), so the bound covers the backward alone; with pipeline=True it gets the GPU
    forward's, and the bound takes the forward's output error and logsumexp tolerance as given."""
    print(f"[parity-bwd] {what} B{q.shape[0]} H{q.shape[1]} Nq{q.shape[2]} Nkv{k.shape[2]} d{q.shape[3]} mask={mask} "
          f"scale={scale} pipeline={pipeline}", flush=True)
    qf, kf, vf, gf = (to_f64(t) for t in (q, k, v, do))
    na = oracle_na(params)
    if pipeline:
        gq, gk, gv, o, _ = run_gpu_bwd(q, k, v, do, scale, MASK_MODES[mask], params=params)
        ref, tol = bwd_reference(qf, kf, vf, gf, scale, mask, na, o_used=to_f64(o), lse_err=6e-3)
    else:
        o, lse = oracle.attention(qf, kf, vf, scale, mask, na, return_lse=True)
        o_b = torch.from_numpy(o.astype(np.float32)).to(torch.bfloat16)
        lse_f = torch.from_numpy(lse.astype(np.float32))
        gq, gk, gv, _, _ = run_gpu_bwd(q, k, v, do, scale, MASK_MODES[mask], o_b, lse_f, params)
        ref, tol = bwd_reference(qf, kf, vf, gf, scale, mask, na, o_used=to_f64(o_b))
    worst = 0.0
    for name, g, r, t in zip(("dq", "dk", "dv"), (gq, gk, gv), ref, tol):
        gv_ = to_f64(g)
        assert np.all(np.isfinite(gv_)), f"{what}: non-finite {name}"
        ratio = np.abs(gv_ - r) / t
        if ratio.max() > 1.0:
            idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
            raise AssertionError(f"{what}: {name} {int((ratio > 1).sum())} of {ratio.size} out of tolerance; worst "
                                 f"err/tol {ratio.max():.3f} at {idx}: got {gv_[idx]}, ref {r[idx]}, tol {t[idx]}")
        worst = max(worst, float(ratio.max()))
    print(f"[parity-bwd] {what}: worst err/tol {worst:.3f}", flush=True)
    return worst

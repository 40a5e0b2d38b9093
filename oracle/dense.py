"""CPU oracle for exact softmax attention, in float64 NumPy.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module. The product path (the
HIP library and its Python binding) never calls it and shares no code with
it.

What it computes
----------------
For every batch b and head h, with Q, K, V of shape (N, d):

    S = scale * Q K^T                      (N x N, materialised)
    S[i, j] = -inf where key j is not allowed for query i
    P = exp(S - rowmax(S)),  l = rowsum(P)
    O = (P V) / l                          (rows with no allowed key give 0)

Sources, as the pages state them:
  * Attention itself, S = Q K^T and R = softmax(S) V over (seqlen, d_head)
    tensors: AWS Neuron NKI tutorial "Fused Self Attention", section
    "Background".
  * The scale 1/sqrt(head_dim), applied before the mask, and masking with
    -inf before the softmax: "Profiling in PyTorch" part 3, section
    "Deconstructing Naive Attention" (the NaiveCausalAttention module).
  * Subtracting the row maximum before the exponential, the row sum, and
    dividing once after the product with V: NKI tutorial, section
    "Softmax implementation". The fused method reaches the same result as
    this plain definition, because softmax attention is exact (PhotoRoom
    post on xformers memory-efficient attention, the FlashAttention
    paragraph) and delaying the division is exact by associativity (NKI
    tutorial, "Softmax implementation").
  * The causal mask (key after query is masked): "Profiling in PyTorch",
    the naive module and the is_causal=True call of SDPA.
  * 2D neighbourhood attention whose window wraps around the borders like a
    convolution with circular padding: NATTEN issue 142 ("circular windowed
    attention"), the 5x5 kernel_size=3 example and its printed output.
  * The standard (clamped) neighbourhood window, where a query near an edge
    keeps a full-size window shifted inside the grid and a key is allowed
    when it falls between the query's window start and end: the same issue,
    the replies on window_start/window_end and on clamping the sliding
    window to the edges.

Readings taken where the pages leave a point open
--------------------------------------------------
  * scale is an explicit argument; callers pass the float32 value the GPU
    path receives (its float64 value is used here unchanged).
  * The mask is applied after scaling, so scale = 0 averages over the
    allowed keys instead of producing 0 * (-inf).
  * A row with no allowed key returns 0 (the NaN guard of SDPA's safe
    softmax, "Profiling in PyTorch", the math-backend section).
  * Tokens map to a row-major grid: token n sits at row y = n // grid_w and
    column x = n % grid_w.
  * Wrapped windows are centred (offsets -r..r with r = kernel // 2 along
    each axis) and wrap modulo the grid size; kernels are odd and at most
    the grid size. Each key counts once.
  * Inputs are the bfloat16 values both sides consume, widened exactly to
    float64; the result is returned unrounded.

Every function is plain NumPy. Internal steps live in module-level functions
so a test can substitute a planted mistake and check that a pin catches it.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

MASKS = ("none", "causal", "na2d")


@dataclass(frozen=True)
class NA2D:
    """A 2D neighbourhood window over a row-major grid of grid_h x grid_w tokens.

    wrap_h / wrap_w select, per axis, the circular window (True) or the
    standard clamped window (False) of NATTEN issue 142.
    """

    grid_h: int
    grid_w: int
    kernel_h: int
    kernel_w: int
    wrap_h: bool = True
    wrap_w: bool = True


def _as_f64(x) -> np.ndarray:
    """Widen an input array to float64 (exact for bfloat16 and float32 values)."""
    return np.asarray(x, dtype=np.float64)


def _axis_allowed(cq: np.ndarray, ck: np.ndarray, length: int, kernel: int, wrap: bool) -> np.ndarray:
    """Allowed (query, key) pairs along one grid axis.

    Wrapped: the circular distance min((a-b) mod L, (b-a) mod L) is at most
    r = kernel // 2 (a centred window that wraps at the borders).
    Clamped: the window of `kernel` cells starts at clamp(c - r, 0, L - kernel)
    and the key coordinate must fall inside it.
    """
    r = kernel // 2
    cq = cq[:, None]
    ck = ck[None, :]
    if wrap:
        fwd = np.mod(ck - cq, length)
        bwd = np.mod(cq - ck, length)
        return np.minimum(fwd, bwd) <= r
    start = np.clip(cq - r, 0, length - kernel)
    return (ck >= start) & (ck < start + kernel)


def allowed(N: int, mask: str = "none", na2d: NA2D | None = None, rows=None) -> np.ndarray:
    """Boolean matrix A[i, j]: may query rows[i] attend to key j (True = allowed)."""
    qi = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    kj = np.arange(N)
    if mask == "none":
        return np.ones((qi.size, N), dtype=bool)
    if mask == "causal":
        return kj[None, :] <= qi[:, None]
    if mask == "na2d":
        if na2d is None:
            raise ValueError("na2d mask needs NA2D parameters")
        p = na2d
        if p.grid_h * p.grid_w != N:
            raise ValueError("grid_h * grid_w must equal N")
        for kern, length in ((p.kernel_h, p.grid_h), (p.kernel_w, p.grid_w)):
            if kern < 1 or kern % 2 == 0 or kern > length:
                raise ValueError("kernel sizes must be odd and between 1 and the grid size")
        yq, xq = np.divmod(qi, p.grid_w)
        yk, xk = np.divmod(kj, p.grid_w)
        return (_axis_allowed(yq, yk, p.grid_h, p.kernel_h, p.wrap_h)
                & _axis_allowed(xq, xk, p.grid_w, p.kernel_w, p.wrap_w))
    raise ValueError(f"unknown mask {mask!r}")


def _scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """S = scale * Q K^T for one head (rows of q are the queries asked for)."""
    return scale * (q @ k.T)


def _apply_mask(s: np.ndarray, allow: np.ndarray) -> np.ndarray:
    """Set disallowed scores to -inf (after scaling)."""
    return np.where(allow, s, -np.inf)


def _softmax_parts(s: np.ndarray):
    """Row maximum, unnormalised weights P = exp(S - m) and row sums l.

    Rows with no allowed key (all -inf) get m = 0, P = 0 and l = 0.
    """
    m = np.max(s, axis=1, keepdims=True)
    m = np.where(np.isneginf(m), 0.0, m)
    p = np.exp(s - m)
    l = np.sum(p, axis=1, keepdims=True)
    return m, p, l


def _combine(p: np.ndarray, l: np.ndarray, v: np.ndarray) -> np.ndarray:
    """O = (P V) / l, dividing once per row after the product; 0 where l = 0."""
    num = p @ v
    safe = np.where(l > 0, l, 1.0)
    return np.where(l > 0, num / safe, 0.0)


def masked_attention(q, k, v, scale: float, allow: np.ndarray) -> np.ndarray:
    """One head: q (R, d), k and v (N, d), allow (R, N) boolean. Returns (R, d) float64."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    s = _apply_mask(_scores(q, k, float(scale)), allow)
    _, p, l = _softmax_parts(s)
    return _combine(p, l, v)


def attention(q, k, v, scale: float, mask: str = "none", na2d: NA2D | None = None, rows=None) -> np.ndarray:
    """Attention over [B, H, N, d] inputs; returns float64 [B, H, R, d].

    rows, if given, selects the query rows to evaluate (the definition is
    evaluated at those rows only; every key still takes part).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if q.ndim != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    B, H, N, d = q.shape
    sel = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    allow = allowed(N, mask, na2d, sel)
    out = np.empty((B, H, sel.size, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            out[b, h] = masked_attention(q[b, h, sel], k[b, h], v[b, h], scale, allow)
    return out


def probs(q, k, scale: float, mask: str = "none", na2d: NA2D | None = None) -> np.ndarray:
    """Normalised attention weights P / l, float64 [B, H, N, N] (small shapes only)."""
    q, k = _as_f64(q), _as_f64(k)
    B, H, N, d = q.shape
    allow = allowed(N, mask, na2d)
    out = np.empty((B, H, N, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            s = _apply_mask(_scores(q[b, h], k[b, h], float(scale)), allow)
            _, p, l = _softmax_parts(s)
            out[b, h] = np.where(l > 0, p / np.where(l > 0, l, 1.0), 0.0)
    return out

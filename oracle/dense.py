"""CPU oracle for exact softmax attention, in float64 NumPy.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module. The product path (the
HIP library and its Python binding) never calls it and shares no code with
it.

What it computes
----------------
For every batch b and head h, with Q of shape (Nq, d) and K, V of shape
(Nkv, d) (Nq = Nkv = N for self-attention):

    S = scale * Q K^T                      (Nq x Nkv, materialised)
    S[i, j] = -inf where key j is not allowed for query i
    m = rowmax(S), P = exp(S - m),  l = rowsum(P)
    O = (P V) / l                          (rows with no allowed key give 0)
    LSE = m + log(l)                       (optional; -inf for such rows)

and, for an output gradient dO (backward), with P = softmax(S):

    dV = P^T dO,  dP = dO V^T
    dS = P * (dP - rowsum(P * dP))         (the softmax Jacobian applied to dP)
    dQ = scale * dS K,  dK = scale * dS^T Q

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
  * 3D neighbourhoods (the MR volumes of the same issue, wrapping in some
    axes only) and dilation (the issue's 1D wrap recipe pads by
    kernel // 2 * dilation before a dilated window).
  * The logsumexp of each row, log(sum_j exp(S[i, j])), which the fused
    forward of the same issue saves beside the output for the backward pass.
  * The backward pass: the gradients of the forward with respect to Q, K and
    V for an output gradient dO (the same issue's autograd function and its
    gradcheck; its backward revisits query tiles per key tile).

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
  * Dilation d along an axis: the window takes every d-th cell. Wrapped, a
    key is allowed when its coordinate is (c + d*t) mod L for some
    t in -r..r (which is what padding by r*d, a dilated window and cropping
    give in the issue's 1D recipe); this needs (kernel - 1) * d < L so each
    key counts once. Clamped, the axis splits into the d interleaved
    sub-grids of cells with equal coordinate mod d, and the undilated clamped
    window is taken inside the query's sub-grid; this needs kernel * d <= L
    so every sub-grid holds a whole window.
  * A 3D grid is row-major: token n sits at depth z, row y, column x with
    n = (z * grid_h + y) * grid_w + x. A key is visible when all three axes
    allow it.
  * Queries and keys may differ in number (cross-attention; the issue notes
    that the neighbourhood kernels assume they are equal, so the
    neighbourhood masks require Nq = Nkv). The causal mask keeps key j for
    query i when j <= i (top-left aligned, as SDPA's is_causal does for
    non-square masks).
  * logsumexp of a row with no allowed key is -inf (the log of an empty sum).

Every function is plain NumPy. Internal steps live in module-level functions
so a test can substitute a planted mistake and check that a pin catches it.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

MASKS = ("none", "causal", "na2d", "na3d")


@dataclass(frozen=True)
class NA2D:
    """A 2D neighbourhood window over a row-major grid of grid_h x grid_w tokens.

    wrap_h / wrap_w select, per axis, the circular window (True) or the
    standard clamped window (False) of NATTEN issue 142; dil_h / dil_w are the
    dilations (1 = contiguous window).
    """

    grid_h: int
    grid_w: int
    kernel_h: int
    kernel_w: int
    wrap_h: bool = True
    wrap_w: bool = True
    dil_h: int = 1
    dil_w: int = 1

    def grid(self):
        return (self.grid_h, self.grid_w)

    def axes(self):
        """(length, kernel, wrap, dilation) per axis, slowest axis first."""
        return ((self.grid_h, self.kernel_h, self.wrap_h, self.dil_h),
                (self.grid_w, self.kernel_w, self.wrap_w, self.dil_w))


@dataclass(frozen=True)
class NA3D:
    """A 3D neighbourhood window over a row-major grid of grid_d x grid_h x grid_w tokens."""

    grid_d: int
    grid_h: int
    grid_w: int
    kernel_d: int
    kernel_h: int
    kernel_w: int
    wrap_d: bool = True
    wrap_h: bool = True
    wrap_w: bool = True
    dil_d: int = 1
    dil_h: int = 1
    dil_w: int = 1

    def grid(self):
        return (self.grid_d, self.grid_h, self.grid_w)

    def axes(self):
        return ((self.grid_d, self.kernel_d, self.wrap_d, self.dil_d),
                (self.grid_h, self.kernel_h, self.wrap_h, self.dil_h),
                (self.grid_w, self.kernel_w, self.wrap_w, self.dil_w))


def _as_f64(x) -> np.ndarray:
    """Widen an input array to float64 (exact for bfloat16 and float32 values)."""
    return np.asarray(x, dtype=np.float64)


def _axis_allowed(cq: np.ndarray, ck: np.ndarray, length: int, kernel: int, wrap: bool, dil: int = 1) -> np.ndarray:
    """Allowed (query, key) pairs along one grid axis.

    Wrapped: the key coordinate is (c + dil * t) mod L for some t in -r..r,
    r = kernel // 2 (a centred window that wraps at the borders; with
    dil = 1, the circular distance is at most r).
    Clamped: inside the query's sub-grid of cells congruent to it mod dil,
    the window of `kernel` cells starts at clamp(i - r, 0, L_g - kernel),
    where i is the query's index in its sub-grid and L_g the sub-grid's
    length; the key must lie in the same sub-grid and inside that window.
    """
    r = kernel // 2
    cq = cq[:, None]
    ck = ck[None, :]
    if wrap:
        fwd = np.mod(ck - cq, length)
        bwd = np.mod(cq - ck, length)
        return ((fwd % dil == 0) & (fwd <= r * dil)) | ((bwd % dil == 0) & (bwd <= r * dil))
    g = np.mod(cq, dil)
    sub_len = (length - 1 - g) // dil + 1
    start = np.clip(cq // dil - r, 0, sub_len - kernel)
    j = ck // dil
    return (np.mod(ck, dil) == g) & (j >= start) & (j < start + kernel)


def _check_na(na, N: int, mask: str) -> None:
    want = {"na2d": NA2D, "na3d": NA3D}[mask]
    if not isinstance(na, want):
        raise ValueError(f"{mask} mask needs {want.__name__} parameters")
    if int(np.prod(na.grid())) != N:
        raise ValueError("the grid must hold exactly N tokens")
    for length, kern, wrap, dil in na.axes():
        if dil < 1:
            raise ValueError("dilation must be at least 1")
        if kern < 1 or kern % 2 == 0:
            raise ValueError("kernel sizes must be odd and positive")
        if wrap and (kern - 1) * dil >= length:
            raise ValueError("a wrapped window must satisfy (kernel - 1) * dilation < grid size")
        if not wrap and kern * dil > length:
            raise ValueError("a clamped window must satisfy kernel * dilation <= grid size")


def allowed(N: int, mask: str = "none", na=None, rows=None, n_kv: int | None = None) -> np.ndarray:
    """Boolean matrix A[i, j]: may query rows[i] attend to key j (True = allowed).

    N is the number of queries, n_kv the number of keys (default N).
    """
    n_kv = N if n_kv is None else n_kv
    qi = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    kj = np.arange(n_kv)
    if mask == "none":
        return np.ones((qi.size, n_kv), dtype=bool)
    if mask == "causal":
        return kj[None, :] <= qi[:, None]
    if mask in ("na2d", "na3d"):
        if n_kv != N:
            raise ValueError("neighbourhood masks need as many keys as queries")
        _check_na(na, N, mask)
        cq = np.unravel_index(qi, na.grid())
        ck = np.unravel_index(kj, na.grid())
        out = np.ones((qi.size, n_kv), dtype=bool)
        for a, (length, kern, wrap, dil) in enumerate(na.axes()):
            out &= _axis_allowed(cq[a], ck[a], length, kern, wrap, dil)
        return out
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


def _logsumexp(m: np.ndarray, l: np.ndarray) -> np.ndarray:
    """log(sum_j exp(S[i, j])) = m + log(l) per row; -inf where no key is allowed."""
    with np.errstate(divide="ignore"):
        return np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)[:, 0]


def masked_attention(q, k, v, scale: float, allow: np.ndarray, return_lse: bool = False):
    """One head: q (R, d), k and v (M, d), allow (R, M) boolean. Returns (R, d) float64
    (and the (R,) logsumexp when return_lse)."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    s = _apply_mask(_scores(q, k, float(scale)), allow)
    m, p, l = _softmax_parts(s)
    out = _combine(p, l, v)
    return (out, _logsumexp(m, l)) if return_lse else out


def attention(q, k, v, scale: float, mask: str = "none", na=None, rows=None, return_lse: bool = False):
    """Attention over q [B, H, Nq, d] and k, v [B, H, Nkv, d]; returns float64 [B, H, R, d]
    (and the logsumexp, float64 [B, H, R], when return_lse).

    rows, if given, selects the query rows to evaluate (the definition is
    evaluated at those rows only; every key still takes part).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if q.ndim != 4 or k.ndim != 4 or v.shape != k.shape or k.shape[:2] != q.shape[:2] or k.shape[3] != q.shape[3]:
        raise ValueError("q must be [B, H, Nq, d] and k, v one [B, H, Nkv, d] shape")
    B, H, Nq, d = q.shape
    sel = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    allow = allowed(Nq, mask, na, sel, n_kv=k.shape[2])
    out = np.empty((B, H, sel.size, d), dtype=np.float64)
    lse = np.empty((B, H, sel.size), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            out[b, h], lse[b, h] = masked_attention(q[b, h, sel], k[b, h], v[b, h], scale, allow, True)
    return (out, lse) if return_lse else out


def probs(q, k, scale: float, mask: str = "none", na=None) -> np.ndarray:
    """Normalised attention weights P / l, float64 [B, H, Nq, Nkv] (small shapes only)."""
    q, k = _as_f64(q), _as_f64(k)
    B, H, Nq, d = q.shape
    allow = allowed(Nq, mask, na, n_kv=k.shape[2])
    out = np.empty((B, H, Nq, k.shape[2]), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            s = _apply_mask(_scores(q[b, h], k[b, h], float(scale)), allow)
            _, p, l = _softmax_parts(s)
            out[b, h] = np.where(l > 0, p / np.where(l > 0, l, 1.0), 0.0)
    return out


def _softmax_grad(p: np.ndarray, dp: np.ndarray) -> np.ndarray:
    """dS = P * (dP - rowsum(P * dP)): the Jacobian of a row softmax applied to dP."""
    return p * (dp - np.sum(p * dp, axis=1, keepdims=True))


def _grad_v(p: np.ndarray, do: np.ndarray) -> np.ndarray:
    """dV = P^T dO."""
    return p.T @ do


def _grad_q(ds: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """dQ = scale * dS K."""
    return scale * (ds @ k)


def _grad_k(ds: np.ndarray, q: np.ndarray, scale: float) -> np.ndarray:
    """dK = scale * dS^T Q."""
    return scale * (ds.T @ q)


def masked_attention_backward(q, k, v, do, scale: float, allow: np.ndarray):
    """One head: gradients (dq, dk, dv) of O = softmax(scale q k^T masked) v for output gradient do."""
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    s = _apply_mask(_scores(q, k, float(scale)), allow)
    _, e, l = _softmax_parts(s)
    p = np.where(l > 0, e / np.where(l > 0, l, 1.0), 0.0)
    ds = _softmax_grad(p, do @ v.T)
    return _grad_q(ds, k, float(scale)), _grad_k(ds, q, float(scale)), _grad_v(p, do)


def attention_backward(q, k, v, do, scale: float, mask: str = "none", na=None):
    """Gradients (dq, dk, dv) of attention(q, k, v, scale, mask, na) for output gradient do [B, H, Nq, d];
    float64, shaped like q, k and v."""
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    if do.shape != q.shape:
        raise ValueError("do must be shaped like q")
    B, H, Nq, d = q.shape
    allow = allowed(Nq, mask, na, n_kv=k.shape[2])
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = masked_attention_backward(q[b, h], k[b, h], v[b, h], do[b, h], scale, allow)
    return dq, dk, dv

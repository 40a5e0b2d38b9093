"""A CPU model of the floating-point steps of the fused forward kernel, and the
per-element error bound derived from them.

TEST INFRASTRUCTURE. This is not the oracle (oracle/dense.py is the float64
definition); it re-enacts, in float32 / bfloat16 NumPy, the arithmetic the HIP
kernel performs, so that the tolerance of the parity tests can be argued from
that arithmetic and checked on the CPU:

  * scores s = q . k in float32 (bf16 inputs, products exact in float32), Q's
    sign flipped for a negative scale, c = |scale| * log2(e) rounded to float32;
  * key tiles of `bn` keys visited in order; the first tile sets the reference
    maximum m = c * (its largest visible score), later tiles use it;
  * P = 2^(fma(s, c, -m)) in float32, rounded to bfloat16 (nearest even), hidden
    keys 0; the row sum adds the rounded values (float32);
  * the overflow guard: a lane holds 64 of a tile's 128 keys (key offsets with
    (offset // 4) odd in the second half-wave); if the sum of a lane's rounded
    probabilities of a tile exceeds 2^20 (or is not finite), the whole wavefront
    (32 query rows) moves its reference to max(m, c * tile maximum), rescales
    O and l by 2^(m_old - m_new) and redoes the tile;
  * O accumulates P V in float32; at the end O * (1 / l) in float32, rounded to
    bfloat16 (nearest even).

The summation order of the matrix core is not modelled (float32 sums in NumPy's
order instead): the model is not bit-exact to the GPU, only to its precision.

The method computes softmax(scale Q K^T) V exactly up to rounding (NKI tutorial
"Fused Self Attention", section "Softmax implementation": the delayed division
is exact; PhotoRoom's xformers post: exact attention). Rounding the
probabilities to bfloat16 is this build's choice for the second matrix product;
the pages fix no precision for it.
"""
from __future__ import annotations

import numpy as np
import torch

LOG2E = 1.4426950408889634
SAFE_SUM = np.float32(2.0 ** 20)
FLT_MAX = np.float32(np.finfo(np.float32).max)
U_BF16 = 2.0 ** -8   # unit roundoff of bfloat16, round to nearest (8-bit significand)
U_FP16 = 2.0 ** -11  # unit roundoff of float16 (11-bit significand)


def to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 (round to nearest even) -> float32."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def to_fp16(x: np.ndarray) -> np.ndarray:
    """float32 -> float16 (round to nearest even; inf past its range) -> float32."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


def _lane_half(bn: int) -> np.ndarray:
    """Which half-wave holds each key offset of a tile: offsets 8g + 4h + (0..3) of a 32-key block."""
    off = np.arange(bn)
    return (off // 4) % 2


def model_head(q, k, v, scale: float, allow=None, bn: int = 128, first_tile: int = 0, p_format: str = "bf16"):
    """Modelled kernel output (float32 values of bfloat16) of one head: q (Nq, d), k, v (Nkv, d)
    holding bfloat16 values. allow: bool (Nq, Nkv) or None. Tiles are visited circularly from
    first_tile. p_format "bf16" is the kernel's; "fp16" models float16 probabilities and values
    (values scaled by 2^-8 into float16 range, probabilities kept below 2^15); "bf16x2" models P
    split into a bfloat16 high part and a bfloat16 remainder (two products with V, both parts in
    the row sum)."""
    q = np.asarray(q, np.float32)
    k = np.asarray(k, np.float32)
    v = np.asarray(v, np.float32)
    Nq, d = q.shape
    Nkv = k.shape[0]
    c = np.float32(abs(float(scale)) * LOG2E)
    qs = -q if scale < 0 else q
    S = qs @ k.T  # float32 products of bf16 values, float32 sums
    if allow is None:
        allow = np.ones((Nq, Nkv), dtype=bool)
    if p_format == "bf16":
        round_p, vv, v_scale, safe = to_bf16, v, np.float32(1.0), SAFE_SUM
    elif p_format == "fp16":
        round_p, vv, v_scale, safe = to_fp16, to_fp16(v * np.float32(2.0 ** -8)), np.float32(2.0 ** 8), np.float32(2.0 ** 15)
    elif p_format == "bf16x2":  # P as the sum of two bfloat16 parts (P V as two products)
        round_p, vv, v_scale, safe = (lambda x: to_bf16(x) + to_bf16(x - to_bf16(x))), v, np.float32(1.0), SAFE_SUM
    else:
        raise ValueError(p_format)
    n_tiles = -(-Nkv // bn)
    order = [(first_tile + i) % n_tiles for i in range(n_tiles)]
    m = np.full(Nq, np.nan, np.float32)
    O = np.zeros((Nq, d), np.float32)
    lsum = np.zeros((Nq, 2), np.float32)
    wave_of_row = (np.arange(Nq) % 128) // 32 + 4 * (np.arange(Nq) // 128)

    def probs(s, a, mref):
        x = (s.astype(np.float64) * float(c) - mref[:, None].astype(np.float64)).astype(np.float32)  # fma
        with np.errstate(over="ignore"):  # a row with no visible key yet: inf, caught by the guard
            p = np.exp2(x).astype(np.float32)
        p = np.where(a, p, np.float32(0.0))
        return round_p(p)

    def visible_max(s, a):
        return np.where(a, s, -np.inf).max(axis=1).astype(np.float32)

    for ti, t in enumerate(order):
        cols = slice(t * bn, min(Nkv, t * bn + bn))
        s, a = S[:, cols], allow[:, cols]
        halves = _lane_half(bn)[: s.shape[1]]
        if ti == 0:
            mx = visible_max(s, a)
            m = np.where(mx == -np.inf, -FLT_MAX, (mx * c).astype(np.float32)).astype(np.float32)
            pt = probs(s, a, m)
        else:
            pt = probs(s, a, m)
            ps = np.stack([pt[:, halves == h].sum(axis=1, dtype=np.float32) for h in (0, 1)], axis=1)
            bad_row = ~np.all(ps <= safe, axis=1)
            bad_waves = np.unique(wave_of_row[bad_row])
            redo = np.isin(wave_of_row, bad_waves)
            if redo.any():
                mx = visible_max(s, a)
                cand = np.where(mx == -np.inf, -FLT_MAX, (mx * c).astype(np.float32)).astype(np.float32)
                m_new = np.where(redo, np.maximum(m, cand), m).astype(np.float32)
                alpha = np.exp2((m - m_new).astype(np.float32)).astype(np.float32)
                O = (O * alpha[:, None]).astype(np.float32)
                lsum = (lsum * alpha[:, None]).astype(np.float32)
                m = m_new
                pt = probs(s, a, m)
        ps = np.stack([pt[:, halves == h].sum(axis=1, dtype=np.float32) for h in (0, 1)], axis=1)
        lsum = (lsum + ps).astype(np.float32)
        O = (O + pt @ vv[cols]).astype(np.float32)
    l = (lsum[:, 0] + lsum[:, 1]).astype(np.float32)
    inv = np.where(l > 0, (np.float32(1.0) / np.where(l > 0, l, 1)).astype(np.float32), np.float32(0.0))
    out = (O * inv[:, None] * v_scale).astype(np.float32)
    return to_bf16(out)


def model_forward(q, k, v, scale: float, allow=None, bn: int = 128, p_format: str = "bf16") -> np.ndarray:
    """model_head over [B, H, N, d] arrays; returns float64."""
    q, k, v = (np.asarray(t, np.float64) for t in (q, k, v))
    B, H = q.shape[:2]
    out = np.zeros(q.shape, np.float64)
    for b in range(B):
        for h in range(H):
            out[b, h] = model_head(q[b, h], k[b, h], v[b, h], scale, allow, bn, p_format=p_format)
    return out


def derived_bound(w: np.ndarray, v: np.ndarray, o: np.ndarray, u_p: float = U_BF16) -> np.ndarray:
    """First-order per-element bound on |kernel - exact| for one head, from the arithmetic above.

    w (Nq, Nkv): exact softmax weights; v (Nkv, d); o (Nq, d): exact output.
    Rounding p_i to p~_i = p_i (1 + e_i), |e_i| <= u_p, with the row sum taken of the same
    rounded values, makes the output an exact convex combination with weights
    w_i (1 + e_i) / (1 + e), e = sum_i w_i e_i, so its error is
        sum_i w_i (e_i - e) (v_i - o) / (1 + e)  <=  2 u_p / (1 - u_p) * sum_i w_i |v_i - o|.
    Rounding the output to bfloat16 adds at most U_BF16 |o|. The float32 scores, exponentials,
    sums and reciprocal add about 1e-6 relative; 1e-5 (|o| + sum_i w_i |v_i|) covers them.
    """
    w = np.asarray(w, np.float64)
    v = np.asarray(v, np.float64)
    o = np.asarray(o, np.float64)
    spread = np.empty_like(o)
    step = max(1, int(2e7 // max(1, w.shape[1] * v.shape[1])))
    for i0 in range(0, o.shape[0], step):
        i1 = min(o.shape[0], i0 + step)
        spread[i0:i1] = np.einsum("ij,ijd->id", w[i0:i1], np.abs(v[None, :, :] - o[i0:i1, None, :]))
    mag = w @ np.abs(v)
    return U_BF16 * np.abs(o) + 2.0 * u_p / (1.0 - u_p) * spread + 1e-5 * (np.abs(o) + mag)

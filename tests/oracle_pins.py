"""Pins for the CPU oracle: checks against facts that do not come from the oracle itself.

Each pin is a plain function that raises AssertionError when the oracle
disagrees with what the pages or the mathematics fix. test_oracle_pins.py
runs them as they are; test_oracle_mutants.py plants mistakes in the oracle
and checks that at least one pin fails for each.

Independent routes used here:
  * the worked 5x5 example printed in NATTEN issue 142 (golden fixture);
  * closed forms for uniform scores (means, prefix means, box filters built
    from array shifts);
  * a pure-Python brute force (math.exp / math.fsum, no max subtraction)
    whose key sets are enumerated window offsets, not the oracle's distance
    predicate;
  * torch's scaled_dot_product_attention on the CPU in float64 (the math
    backend "Profiling in PyTorch" calls the reference implementation);
  * the pad -> clamped window -> crop route of NATTEN issue 142;
  * symmetries (torus translation, key permutation) and special cases.
"""
from __future__ import annotations

import math
import pathlib

import numpy as np
import torch

import oracle.dense as O

GOLDEN = pathlib.Path(__file__).parent / "golden"
TIGHT = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _rand(seed, *shape, gain=1.0):
    """bfloat16-representable random values (float32 N(0,1) rounded to bf16)."""
    x = torch.from_numpy(_rng(seed).standard_normal(shape).astype(np.float32) * np.float32(gain))
    return x.to(torch.bfloat16).float().numpy().astype(np.float64)


# ---------------------------------------------------------------- brute force
def _window_keys(i, mask, N, na2d):
    """Key indices visible to query i, enumerated directly (each once)."""
    if mask == "none":
        return list(range(N))
    if mask == "causal":
        return list(range(i + 1))
    p = na2d
    y, x = divmod(i, p.grid_w)
    rh, rw = p.kernel_h // 2, p.kernel_w // 2
    if p.wrap_h:
        rows = [(y + dy) % p.grid_h for dy in range(-rh, rh + 1)]
    else:
        sy = min(max(y - rh, 0), p.grid_h - p.kernel_h)
        rows = list(range(sy, sy + p.kernel_h))
    if p.wrap_w:
        cols = [(x + dx) % p.grid_w for dx in range(-rw, rw + 1)]
    else:
        sx = min(max(x - rw, 0), p.grid_w - p.kernel_w)
        cols = list(range(sx, sx + p.kernel_w))
    keys = sorted({r * p.grid_w + c for r in rows for c in cols})
    assert len(keys) == p.kernel_h * p.kernel_w
    return keys


def brute_head(q, k, v, scale, mask="none", na2d=None, subtract_max=False):
    """One head by the textbook formula, in pure Python floats."""
    n_keys, d = len(k), len(q[0])
    out = []
    for i in range(len(q)):
        keys = _window_keys(i, mask, n_keys, na2d)
        s = [scale * math.fsum(q[i][t] * k[j][t] for t in range(d)) for j in keys]
        ref = max(s) if subtract_max else 0.0
        w = [math.exp(x - ref) for x in s]
        den = math.fsum(w)
        out.append([math.fsum(w[a] * v[j][t] for a, j in enumerate(keys)) / den for t in range(d)])
    return np.array(out)


def _check_brute(mask, na2d, N, d, seed, scale, gain=1.0, subtract_max=False):
    q, k, v = (_rand(seed + i, 1, 2, N, d, gain=gain if i == 0 else 1.0) for i in range(3))
    got = O.attention(q, k, v, scale, mask, na2d)
    for h in range(2):
        want = brute_head(q[0, h].tolist(), k[0, h].tolist(), v[0, h].tolist(), scale, mask, na2d, subtract_max)
        assert np.all(np.isfinite(got[0, h]))
        err = np.max(np.abs(got[0, h] - want))
        assert err <= TIGHT, f"{mask} {na2d} brute-force mismatch {err}"


# ---------------------------------------------------------------- pins
def pin_wrap_5x5_example():
    """NATTEN issue 142: 5x5 grid, kernel 3, wrap; q = k = 1, v one-hot at the top-left pixel."""
    q = np.ones((1, 5, 5, 1, 8))
    k = np.ones((1, 5, 5, 1, 8))
    v = np.zeros((1, 5, 5, 1, 8))
    v[:, 0, 0, :, :] = 1.0
    # [B, X, Y, heads, d] -> [B, heads, X*Y, d], token n = row * 5 + col
    to_bhnd = lambda t: t.transpose(0, 3, 1, 2, 4).reshape(1, 1, 25, 8)
    out = O.attention(to_bhnd(q), to_bhnd(k), to_bhnd(v), 1 / math.sqrt(8), "na2d",
                      O.NA2D(5, 5, 3, 3, True, True))
    grid = out[0, 0, :, 0].reshape(5, 5)
    printed = np.loadtxt(GOLDEN / "na2d_wrap_5x5_k3.txt")
    assert np.max(np.abs(grid - printed)) <= 5e-5 + 1e-12, grid
    exact = np.where(printed > 0, 1.0 / 9.0, 0.0)
    assert np.max(np.abs(grid - exact)) <= TIGHT
    # every channel carries the same pattern
    assert np.max(np.abs(out[0, 0] - grid.reshape(25, 1))) <= TIGHT


def pin_probability_rows_sum_to_one():
    for mask, na2d, N in (("none", None, 12), ("causal", None, 12),
                          ("na2d", O.NA2D(3, 4, 3, 3, True, True), 12),
                          ("na2d", O.NA2D(4, 5, 3, 5, False, True), 20)):
        q, k = _rand(10, 2, 2, N, 8), _rand(11, 2, 2, N, 8)
        p = O.probs(q, k, 0.7, mask, na2d)
        assert np.all(p >= 0)
        assert np.max(np.abs(p.sum(-1) - 1.0)) <= TIGHT, mask
        allow = O.allowed(N, mask, na2d)
        assert np.all(p[..., ~allow] == 0.0)


def pin_uniform_scores_give_means():
    """scale = 0 makes every allowed score equal: the output is the mean of V over the allowed keys."""
    B, H, d = 1, 2, 6
    # none: column mean of V
    v = _rand(20, B, H, 10, d)
    q, k = _rand(21, B, H, 10, d), _rand(22, B, H, 10, d)
    out = O.attention(q, k, v, 0.0, "none")
    assert np.max(np.abs(out - v.mean(axis=2, keepdims=True))) <= TIGHT
    # causal: prefix means
    out = O.attention(q, k, v, 0.0, "causal")
    prefix = np.cumsum(v, axis=2) / np.arange(1, 11)[None, None, :, None]
    assert np.max(np.abs(out - prefix)) <= TIGHT
    # wrapped window: circular box filter made of array shifts
    gh, gw, kh, kw = 5, 6, 3, 5
    N = gh * gw
    q, k, v = _rand(23, B, H, N, d), _rand(24, B, H, N, d), _rand(25, B, H, N, d)
    out = O.attention(q, k, v, 0.0, "na2d", O.NA2D(gh, gw, kh, kw, True, True))
    vg = v.reshape(B, H, gh, gw, d)
    box = sum(np.roll(vg, shift=(-dy, -dx), axis=(2, 3))
              for dy in range(-(kh // 2), kh // 2 + 1) for dx in range(-(kw // 2), kw // 2 + 1)) / (kh * kw)
    assert np.max(np.abs(out - box.reshape(B, H, N, d))) <= TIGHT
    # clamped window: mean over the shifted in-grid window
    out = O.attention(q, k, v, 0.0, "na2d", O.NA2D(gh, gw, kh, kw, False, False))
    want = np.empty_like(vg)
    for y in range(gh):
        for x in range(gw):
            sy = min(max(y - kh // 2, 0), gh - kh)
            sx = min(max(x - kw // 2, 0), gw - kw)
            want[:, :, y, x] = vg[:, :, sy:sy + kh, sx:sx + kw].mean(axis=(2, 3))
    assert np.max(np.abs(out - want.reshape(B, H, N, d))) <= TIGHT


def pin_brute_force_tiny():
    _check_brute("none", None, 13, 5, 30, 0.45)
    _check_brute("causal", None, 16, 4, 31, 0.6)
    _check_brute("na2d", O.NA2D(3, 5, 3, 3, True, True), 15, 4, 32, 0.5)
    _check_brute("na2d", O.NA2D(4, 4, 3, 1, True, True), 16, 3, 33, 0.8)
    _check_brute("na2d", O.NA2D(3, 5, 3, 3, False, False), 15, 4, 34, 0.5)
    _check_brute("na2d", O.NA2D(4, 3, 3, 3, True, False), 12, 4, 35, 0.5)
    _check_brute("none", None, 9, 4, 36, -0.3)   # negative scale is legal


def pin_sdpa_float64():
    """torch's SDPA math path on the CPU in float64 (none, causal, and a boolean window mask)."""
    B, H, N, d = 2, 3, 24, 8
    q, k, v = _rand(40, B, H, N, d), _rand(41, B, H, N, d), _rand(42, B, H, N, d)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    F = torch.nn.functional.scaled_dot_product_attention
    with torch.nn.attention.sdpa_kernel(torch.nn.attention.SDPBackend.MATH):
        ref = F(tq, tk, tv, scale=0.35).numpy()
        assert np.max(np.abs(O.attention(q, k, v, 0.35, "none") - ref)) <= 1e-10
        ref = F(tq, tk, tv, is_causal=True, scale=0.35).numpy()
        assert np.max(np.abs(O.attention(q, k, v, 0.35, "causal") - ref)) <= 1e-10
        p = O.NA2D(4, 6, 3, 5, True, True)
        m = np.zeros((N, N), dtype=bool)
        for i in range(N):
            m[i, _window_keys(i, "na2d", N, p)] = True
        ref = F(tq, tk, tv, attn_mask=torch.from_numpy(m), scale=0.35).numpy()
        assert np.max(np.abs(O.attention(q, k, v, 0.35, "na2d", p) - ref)) <= 1e-10


def pin_wrap_equals_pad_then_crop():
    """NATTEN issue 142: circular padding by r, the standard clamped window, then cropping equals the wrap window."""
    B, H, d = 1, 2, 4
    for gh, gw, kh, kw, seed in ((5, 6, 3, 3, 50), (7, 5, 5, 3, 51), (6, 6, 5, 5, 52)):
        N = gh * gw
        q, k, v = _rand(seed, B, H, N, d), _rand(seed + 1, B, H, N, d), _rand(seed + 2, B, H, N, d)
        want = O.attention(q, k, v, 0.6, "na2d", O.NA2D(gh, gw, kh, kw, True, True))
        rh, rw = kh // 2, kw // 2
        pad = lambda t: np.pad(t.reshape(B, H, gh, gw, d), ((0, 0), (0, 0), (rh, rh), (rw, rw), (0, 0)), mode="wrap")
        ph, pw = gh + 2 * rh, gw + 2 * rw
        qp, kp, vp = (pad(t).reshape(B, H, ph * pw, d) for t in (q, k, v))
        outp = O.attention(qp, kp, vp, 0.6, "na2d", O.NA2D(ph, pw, kh, kw, False, False))
        got = outp.reshape(B, H, ph, pw, d)[:, :, rh:rh + gh, rw:rw + gw].reshape(B, H, N, d)
        assert np.max(np.abs(got - want)) <= TIGHT, (gh, gw, kh, kw)


def pin_wrap_translation_symmetry():
    B, H, d, gh, gw = 1, 2, 4, 6, 7
    N = gh * gw
    p = O.NA2D(gh, gw, 3, 5, True, True)
    q, k, v = _rand(60, B, H, N, d), _rand(61, B, H, N, d), _rand(62, B, H, N, d)
    base = O.attention(q, k, v, 0.5, "na2d", p)
    roll = lambda t: np.roll(t.reshape(B, H, gh, gw, d), shift=(2, -3), axis=(2, 3)).reshape(B, H, N, d)
    moved = O.attention(roll(q), roll(k), roll(v), 0.5, "na2d", p)
    assert np.max(np.abs(moved - roll(base))) <= TIGHT


def pin_full_window_is_full_attention():
    B, H, d = 1, 2, 4
    for gh, gw in ((5, 3), (3, 7)):
        N = gh * gw
        q, k, v = _rand(70, B, H, N, d), _rand(71, B, H, N, d), _rand(72, B, H, N, d)
        full = O.attention(q, k, v, 0.5, "none")
        for wrap in (True, False):
            na = O.attention(q, k, v, 0.5, "na2d", O.NA2D(gh, gw, gh, gw, wrap, wrap))
            assert np.max(np.abs(na - full)) <= TIGHT


def pin_causal_first_row_is_first_value():
    q, k, v = _rand(80, 2, 2, 9, 5), _rand(81, 2, 2, 9, 5), _rand(82, 2, 2, 9, 5)
    out = O.attention(q, k, v, 0.9, "causal")
    assert np.array_equal(out[:, :, 0], v[:, :, 0])


def pin_key_permutation_invariance():
    q, k, v = _rand(90, 1, 2, 17, 6), _rand(91, 1, 2, 17, 6), _rand(92, 1, 2, 17, 6)
    perm = _rng(93).permutation(17)
    a = O.attention(q, k, v, 0.4, "none")
    b = O.attention(q, k[:, :, perm], v[:, :, perm], 0.4, "none")
    assert np.max(np.abs(a - b)) <= TIGHT


def pin_stability_large_scores():
    """Scores of size ~1000 (exp would overflow without the max subtraction)."""
    _check_brute("none", None, 12, 8, 100, 1.0 / math.sqrt(8), gain=256.0, subtract_max=True)
    _check_brute("causal", None, 12, 8, 101, 1.0 / math.sqrt(8), gain=256.0, subtract_max=True)


def pin_fully_masked_row_gives_zero():
    q, k, v = _rand(110, 3, 4), _rand(111, 5, 4), _rand(112, 5, 4)
    allow = np.ones((3, 5), dtype=bool)
    allow[1] = False
    out = O.masked_attention(q, k, v, 0.5, allow)
    assert np.all(out[1] == 0.0)
    assert np.all(np.isfinite(out))
    want = brute_head(q.tolist(), k.tolist(), v.tolist(), 0.5)
    assert np.max(np.abs(out[[0, 2]] - want[[0, 2]])) <= TIGHT


def pin_row_subset_matches_full():
    q, k, v = _rand(120, 1, 2, 40, 8), _rand(121, 1, 2, 40, 8), _rand(122, 1, 2, 40, 8)
    rows = [0, 7, 39, 13]
    for mask, na2d in (("causal", None), ("na2d", O.NA2D(5, 8, 3, 5, True, True))):
        full = O.attention(q, k, v, 0.3, mask, na2d)
        part = O.attention(q, k, v, 0.3, mask, na2d, rows=rows)
        assert np.max(np.abs(part - full[:, :, rows])) <= TIGHT


ALL_PINS = [
    pin_wrap_5x5_example,
    pin_probability_rows_sum_to_one,
    pin_uniform_scores_give_means,
    pin_brute_force_tiny,
    pin_sdpa_float64,
    pin_wrap_equals_pad_then_crop,
    pin_wrap_translation_symmetry,
    pin_full_window_is_full_attention,
    pin_causal_first_row_is_first_value,
    pin_key_permutation_invariance,
    pin_stability_large_scores,
    pin_fully_masked_row_gives_zero,
    pin_row_subset_matches_full,
]

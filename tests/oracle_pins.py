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
  * symmetries (torus translation, key permutation) and special cases;
  * for dilation, the interleaved sub-grids (a dilated window is the
    undilated window inside the sub-grid of cells congruent mod the
    dilation) and the issue's 1D recipe (circular pad by kernel//2 * dilation,
    dilated window, crop);
  * for 3D grids, the 2D case at depth 1, a 3D box filter built from array
    shifts, and the pad/crop route along the wrapped axes;
  * for logsumexp, log(count) at scale 0 and torch.logsumexp in float64;
  * for Nq != Nkv, SDPA in float64 (its is_causal is top-left aligned).
"""
from __future__ import annotations

import itertools
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
def _axis_cells(c, length, kernel, wrap, dil):
    """Window cells of coordinate c along one axis, enumerated from offsets.

    Wrapped: c + dil*t for t = -r..r, taken mod the length. Clamped: the list
    of cells congruent to c mod dil, with a kernel-long window slid inside it
    so that it stays whole at the ends.
    """
    r = kernel // 2
    if wrap:
        return [(c + dil * t) % length for t in range(-r, r + 1)]
    sub = list(range(c % dil, length, dil))
    i = sub.index(c)
    s = min(max(i - r, 0), len(sub) - kernel)
    return sub[s:s + kernel]


def _window_keys(i, mask, N, na=None, n_kv=None):
    """Key indices visible to query i, enumerated directly (each once)."""
    n_kv = N if n_kv is None else n_kv
    if mask == "none":
        return list(range(n_kv))
    if mask == "causal":
        return list(range(min(i + 1, n_kv)))
    grid = na.grid()
    coords = []
    rest = i
    for length in reversed(grid):
        rest, c = divmod(rest, length)
        coords.append(c)
    coords.reverse()
    cells = [_axis_cells(c, *ax) for c, ax in zip(coords, na.axes())]
    keys = set()
    for combo in itertools.product(*cells):
        n = 0
        for c, length in zip(combo, grid):
            n = n * length + c
        keys.add(n)
    keys = sorted(keys)
    assert len(keys) == math.prod(ax[1] for ax in na.axes())
    return keys


def brute_head(q, k, v, scale, mask="none", na=None, subtract_max=False, with_lse=False):
    """One head by the textbook formula, in pure Python floats (lse = log of the plain sum)."""
    n_keys, d = len(k), len(q[0])
    out, lse = [], []
    for i in range(len(q)):
        keys = _window_keys(i, mask, len(q), na, n_keys)
        s = [scale * math.fsum(q[i][t] * k[j][t] for t in range(d)) for j in keys]
        ref = max(s) if subtract_max else 0.0
        w = [math.exp(x - ref) for x in s]
        den = math.fsum(w)
        out.append([math.fsum(w[a] * v[j][t] for a, j in enumerate(keys)) / den for t in range(d)])
        lse.append(ref + math.log(den))
    return (np.array(out), np.array(lse)) if with_lse else np.array(out)


def _check_brute(mask, na, N, d, seed, scale, gain=1.0, subtract_max=False, n_kv=None):
    n_kv = N if n_kv is None else n_kv
    q = _rand(seed, 1, 2, N, d, gain=gain)
    k, v = _rand(seed + 1, 1, 2, n_kv, d), _rand(seed + 2, 1, 2, n_kv, d)
    got, got_lse = O.attention(q, k, v, scale, mask, na, return_lse=True)
    for h in range(2):
        want, want_lse = brute_head(q[0, h].tolist(), k[0, h].tolist(), v[0, h].tolist(), scale, mask, na,
                                    subtract_max, with_lse=True)
        assert np.all(np.isfinite(got[0, h]))
        err = np.max(np.abs(got[0, h] - want))
        assert err <= TIGHT, f"{mask} {na} brute-force mismatch {err}"
        err = np.max(np.abs(got_lse[0, h] - want_lse) / np.maximum(1.0, np.abs(want_lse)))
        assert err <= TIGHT, f"{mask} {na} brute-force logsumexp mismatch {err}"


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


# ---------------------------------------------------------------- logsumexp
def pin_logsumexp_uniform_is_log_count():
    """scale = 0: every allowed score is 0, so the row's logsumexp is log(number of allowed keys)."""
    d = 4
    cases = (("none", None, 10, 10), ("causal", None, 10, 10), ("none", None, 6, 15), ("causal", None, 12, 5),
             ("na2d", O.NA2D(4, 5, 3, 5, True, False), 20, 20),
             ("na2d", O.NA2D(6, 7, 3, 3, False, True, 2, 2), 42, 42),
             ("na3d", O.NA3D(3, 4, 5, 3, 3, 3, True, False, True), 60, 60))
    for mask, na, nq, nkv in cases:
        q, k, v = _rand(130, 1, 2, nq, d), _rand(131, 1, 2, nkv, d), _rand(132, 1, 2, nkv, d)
        _, lse = O.attention(q, k, v, 0.0, mask, na, return_lse=True)
        i = np.arange(nq)
        if mask == "none":
            count = np.full(nq, nkv)
        elif mask == "causal":
            count = np.minimum(i + 1, nkv)
        else:
            count = np.full(nq, math.prod(ax[1] for ax in na.axes()))
        assert np.max(np.abs(lse - np.log(count)[None, None, :])) <= TIGHT, (mask, na)


def pin_logsumexp_torch():
    """torch.logsumexp over the masked float64 score matrix (window masks enumerated by brute force)."""
    B, H, d = 1, 2, 8
    cases = (("none", None, 24, 24, 1.0), ("causal", None, 24, 24, 1.0), ("causal", None, 9, 20, 1.0),
             ("none", None, 16, 16, 64.0),
             ("na2d", O.NA2D(4, 6, 3, 5, True, True), 24, 24, 1.0),
             ("na3d", O.NA3D(2, 3, 4, 1, 3, 3, False, True, True), 24, 24, 1.0))
    for mask, na, nq, nkv, gain in cases:
        q = _rand(140, B, H, nq, d, gain=gain)
        k, v = _rand(141, B, H, nkv, d), _rand(142, B, H, nkv, d)
        _, lse = O.attention(q, k, v, 0.35, mask, na, return_lse=True)
        allow = np.zeros((nq, nkv), dtype=bool)
        for i in range(nq):
            allow[i, _window_keys(i, mask, nq, na, nkv)] = True
        s = torch.from_numpy(q) @ torch.from_numpy(k).transpose(-1, -2) * 0.35
        s = s.masked_fill(~torch.from_numpy(allow), -math.inf)
        want = torch.logsumexp(s, dim=-1).numpy()
        assert np.all(np.isfinite(lse))
        assert np.max(np.abs(lse - want) / np.maximum(1.0, np.abs(want))) <= TIGHT, (mask, na, gain)


# ---------------------------------------------------------------- queries and keys of different lengths
def pin_cross_attention_sdpa():
    """Nq != Nkv against torch's SDPA math path in float64; its is_causal keeps key j <= query i."""
    B, H, d = 2, 2, 8
    F = torch.nn.functional.scaled_dot_product_attention
    for nq, nkv in ((20, 13), (7, 30), (1, 9)):
        q, k, v = _rand(150, B, H, nq, d), _rand(151, B, H, nkv, d), _rand(152, B, H, nkv, d)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        with torch.nn.attention.sdpa_kernel(torch.nn.attention.SDPBackend.MATH):
            for mask in ("none", "causal"):
                ref = F(tq, tk, tv, is_causal=mask == "causal", scale=0.4).numpy()
                assert np.max(np.abs(O.attention(q, k, v, 0.4, mask) - ref)) <= 1e-10, (nq, nkv, mask)


def pin_cross_attention_uniform_and_brute():
    """scale = 0 with Nq != Nkv: means of V over all keys, or over keys 0..min(i, Nkv-1) (causal)."""
    B, H, d = 1, 2, 5
    for nq, nkv in ((12, 5), (4, 11)):
        q, k, v = _rand(160, B, H, nq, d), _rand(161, B, H, nkv, d), _rand(162, B, H, nkv, d)
        out = O.attention(q, k, v, 0.0, "none")
        assert np.max(np.abs(out - v.mean(axis=2, keepdims=True))) <= TIGHT
        out = O.attention(q, k, v, 0.0, "causal")
        prefix = np.cumsum(v, axis=2) / np.arange(1, nkv + 1)[None, None, :, None]
        want = prefix[:, :, np.minimum(np.arange(nq), nkv - 1)]
        assert np.max(np.abs(out - want)) <= TIGHT
    _check_brute("none", None, 7, 4, 163, 0.5, n_kv=12)
    _check_brute("causal", None, 12, 4, 164, 0.5, n_kv=5)


# ---------------------------------------------------------------- dilation
def _subgrid_attention(q, k, v, scale, grid, dils, make_na):
    """Undilated neighbourhood attention run separately on each interleaved sub-grid
    (cells with equal coordinates mod the dilations), scattered back."""
    B, H, N, d = q.shape
    coords = np.stack(np.unravel_index(np.arange(N), grid), axis=1)
    out = np.full((B, H, N, d), np.nan)
    for res in itertools.product(*(range(dl) for dl in dils)):
        sel = np.flatnonzero(np.all(coords % np.array(dils) == np.array(res), axis=1))
        sub_grid = tuple(len(range(r, g, dl)) for r, g, dl in zip(res, grid, dils))
        assert math.prod(sub_grid) == sel.size
        out[:, :, sel] = O.attention(q[:, :, sel], k[:, :, sel], v[:, :, sel], scale,
                                     "na2d" if len(grid) == 2 else "na3d", make_na(sub_grid))
    return out


def pin_dilation_is_undilated_window_on_subgrids():
    """A dilated window equals the undilated window inside each interleaved sub-grid
    (clamped axes: any size with kernel * dilation <= L; wrapped axes: L divisible by the dilation)."""
    B, H, d = 1, 2, 4
    cases = ((7, 9, 3, 3, False, False, 2, 3), (8, 6, 3, 3, True, True, 2, 2), (12, 9, 3, 3, True, False, 4, 3),
             (6, 10, 3, 5, False, True, 2, 2), (5, 12, 5, 3, False, True, 1, 4))
    for gh, gw, kh, kw, wh, ww, dh, dw in cases:
        N = gh * gw
        q, k, v = _rand(170, B, H, N, d), _rand(171, B, H, N, d), _rand(172, B, H, N, d)
        got = O.attention(q, k, v, 0.55, "na2d", O.NA2D(gh, gw, kh, kw, wh, ww, dh, dw))
        want = _subgrid_attention(q, k, v, 0.55, (gh, gw), (dh, dw),
                                  lambda sg: O.NA2D(sg[0], sg[1], kh, kw, wh, ww))
        assert np.max(np.abs(got - want)) <= TIGHT, (gh, gw, kh, kw, wh, ww, dh, dw)
    gd, gh, gw = 4, 6, 5
    N = gd * gh * gw
    q, k, v = _rand(173, B, H, N, d), _rand(174, B, H, N, d), _rand(175, B, H, N, d)
    got = O.attention(q, k, v, 0.55, "na3d", O.NA3D(gd, gh, gw, 1, 3, 3, True, False, True, 2, 2, 1))
    want = _subgrid_attention(q, k, v, 0.55, (gd, gh, gw), (2, 2, 1),
                              lambda sg: O.NA3D(sg[0], sg[1], sg[2], 1, 3, 3, True, False, True))
    assert np.max(np.abs(got - want)) <= TIGHT


def _pad_crop(q, k, v, scale, grid, kernels, wraps, dils):
    """NATTEN issue 142's recipe: pad the wrapped axes circularly by kernel//2 * dilation,
    run the clamped (dilated) window on the padded grid, crop the output back."""
    B, H, N, d = q.shape
    pads = [(kk // 2) * dl if w else 0 for kk, w, dl in zip(kernels, wraps, dils)]
    widths = ((0, 0), (0, 0)) + tuple((p, p) for p in pads) + ((0, 0),)
    padded = tuple(g + 2 * p for g, p in zip(grid, pads))
    pad = lambda t: np.pad(t.reshape(B, H, *grid, d), widths, mode="wrap").reshape(B, H, -1, d)
    qp, kp, vp = (pad(t) for t in (q, k, v))
    if len(grid) == 2:
        na = O.NA2D(*padded, *kernels, False, False, *dils)
        outp = O.attention(qp, kp, vp, scale, "na2d", na)
    else:
        na = O.NA3D(*padded, *kernels, False, False, False, *dils)
        outp = O.attention(qp, kp, vp, scale, "na3d", na)
    crop = tuple(slice(p, p + g) for p, g in zip(pads, grid))
    return outp.reshape(B, H, *padded, d)[(slice(None), slice(None)) + crop].reshape(B, H, N, d)


def pin_dilated_wrap_equals_pad_then_crop():
    B, H, d = 1, 2, 4
    for gh, gw, kh, kw, wh, ww, dh, dw in ((7, 8, 3, 3, True, True, 2, 3), (9, 5, 5, 3, True, False, 2, 1),
                                           (6, 11, 3, 5, False, True, 2, 2)):
        N = gh * gw
        q, k, v = _rand(180, B, H, N, d), _rand(181, B, H, N, d), _rand(182, B, H, N, d)
        got = O.attention(q, k, v, 0.6, "na2d", O.NA2D(gh, gw, kh, kw, wh, ww, dh, dw))
        want = _pad_crop(q, k, v, 0.6, (gh, gw), (kh, kw), (wh, ww), (dh, dw))
        assert np.max(np.abs(got - want)) <= TIGHT, (gh, gw, kh, kw, wh, ww, dh, dw)


# ---------------------------------------------------------------- 3D neighbourhoods
def pin_na3d_depth_one_is_na2d():
    B, H, d, gh, gw = 1, 2, 4, 5, 6
    N = gh * gw
    q, k, v = _rand(190, B, H, N, d), _rand(191, B, H, N, d), _rand(192, B, H, N, d)
    for kh, kw, wh, ww, dh, dw in ((3, 5, True, False, 1, 1), (3, 3, False, True, 1, 2)):
        a = O.attention(q, k, v, 0.45, "na2d", O.NA2D(gh, gw, kh, kw, wh, ww, dh, dw))
        for wd in (True, False):
            b = O.attention(q, k, v, 0.45, "na3d", O.NA3D(1, gh, gw, 1, kh, kw, wd, wh, ww, 1, dh, dw))
            assert np.max(np.abs(a - b)) <= TIGHT


def pin_na3d_brute_force():
    _check_brute("na3d", O.NA3D(3, 3, 4, 3, 3, 3, True, True, True), 36, 4, 200, 0.5)
    _check_brute("na3d", O.NA3D(4, 3, 3, 3, 1, 3, False, True, False), 36, 4, 201, 0.5)
    _check_brute("na3d", O.NA3D(5, 2, 4, 3, 1, 3, True, False, True, 2, 1, 1), 40, 3, 202, 0.7)
    _check_brute("na2d", O.NA2D(7, 6, 3, 3, True, False, 2, 2), 42, 3, 203, 0.7)


def pin_na3d_uniform_box_filter():
    """scale = 0, every axis wrapped: the mean of V over the (dilated) window, as a sum of array shifts."""
    B, H, d = 1, 2, 3
    gd, gh, gw = 4, 5, 6
    N = gd * gh * gw
    q, k, v = _rand(210, B, H, N, d), _rand(211, B, H, N, d), _rand(212, B, H, N, d)
    for (kd, kh, kw), (dd, dh, dw) in (((3, 3, 5), (1, 1, 1)), ((3, 1, 3), (1, 1, 2)), ((1, 3, 3), (1, 2, 1))):
        out = O.attention(q, k, v, 0.0, "na3d", O.NA3D(gd, gh, gw, kd, kh, kw, True, True, True, dd, dh, dw))
        vg = v.reshape(B, H, gd, gh, gw, d)
        box = sum(np.roll(vg, shift=(-a * dd, -b * dh, -c * dw), axis=(2, 3, 4))
                  for a in range(-(kd // 2), kd // 2 + 1)
                  for b in range(-(kh // 2), kh // 2 + 1)
                  for c in range(-(kw // 2), kw // 2 + 1)) / (kd * kh * kw)
        assert np.max(np.abs(out - box.reshape(B, H, N, d))) <= TIGHT


def pin_na3d_translation_and_pad_crop():
    B, H, d = 1, 2, 4
    gd, gh, gw = 4, 5, 6
    N = gd * gh * gw
    q, k, v = _rand(220, B, H, N, d), _rand(221, B, H, N, d), _rand(222, B, H, N, d)
    p = O.NA3D(gd, gh, gw, 3, 3, 5, True, True, True)
    base = O.attention(q, k, v, 0.5, "na3d", p)
    roll = lambda t: np.roll(t.reshape(B, H, gd, gh, gw, d), shift=(1, -2, 3), axis=(2, 3, 4)).reshape(B, H, N, d)
    moved = O.attention(roll(q), roll(k), roll(v), 0.5, "na3d", p)
    assert np.max(np.abs(moved - roll(base))) <= TIGHT
    for kernels, wraps, dils in (((3, 3, 5), (True, True, True), (1, 1, 1)),
                                 ((3, 3, 3), (True, False, True), (1, 1, 2)),
                                 ((1, 3, 3), (False, True, True), (1, 2, 1))):
        got = O.attention(q, k, v, 0.5, "na3d", O.NA3D(gd, gh, gw, *kernels, *wraps, *dils))
        want = _pad_crop(q, k, v, 0.5, (gd, gh, gw), kernels, wraps, dils)
        assert np.max(np.abs(got - want)) <= TIGHT, (kernels, wraps, dils)


def pin_na3d_sdpa():
    B, H, d = 1, 2, 8
    p = O.NA3D(3, 4, 5, 3, 3, 3, True, False, True, 1, 1, 2)
    N = 60
    q, k, v = _rand(230, B, H, N, d), _rand(231, B, H, N, d), _rand(232, B, H, N, d)
    m = np.zeros((N, N), dtype=bool)
    for i in range(N):
        m[i, _window_keys(i, "na3d", N, p)] = True
    F = torch.nn.functional.scaled_dot_product_attention
    with torch.nn.attention.sdpa_kernel(torch.nn.attention.SDPBackend.MATH):
        ref = F(*(torch.from_numpy(x) for x in (q, k, v)), attn_mask=torch.from_numpy(m), scale=0.35).numpy()
    assert np.max(np.abs(O.attention(q, k, v, 0.35, "na3d", p) - ref)) <= 1e-10


# ---------------------------------------------------------------- backward
def pin_backward_autograd_sdpa():
    """Gradients against torch autograd through SDPA's math path in float64 (none, causal square and
    cross, boolean window masks in 2D and 3D, a negative scale)."""
    B, H, d = 1, 2, 6
    F = torch.nn.functional.scaled_dot_product_attention
    cases = (("none", None, 14, 14, 0.4), ("causal", None, 14, 14, 0.4), ("none", None, 9, 17, -0.3),
             ("causal", None, 12, 7, 0.5), ("na2d", O.NA2D(4, 5, 3, 3, True, False, 1, 1), 20, 20, 0.45),
             ("na3d", O.NA3D(3, 3, 5, 3, 1, 3, False, True, True, 1, 1, 2), 45, 45, 0.45))
    for mask, na, nq, nkv, scale in cases:
        q, k, v = _rand(240, B, H, nq, d), _rand(241, B, H, nkv, d), _rand(242, B, H, nkv, d)
        do = _rand(243, B, H, nq, d)
        tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
        kw = {}
        if mask == "causal":
            kw["is_causal"] = True
        elif mask in ("na2d", "na3d"):
            m = np.zeros((nq, nkv), dtype=bool)
            for i in range(nq):
                m[i, _window_keys(i, mask, nq, na, nkv)] = True
            kw["attn_mask"] = torch.from_numpy(m)
        with torch.nn.attention.sdpa_kernel(torch.nn.attention.SDPBackend.MATH):
            out = F(tq, tk, tv, scale=scale, **kw)
        out.backward(torch.from_numpy(do))
        got = O.attention_backward(q, k, v, do, scale, mask, na)
        for g, t in zip(got, (tq, tk, tv)):
            assert np.max(np.abs(g - t.grad.numpy())) <= 1e-10, (mask, nq, nkv)


def pin_backward_finite_differences():
    """Central differences of L = sum(dO * O) through the pure-Python forward, at every input element."""
    for mask, na, n, nkv in (("causal", None, 4, 4), ("none", None, 3, 5), ("na2d", O.NA2D(2, 3, 1, 3, True, True), 6, 6)):
        d = 3
        q, k, v = _rand(250, 1, 1, n, d), _rand(251, 1, 1, nkv, d), _rand(252, 1, 1, nkv, d)
        do = _rand(253, 1, 1, n, d)
        scale = 0.7
        dq, dk, dv = O.attention_backward(q, k, v, do, scale, mask, na)

        def loss(qq, kk, vv):
            out = brute_head(qq[0, 0].tolist(), kk[0, 0].tolist(), vv[0, 0].tolist(), scale, mask, na)
            return math.fsum((out * do[0, 0]).ravel().tolist())

        h = 1e-5
        for which, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            for idx in np.ndindex(arr.shape):
                plus, minus = arr.copy(), arr.copy()
                plus[idx] += h
                minus[idx] -= h
                args_p = {"q": (plus, k, v), "k": (q, plus, v), "v": (q, k, plus)}[which]
                args_m = {"q": (minus, k, v), "k": (q, minus, v), "v": (q, k, minus)}[which]
                fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
                assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(fd)), (mask, which, idx, fd, grad[idx])


def pin_backward_identities():
    """Rows of P sum to 1, so the key gradients of V add up to the output gradients; scale = 0 makes
    dQ and dK vanish and dV the window-count-weighted sums of dO."""
    B, H, d = 1, 2, 5
    for mask, na, nq, nkv in (("none", None, 10, 13), ("causal", None, 11, 11),
                              ("na2d", O.NA2D(4, 5, 3, 3, True, True, 1, 1), 20, 20),
                              ("na3d", O.NA3D(3, 4, 5, 3, 3, 3, True, False, True, 1, 1, 2), 60, 60)):
        q, k, v = _rand(260, B, H, nq, d), _rand(261, B, H, nkv, d), _rand(262, B, H, nkv, d)
        do = _rand(263, B, H, nq, d)
        dq, dk, dv = O.attention_backward(q, k, v, do, 0.6, mask, na)
        assert np.max(np.abs(dv.sum(axis=2) - do.sum(axis=2))) <= TIGHT, mask
        # dQ_i = scale * sum_j dS_ij k_j with sum_j dS_ij = 0: adding one vector to every key changes nothing
        shift = k + _rand(264, 1, 1, 1, d)
        dq2, _, _ = O.attention_backward(q, shift, v, do, 0.6, mask, na)
        assert np.max(np.abs(dq2 - dq)) <= 1e-10, mask
        dq0, dk0, dv0 = O.attention_backward(q, k, v, do, 0.0, mask, na)
        assert np.all(dq0 == 0.0) and np.all(dk0 == 0.0)
        want = np.zeros_like(dv0)
        for i in range(nq):
            keys = _window_keys(i, mask, nq, na, nkv)
            want[:, :, keys] += do[:, :, i:i + 1] / len(keys)
        assert np.max(np.abs(dv0 - want)) <= TIGHT, mask


def pin_backward_wrap_equals_pad_fold():
    """NATTEN issue 142's 1D backward recipe in 2D: pad q, k, v circularly by r, pad dO with zeros, take the
    clamped window's gradients on the padded grid, crop, and fold the margins back onto the cells they copy."""
    B, H, d = 1, 2, 4
    for gh, gw, kh, kw in ((5, 6, 3, 3), (6, 7, 5, 3)):
        N = gh * gw
        q, k, v = _rand(270, B, H, N, d), _rand(271, B, H, N, d), _rand(272, B, H, N, d)
        do = _rand(273, B, H, N, d)
        want = O.attention_backward(q, k, v, do, 0.5, "na2d", O.NA2D(gh, gw, kh, kw, True, True))
        rh, rw = kh // 2, kw // 2
        ph, pw = gh + 2 * rh, gw + 2 * rw
        grid = lambda t: t.reshape(B, H, gh, gw, d)
        pad = lambda t, mode: np.pad(grid(t), ((0, 0), (0, 0), (rh, rh), (rw, rw), (0, 0)), mode=mode).reshape(B, H, ph * pw, d)
        got = O.attention_backward(pad(q, "wrap"), pad(k, "wrap"), pad(v, "wrap"), pad(do, "constant"), 0.5, "na2d",
                                   O.NA2D(ph, pw, kh, kw, False, False))

        def fold(x):
            x = x.reshape(B, H, ph, pw, d).copy()
            for ax, r, n in ((2, rh, gh), (3, rw, gw)):
                if r == 0:
                    continue
                core = [slice(None)] * 5
                lo, hi = list(core), list(core)
                lo[ax], hi[ax] = slice(r, 2 * r), slice(n, n + r)             # cells the margins copy
                top, bot = list(core), list(core)
                top[ax], bot[ax] = slice(n + r, n + 2 * r), slice(0, r)        # the margins
                x[tuple(lo)] += x[tuple(top)]
                x[tuple(hi)] += x[tuple(bot)]
            return x[:, :, rh:rh + gh, rw:rw + gw].reshape(B, H, N, d)

        for g, w in zip(got, want):
            assert np.max(np.abs(fold(g) - w)) <= TIGHT, (gh, gw, kh, kw)


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
    pin_logsumexp_uniform_is_log_count,
    pin_logsumexp_torch,
    pin_cross_attention_sdpa,
    pin_cross_attention_uniform_and_brute,
    pin_dilation_is_undilated_window_on_subgrids,
    pin_dilated_wrap_equals_pad_then_crop,
    pin_na3d_depth_one_is_na2d,
    pin_na3d_brute_force,
    pin_na3d_uniform_box_filter,
    pin_na3d_translation_and_pad_crop,
    pin_na3d_sdpa,
    pin_backward_autograd_sdpa,
    pin_backward_finite_differences,
    pin_backward_identities,
    pin_backward_wrap_equals_pad_fold,
]

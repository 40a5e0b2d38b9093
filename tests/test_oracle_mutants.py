"""Plant plausible mistakes in the CPU oracle and check that a pin catches each.

Each mutant replaces one internal step of oracle.dense (a dropped term, a
wrong sign or index, a transposed operand, an off-by-one window). The test
passes when at least one pin raises for every mutant; the unmutated oracle
passing every pin is checked in test_oracle_pins.py.
"""
import numpy as np
import pytest

import oracle.dense as O
import oracle_pins

_orig_axis = O._axis_allowed


def _axis_wrap_off_by_one(cq, ck, length, kernel, wrap, dil=1):
    if wrap:
        r = kernel // 2
        d = np.minimum(np.mod(ck[None, :] - cq[:, None], length), np.mod(cq[:, None] - ck[None, :], length))
        return (d < r * dil) & (d % dil == 0)
    return _orig_axis(cq, ck, length, kernel, wrap, dil)


def _axis_one_sided_wrap(cq, ck, length, kernel, wrap, dil=1):
    if wrap:
        fwd = np.mod(ck[None, :] - cq[:, None], length)
        return (fwd <= (kernel // 2) * dil) & (fwd % dil == 0)
    return _orig_axis(cq, ck, length, kernel, wrap, dil)


def _axis_clamp_unclipped(cq, ck, length, kernel, wrap, dil=1):
    if not wrap and dil == 1:
        start = cq[:, None] - kernel // 2
        return (ck[None, :] >= start) & (ck[None, :] < start + kernel)
    return _orig_axis(cq, ck, length, kernel, wrap, dil)


def _axis_dilation_ignored(cq, ck, length, kernel, wrap, dil=1):
    return _orig_axis(cq, ck, length, kernel, wrap, 1)


def _axis_wrap_dilation_no_residue(cq, ck, length, kernel, wrap, dil=1):
    if wrap:
        r = kernel // 2
        fwd = np.mod(ck[None, :] - cq[:, None], length)
        bwd = np.mod(cq[:, None] - ck[None, :], length)
        return (fwd <= r * dil) | (bwd <= r * dil)
    return _orig_axis(cq, ck, length, kernel, wrap, dil)


def _axis_clamp_dilation_no_residue(cq, ck, length, kernel, wrap, dil=1):
    if not wrap:
        g = np.mod(cq[:, None], dil)
        sub_len = (length - 1 - g) // dil + 1
        start = np.clip(cq[:, None] // dil - kernel // 2, 0, sub_len - kernel)
        j = ck[None, :] // dil
        return (j >= start) & (j < start + kernel)
    return _orig_axis(cq, ck, length, kernel, wrap, dil)


def _axis_clamp_dilation_short_subgrid(cq, ck, length, kernel, wrap, dil=1):
    if not wrap:
        g = np.mod(cq[:, None], dil)
        sub_len = length // dil          # wrong for the residues that hold one more cell
        start = np.clip(cq[:, None] // dil - kernel // 2, 0, sub_len - kernel)
        j = ck[None, :] // dil
        return (np.mod(ck[None, :], dil) == g) & (j >= start) & (j < start + kernel)
    return _orig_axis(cq, ck, length, kernel, wrap, dil)


def _axis_clamp_dilation_window_in_cells(cq, ck, length, kernel, wrap, dil=1):
    if not wrap:
        # a clamped window of kernel*dil cells around the query, stepping by dil
        start = np.clip(cq[:, None] - (kernel // 2) * dil, 0, length - kernel * dil)
        off = ck[None, :] - start
        return (off >= 0) & (off < kernel * dil) & (off % dil == 0)
    return _orig_axis(cq, ck, length, kernel, wrap, dil)


def _softmax_no_max(s):
    m = np.zeros((s.shape[0], 1))
    p = np.exp(s)
    return m, p, np.sum(p, axis=1, keepdims=True)


def _softmax_wrong_axis(s):
    m = np.max(s, axis=1, keepdims=True)
    m = np.where(np.isneginf(m), 0.0, m)
    p = np.exp(s - m)
    return m, p, np.sum(p, axis=0)[:, None]   # sums over queries instead of keys


_orig_allowed = O.allowed


def _allowed_causal_strict(N, mask="none", na=None, rows=None, n_kv=None):
    a = _orig_allowed(N, mask, na, rows, n_kv)
    if mask == "causal":
        qi = np.arange(N) if rows is None else np.asarray(rows)
        a = np.arange(a.shape[1])[None, :] < qi[:, None]
    return a


def _allowed_causal_bottom_right(N, mask="none", na=None, rows=None, n_kv=None):
    a = _orig_allowed(N, mask, na, rows, n_kv)
    if mask == "causal":
        qi = np.arange(N) if rows is None else np.asarray(rows)
        a = np.arange(a.shape[1])[None, :] <= qi[:, None] + (a.shape[1] - N)
    return a


def _allowed_grid_transposed(N, mask="none", na=None, rows=None, n_kv=None):
    if mask != "na2d":
        return _orig_allowed(N, mask, na, rows, n_kv)
    p = na
    qi = np.arange(N) if rows is None else np.asarray(rows)
    kj = np.arange(N)
    yq, xq = np.divmod(qi, p.grid_h)   # wrong: divides by the row count
    yk, xk = np.divmod(kj, p.grid_h)
    return (O._axis_allowed(yq, yk, p.grid_h, p.kernel_h, p.wrap_h, p.dil_h)
            & O._axis_allowed(xq, xk, p.grid_w, p.kernel_w, p.wrap_w, p.dil_w))


def _allowed_3d_axes_reversed(N, mask="none", na=None, rows=None, n_kv=None):
    if mask != "na3d":
        return _orig_allowed(N, mask, na, rows, n_kv)
    qi = np.arange(N) if rows is None else np.asarray(rows)
    kj = np.arange(N)
    grid = na.grid()[::-1]              # wrong: column-major token order
    cq, ck = np.unravel_index(qi, grid), np.unravel_index(kj, grid)
    out = np.ones((qi.size, N), dtype=bool)
    for a, (length, kern, wrap, dil) in enumerate(na.axes()[::-1]):
        out &= O._axis_allowed(cq[a], ck[a], length, kern, wrap, dil)
    return out


def _allowed_3d_depth_ignored(N, mask="none", na=None, rows=None, n_kv=None):
    if mask != "na3d":
        return _orig_allowed(N, mask, na, rows, n_kv)
    qi = np.arange(N) if rows is None else np.asarray(rows)
    kj = np.arange(N)
    cq, ck = np.unravel_index(qi, na.grid()), np.unravel_index(kj, na.grid())
    out = np.ones((qi.size, N), dtype=bool)
    for a, (length, kern, wrap, dil) in enumerate(na.axes()):
        if a > 0:
            out &= O._axis_allowed(cq[a], ck[a], length, kern, wrap, dil)
    return out


def _lse_log2(m, l):
    return np.where(l > 0, m + np.log2(np.where(l > 0, l, 1.0)), -np.inf)[:, 0]


def _lse_no_max(m, l):
    return np.where(l > 0, np.log(np.where(l > 0, l, 1.0)), -np.inf)[:, 0]


def _lse_max_only(m, l):
    return np.where(l > 0, m, -np.inf)[:, 0]


MUTANTS = {
    "scale_dropped": ("_scores", lambda q, k, s: q @ k.T),
    "scale_squared": ("_scores", lambda q, k, s: s * s * (q @ k.T)),
    "scores_transposed": ("_scores", lambda q, k, s: s * (k @ q.T)),
    "mask_ignored": ("_apply_mask", lambda s, a: s),
    "mask_inverted": ("_apply_mask", lambda s, a: np.where(a, -np.inf, s)),
    "mask_zero_not_neginf": ("_apply_mask", lambda s, a: np.where(a, s, 0.0)),
    "no_max_subtraction": ("_softmax_parts", _softmax_no_max),
    "row_sum_wrong_axis": ("_softmax_parts", _softmax_wrong_axis),
    "no_division": ("_combine", lambda p, l, v: p @ v),
    "no_empty_row_guard": ("_combine", lambda p, l, v: (p @ v) / l),
    "values_reversed": ("_combine", lambda p, l, v: (p @ v[::-1]) / l),
    "divide_by_sqrt_l": ("_combine", lambda p, l, v: (p @ v) / np.sqrt(l)),
    "wrap_off_by_one": ("_axis_allowed", _axis_wrap_off_by_one),
    "wrap_one_sided": ("_axis_allowed", _axis_one_sided_wrap),
    "clamp_unclipped": ("_axis_allowed", _axis_clamp_unclipped),
    "causal_strict": ("allowed", _allowed_causal_strict),
    "causal_bottom_right": ("allowed", _allowed_causal_bottom_right),
    "grid_transposed": ("allowed", _allowed_grid_transposed),
    "grid3d_axes_reversed": ("allowed", _allowed_3d_axes_reversed),
    "grid3d_depth_ignored": ("allowed", _allowed_3d_depth_ignored),
    "dilation_ignored": ("_axis_allowed", _axis_dilation_ignored),
    "wrap_dilation_no_residue": ("_axis_allowed", _axis_wrap_dilation_no_residue),
    "clamp_dilation_no_residue": ("_axis_allowed", _axis_clamp_dilation_no_residue),
    "clamp_dilation_short_subgrid": ("_axis_allowed", _axis_clamp_dilation_short_subgrid),
    "clamp_dilation_window_in_cells": ("_axis_allowed", _axis_clamp_dilation_window_in_cells),
    "lse_log2": ("_logsumexp", _lse_log2),
    "lse_no_max": ("_logsumexp", _lse_no_max),
    "lse_max_only": ("_logsumexp", _lse_max_only),
    "softmax_grad_no_rowsum": ("_softmax_grad", lambda p, dp: p * dp),
    "softmax_grad_wrong_axis": ("_softmax_grad", lambda p, dp: p * (dp - np.sum(p * dp, axis=0, keepdims=True))),
    "softmax_grad_sign": ("_softmax_grad", lambda p, dp: p * (np.sum(p * dp, axis=1, keepdims=True) - dp)),
    "grad_v_untransposed": ("_grad_v", lambda p, do: p @ do),
    "grad_q_no_scale": ("_grad_q", lambda ds, k, s: ds @ k),
    "grad_k_untransposed_ds": ("_grad_k", lambda ds, q, s: s * (ds @ q)),
    "grad_k_scale_squared": ("_grad_k", lambda ds, q, s: s * s * (ds.T @ q)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    with np.errstate(all="ignore"):
        for pin in oracle_pins.ALL_PINS:
            try:
                pin()
            except TypeError:  # a call the mutant cannot take is not a catch
                raise
            except Exception as e:  # an assertion, or a shape error the mistake causes
                caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught mutant {name}"

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


def _axis_wrap_off_by_one(cq, ck, length, kernel, wrap):
    if wrap:
        r = kernel // 2
        d = np.minimum(np.mod(ck[None, :] - cq[:, None], length), np.mod(cq[:, None] - ck[None, :], length))
        return d < r
    return _orig_axis(cq, ck, length, kernel, wrap)


def _axis_one_sided_wrap(cq, ck, length, kernel, wrap):
    if wrap:
        return np.mod(ck[None, :] - cq[:, None], length) <= kernel // 2
    return _orig_axis(cq, ck, length, kernel, wrap)


def _axis_clamp_unclipped(cq, ck, length, kernel, wrap):
    if not wrap:
        start = cq[:, None] - kernel // 2
        return (ck[None, :] >= start) & (ck[None, :] < start + kernel)
    return _orig_axis(cq, ck, length, kernel, wrap)


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


def _allowed_causal_strict(N, mask="none", na2d=None, rows=None):
    a = _orig_allowed(N, mask, na2d, rows)
    if mask == "causal":
        qi = np.arange(N) if rows is None else np.asarray(rows)
        a = np.arange(N)[None, :] < qi[:, None]
    return a


def _allowed_grid_transposed(N, mask="none", na2d=None, rows=None):
    if mask != "na2d":
        return _orig_allowed(N, mask, na2d, rows)
    p = na2d
    qi = np.arange(N) if rows is None else np.asarray(rows)
    kj = np.arange(N)
    yq, xq = np.divmod(qi, p.grid_h)   # wrong: divides by the row count
    yk, xk = np.divmod(kj, p.grid_h)
    return (O._axis_allowed(yq, yk, p.grid_h, p.kernel_h, p.wrap_h)
            & O._axis_allowed(xq, xk, p.grid_w, p.kernel_w, p.wrap_w))


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
    "grid_transposed": ("allowed", _allowed_grid_transposed),
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
            except Exception as e:  # an assertion, or a shape error the mistake causes
                caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught mutant {name}"

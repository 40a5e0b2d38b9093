"""The tolerance argument of the parity tests, checked on the CPU.

tests/kernel_model.py re-enacts the float32 / bfloat16 arithmetic of the fused
forward kernel. Against the float64 oracle these tests show:

  * on the benchmark inputs (N(0, 1) q, k, v, scale 1/sqrt(d)) the modelled
    arithmetic stays well inside the parity bound 4e-3 max(1, |ref|) + 2e-3;
  * on sharper rows (score std 4 or 8) bfloat16 probabilities alone can pass that
    bound on single elements, while every element stays inside the bound derived
    from the arithmetic (kernel_model.derived_bound); the GPU parity tests of such
    inputs use max(parity bound, derived);
  * the model reproduces the one element the GPU gave outside the parity
    bound (a dilated 16x20 window at d = 128, seed 10022): same bfloat16 value;
  * float16 probabilities and values (modelled) meet the parity bound on the
    same sharp inputs.
"""
import math

import numpy as np
import pytest

import oracle
import workloads
from kernel_model import U_FP16, derived_bound, model_forward


def _ns(ref):
    return 4e-3 * np.maximum(1.0, np.abs(ref)) + 2e-3


def _f64(*ts):
    return [t.float().numpy().astype(np.float64) for t in ts]


def _ratios(B, H, N, d, seed, scale, q_gain=1.0, mask="none", na=None, bn=128, p_format="bf16", cross=False):
    """(worst err / parity bound, worst err / max(parity bound, derived)) of the model against the oracle."""
    q, k, v = (workloads.make_qkv_cross(B, H, N, N, d, seed, q_gain) if cross
               else workloads.make_qkv(B, H, N, d, seed, q_gain))
    qf, kf, vf = _f64(q, k, v)
    allow = oracle.allowed(N, mask, na)
    got = model_forward(qf, kf, vf, scale, allow, bn=bn, p_format=p_format)
    ref = oracle.attention(qf, kf, vf, scale, mask, na)
    p = oracle.probs(qf, kf, scale, mask, na)
    u_p = {"fp16": U_FP16, "bf16x2": 2.0 ** -16}.get(p_format, 2.0 ** -8)
    worst_ns, worst_derived = 0.0, 0.0
    for b in range(B):
        for h in range(H):
            err = np.abs(got[b, h] - ref[b, h])
            bound = np.maximum(_ns(ref[b, h]), derived_bound(p[b, h], vf[b, h], ref[b, h], u_p))
            worst_ns = max(worst_ns, float((err / _ns(ref[b, h])).max()))
            worst_derived = max(worst_derived, float((err / bound).max()))
    return worst_ns, worst_derived


@pytest.mark.parametrize("N,mask,seed", [(256, "none", 6801), (1024, "none", 11), (1024, "causal", 12)])
def test_benchmark_inputs_meet_parity_bound(N, mask, seed):
    worst_ns, worst_derived = _ratios(1, 2, N, 64, seed, 0.125, mask=mask)
    assert worst_ns < 0.8 and worst_derived < 0.8, (worst_ns, worst_derived)


# score std 4 (Q x 4 at scale 1/8) and std 8 (scale 1): bfloat16 probabilities pass the parity
# bound on single elements for some seeds (the seeds below, 1.16 and 1.07 of it), never the derived one
@pytest.mark.parametrize("scale,q_gain,seed,exceeds", [
    (0.125, 4.0, 2000, False), (0.125, 4.0, 2003, True), (1.0, 1.0, 2000, True), (1.0, 1.0, 2001, False)])
@pytest.mark.parametrize("mask", ["none", "causal"])
def test_sharp_rows_within_derived_bound(scale, q_gain, seed, exceeds, mask):
    worst_ns, worst_derived = _ratios(2, 3, 300, 64, seed, scale, q_gain, mask)
    assert worst_derived < 0.9, worst_derived
    if mask == "none":
        assert (worst_ns > 1.0) == exceeds, worst_ns


@pytest.mark.parametrize("scale,q_gain,seed", [(0.125, 4.0, 2003), (1.0, 1.0, 2000), (0.125, 4.0, 2001)])
@pytest.mark.parametrize("p_format", ["fp16", "bf16x2"])
def test_wider_probabilities_meet_parity_bound(scale, q_gain, seed, p_format):
    """Either float16 probabilities and values, or P kept as two bfloat16 parts (the variant
    timed on the GPU at 0.56-0.73x of the kernel's throughput), bring the sharp rows inside the
    parity bound: the output's own bfloat16 rounding is then the main error."""
    worst_ns, _ = _ratios(2, 3, 300, 64, seed, scale, q_gain, p_format=p_format)
    assert worst_ns < 0.85, worst_ns


def test_reproduces_recorded_dilated_element():
    """A dilated 16x20 grid, 3x5 window (dilation 2, 3), both axes wrapped, d = 128 (64-key tiles),
    seed 10022: the GPU gave 1.015625 at (b 0, h 1, query 231, d 36) against an exact 1.00924
    (1.058 of the parity bound). The modelled arithmetic gives the same bfloat16 value, and the
    derived bound there is about three times the error."""
    N, d = 320, 128
    q, k, v = workloads.make_qkv_cross(1, 2, N, N, d, 10022)
    qf, kf, vf = _f64(q, k, v)
    na = oracle.NA2D(16, 20, 3, 5, True, True, 2, 3)
    scale = 1 / math.sqrt(d)
    got = model_forward(qf, kf, vf, scale, oracle.allowed(N, "na2d", na), bn=64)
    ref = oracle.attention(qf, kf, vf, scale, "na2d", na)
    idx = (0, 1, 231, 36)
    assert got[idx] == 1.015625
    assert abs(ref[idx] - 1.00924) < 1e-5
    assert abs(got[idx] - ref[idx]) / _ns(ref[idx]) == pytest.approx(1.058, abs=1e-3)
    bound = derived_bound(oracle.probs(qf, kf, scale, "na2d", na)[0, 1], vf[0, 1], ref[0, 1])[231, 36]
    assert abs(got[idx] - ref[idx]) < 0.4 * bound


def test_derived_bound_is_not_vacuous():
    """The derived bound follows the rows: about the parity bound's size on flat benchmark rows, several
    times larger where few keys with different values share the weight."""
    q, k, v = workloads.make_qkv(1, 1, 256, 64, 6801)
    qf, kf, vf = _f64(q, k, v)
    for scale, lo, hi in ((0.125, 0.5, 2.0), (1.0, 1.5, 5.0)):
        ref = oracle.attention(qf, kf, vf, scale)
        ratio = derived_bound(oracle.probs(qf, kf, scale)[0, 0], vf[0, 0], ref[0, 0]) / _ns(ref[0, 0])
        assert lo < ratio.max() < hi, (scale, ratio.max())

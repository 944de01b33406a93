"""Pins of the oracle's exp, SwiGLU, ReLU^2 and sigmoid against exact math.

The oracle's exp is a fixed binary32 evaluation (argument reduction + Taylor
polynomial); here it is checked against float64 ``math.exp`` (error far below a
binary32 ulp) with an ulp bound, plus its defined boundary behaviour.  SwiGLU is
silu(gate)*up ("Building Custom TensorRT-LLM Plugins for Low-Latency FP8
Inference at Scale", "The Cost of Non-Fused Quantization": X [N,2H] -> Y [N,H]);
ReLU^2 is the activation of "Nvfp4 A16 Blackwell Moe Runner".
"""
import math

import numpy as np
import pytest


def ulp32(x: float) -> float:
    x = abs(np.float32(x))
    return float(np.nextafter(x, np.float32(np.inf)) - x)


def _sweep(lo, hi, n, seed=0):
    rng = np.random.default_rng(seed)
    xs = np.concatenate([np.linspace(lo, hi, n), rng.uniform(lo, hi, n)]).astype(np.float32)
    return xs


def test_exp_ulp_bound(oracle):
    worst = 0.0
    for x in _sweep(-87.0, 88.7, 20000):
        got = oracle.exp_f32(float(x))
        want = math.exp(float(x))
        err = abs(got - want) / ulp32(want)
        worst = max(worst, err)
    assert worst < 1.0, worst       # measured 0.89 ulp on 2e5 random points


def test_exp_special_points(oracle):
    assert oracle.exp_f32(0.0) == 1.0
    assert oracle.exp_f32(-0.0) == 1.0
    assert math.isinf(oracle.exp_f32(88.76)) and math.isinf(oracle.exp_f32(1e30))
    assert oracle.exp_f32(-87.01) == 0.0 and oracle.exp_f32(-1e30) == 0.0
    # last finite region: e^88.72 is just below FLT_MAX
    x = float(np.float32(88.72))
    v = oracle.exp_f32(x)
    assert math.isfinite(v) and abs(v - math.exp(x)) <= 2 * ulp32(v)
    # smallest accepted argument still gives a normal number
    assert oracle.exp_f32(-87.0) >= 2.0 ** -126


def test_exp_monotone(oracle):
    xs = np.sort(_sweep(-20.0, 20.0, 5000, seed=1))
    ys = [oracle.exp_f32(float(x)) for x in xs]
    assert all(a <= b for a, b in zip(ys, ys[1:]))


def test_swiglu_close_to_exact(oracle):
    rng = np.random.default_rng(2)
    g = (rng.standard_normal(20000) * 4).astype(np.float32)
    u = (rng.standard_normal(20000) * 4).astype(np.float32)
    for gi, ui in zip(g, u):
        got = oracle.swiglu_f32(float(gi), float(ui))
        want = float(gi) / (1.0 + math.exp(-float(gi))) * float(ui)
        assert abs(got - want) <= 4 * ulp32(want) + 1e-44, (gi, ui, got, want)


def test_swiglu_special_cases(oracle):
    assert oracle.swiglu_f32(0.0, 5.0) == 0.0
    assert oracle.swiglu_f32(3.0, 0.0) == 0.0
    # large positive gate: silu(g) == g exactly (exp(-g) underflows to 0)
    assert oracle.swiglu_f32(100.0, 2.0) == 200.0
    # large negative gate: 1 + exp(-g) overflows, silu -> -0
    v = oracle.swiglu_f32(-100.0, 2.0)
    assert v == 0.0 and math.copysign(1.0, v) < 0


def test_relu2_is_correctly_rounded_square(oracle):
    rng = np.random.default_rng(3)
    xs = (rng.standard_normal(20000) * 30).astype(np.float32)
    for x in xs:
        r = max(float(x), 0.0)
        # the product of two binary32 numbers is exact in binary64
        assert oracle.relu2_f32(float(x)) == float(np.float32(r * r))
    assert oracle.relu2_f32(-0.0) == 0.0 and math.copysign(1, oracle.relu2_f32(-0.0)) > 0


def test_sigmoid_close_to_exact(oracle):
    for x in _sweep(-30.0, 30.0, 5000, seed=4):
        got = oracle.sigmoid_f32(float(x))
        want = 1.0 / (1.0 + math.exp(-float(x)))
        assert abs(got - want) <= 3 * ulp32(want), x

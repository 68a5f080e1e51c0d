"""Host checks of closed-form device math that the kernels inline (no GPU needed).

The bf16 GELU epilogue evaluates GELU(x) ~= x * sigmoid(x q(x^2)) with a fitted
quadratic q; its constants are read from the device source and the formula is
evaluated here in float32, step by step as the kernel does, against the exact
erf form in float64."""
import os
import re

import numpy as np
from scipy.special import erf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COMMON = os.path.join(ROOT, "cem_jepa_predictor_amd", "csrc", "common.hpp")


def _gelu_bf16_constants():
    src = open(COMMON).read()
    body = src[src.index("float gelu_bf16_path(float x)"):]
    body = body[:body.index("\n}\n")]
    cap = float(re.search(r"fminf\(x \* x, ([0-9.e+-]+)f\)", body).group(1))
    c2, c1, c0 = (float(v) for v in re.search(
        r"fmaf\(fmaf\(u, ([0-9.e+-]+)f, ([0-9.e+-]+)f\), u, ([0-9.e+-]+)f\)", body).groups())
    return cap, c0, c1, c2


def _gelu_bf16_path(x):
    cap, c0, c1, c2 = (np.float32(v) for v in _gelu_bf16_constants())
    with np.errstate(over="ignore"):
        u = np.minimum(x * x, cap)
        s = (np.float32(c2) * u + c1) * u + c0
        return x * (np.float32(1) / (np.float32(1) + np.exp2(x * s)))


def test_bf16_gelu_within_bound_of_exact():
    x = np.concatenate([np.linspace(-12, 12, 480001), [-1e4, -80.0, 80.0, 1e4]]).astype(np.float32)
    got = _gelu_bf16_path(x).astype(np.float64)
    xd = x.astype(np.float64)
    want = 0.5 * xd * (1.0 + erf(xd / np.sqrt(2.0)))
    assert np.abs(got - want).max() <= 3e-5
    # the bf16 rounding bound (half the spacing) at GELU's minimum is 2^-11
    assert np.abs(got - want).max() < 2.0 ** -11 / 15


def test_bf16_gelu_cap_keeps_the_sigmoid_saturated():
    cap, c0, c1, c2 = _gelu_bf16_constants()
    q_cap = (c2 * cap + c1) * cap + c0            # = -log2(e) q(cap)
    assert q_cap < 0                              # q stays positive up to the cap
    u = np.linspace(0, cap, 10001)
    assert np.all((c2 * u + c1) * u + c0 < 0)
    # past the cap x q(cap) >= sqrt(cap) q(cap): sigmoid within 1e-7 of 1
    assert 2.0 ** (np.sqrt(cap) * q_cap) < 1e-7

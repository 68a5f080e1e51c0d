"""Host checks of closed-form device math that the kernels inline (no GPU needed).

The bf16 GELU epilogue evaluates GELU(x) ~= x * sigmoid(x q(x^2)) with a fitted
quadratic q; its constants are read from the device source and the formula is
evaluated here in float32, step by step as the kernel does, against the exact
erf form in float64.  The LayerNorm fold of the bf16 projections and the GEMM
tile start's three-part bf16 splits are checked as identities in float64."""
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


def _split3_bf16(v):
    """v = v1 + v2 + v3 with each part rounded to bf16 (nearest even), as the GEMM
    tile start splits its fp32 factors."""
    def rne_bf16(a):
        u = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
        u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
        return u.astype(np.uint32).view(np.float32)
    v = np.asarray(v, np.float32)
    v1 = rne_bf16(v)
    r1 = (v - v1).astype(np.float32)
    v2 = rne_bf16(r1)
    v3 = rne_bf16((r1 - v2).astype(np.float32))
    return v1, v2, v3


def test_layernorm_fold_identity():
    """The fold the bf16 projections use (LayerNorm with gain g and shift b before a
    linear layer W, c): LN(x) W + c = rstd (x W' - mean 1^T W') + (c + b W) with
    W' = diag(g) W.  Checked in float64 on rows with a large mean, where the
    subtraction cancels most of x W'."""
    rng = np.random.default_rng(5)
    d, n_out, rows = 256, 96, 40
    x = rng.standard_normal((rows, d)) * 0.7 + rng.standard_normal((rows, 1)) * 6.0
    g = 1.0 + 0.02 * rng.standard_normal(d)
    b = 0.02 * rng.standard_normal(d)
    W = 0.02 * rng.standard_normal((d, n_out))
    c = 0.02 * rng.standard_normal(n_out)
    eps = 1e-5
    mean = x.mean(1, keepdims=True)
    rstd = 1.0 / np.sqrt(((x - mean) ** 2).mean(1, keepdims=True) + eps)
    want = ((x - mean) * rstd * g + b) @ W + c
    Wf = g[:, None] * W
    got = rstd * (x @ Wf - mean * Wf.sum(0)[None, :]) + (c + b @ W)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_tile_start_split_reaches_fp32():
    """The GEMM tile start writes bias / scale - shift * col through one MFMA from
    three-part bf16 splits of each factor (six cross terms per product).  The sum of
    those terms, taken in float64, stays within a few fp32 ulps of the product."""
    rng = np.random.default_rng(6)
    s = (rng.standard_normal(4000) * np.exp2(rng.integers(-20, 20, 4000))).astype(np.float32)
    t = (rng.standard_normal(4000) * np.exp2(rng.integers(-20, 20, 4000))).astype(np.float32)
    s1, s2, s3 = (p.astype(np.float64) for p in _split3_bf16(s))
    t1, t2, t3 = (p.astype(np.float64) for p in _split3_bf16(t))
    assert np.all(s1 + s2 + s3 == s.astype(np.float64))   # the split itself is exact
    approx = s1 * t1 + s1 * t2 + s2 * t1 + s1 * t3 + s2 * t2 + s3 * t1
    exact = s.astype(np.float64) * t.astype(np.float64)
    rel = np.abs(approx - exact) / np.abs(exact)
    assert rel.max() < 2.0 ** -22

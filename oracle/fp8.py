"""OCP 8-bit floating point, E4M3 ("e4m3fn"): the format of the optional fp8
predictor projections.

Encoding (OCP 8-bit Floating Point Specification, E4M3): 1 sign bit, 4
exponent bits with bias 7, 3 mantissa bits; normal values (1 + m/8) 2^(e-7)
for e = 1..15, subnormals (m/8) 2^-6 for e = 0; no infinities; S.1111.111 is
NaN, so the largest finite magnitude is 448 (S.1111.110).  Conversion from a
real value rounds to the nearest representable value, ties to the one with an
even mantissa.  The predictor never converts a magnitude above 448 (its
scales map each row's largest magnitude to 448), so overflow handling is not
needed; encode() rejects it.

Test infrastructure only (the oracle); nothing here is used by the HIP path.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_encode(x) -> np.ndarray:
    """Round each element of x (|x| <= 448, no NaN) to E4M3, ties to even; returns uint8 codes."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.isnan(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_encode: NaN or magnitude above 448")
    sign = np.signbit(x).astype(np.uint8) << 7
    a = np.abs(x)
    out = np.zeros(a.shape, dtype=np.uint8)
    nz = a > 0
    # exponent of the binade holding a (exact: frexp), clamped to the subnormal range
    _, ex = np.frexp(np.where(nz, a, 1.0))
    e = np.maximum(ex - 1, -6)                  # a in [2^e, 2^(e+1)) for normal values
    quantum = np.ldexp(1.0, e - 3)              # spacing of E4M3 values in that binade
    m = np.rint(a / quantum)                    # exact division by a power of two; half to even
    # m in [0, 16]: subnormal binade gives m in [0, 8]; m == 16 carries into the next binade
    carry = m >= 16
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 8, m)
    normal = m >= 8
    code = np.where(normal, ((e + 7).astype(np.int64) << 3) | (m.astype(np.int64) - 8), m.astype(np.int64))
    out[nz] = code[nz].astype(np.uint8)
    return out | sign


def e4m3_decode(code) -> np.ndarray:
    """E4M3 codes (uint8) to float64; NaN codes give NaN."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    v = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return s * v


def quantize_rows(x: np.ndarray):
    """Per-row E4M3 quantization of a float32 matrix [R, C]: scale s_r = amax_r / 448
    (1 for an all-zero row), q = E4M3(min(max(x * (448 / amax_r), -448), 448)), with
    every step in float32 as the device does it.  Returns (codes uint8 [R, C],
    scales float32 [R]); the dequantized row is decode(q) * s_r."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1)
    zero = amax == 0
    safe = np.where(zero, np.float32(448.0), amax).astype(np.float32)
    inv = (np.float32(448.0) / safe).astype(np.float32)
    scale = (safe / np.float32(448.0)).astype(np.float32)
    scale = np.where(zero, np.float32(1.0), scale).astype(np.float32)
    y = (x * inv[:, None]).astype(np.float32)
    y = np.clip(y, np.float32(-448.0), np.float32(448.0))
    return e4m3_encode(y), scale


def quantize_tensor(w: np.ndarray):
    """Per-tensor E4M3 quantization of float32 weights: one scale s = amax / 448 for
    the whole tensor (1 if all zero), codes E4M3(clip(w * (448 / amax))), float32 steps.
    Returns (codes uint8, scale float32); the dequantized tensor is decode(codes) * s."""
    w = np.asarray(w, dtype=np.float32)
    amax = np.float32(np.max(np.abs(w))) if w.size else np.float32(0.0)
    if amax == 0:
        return np.zeros(w.shape, np.uint8), np.float32(1.0)
    inv = np.float32(np.float32(448.0) / amax)
    y = np.clip((w * inv).astype(np.float32), np.float32(-448.0), np.float32(448.0))
    return e4m3_encode(y), np.float32(amax / np.float32(448.0))


def dequantize(codes: np.ndarray, scale) -> np.ndarray:
    """decode(codes) * scale in float64 (scale broadcast: scalar or per row [R, 1])."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)

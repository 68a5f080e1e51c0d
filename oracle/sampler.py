"""Gaussian candidate sampler: Philox-4x32-10 words -> Box-Muller -> clamp.

Page "Real-Time Inference for JEPA World Model Architectures with Ray",
section 01 ("Where the sixteen seconds actually goes"): each round draws the
candidate action sequences from a Gaussian centred on the current best guess.
The pages fix neither the generator layout nor the Gaussian transform; the
readings taken here are:

  * element e = (n*H + h)*A + a of the [N, H, A] sample uses Philox counter
    (e >> 2, round, plan_id, 0) under key (seed low word, seed high word);
  * words (w0, w1) serve elements with e & 3 in {0, 1}, (w2, w3) serve {2, 3};
  * Box-Muller in float64: u1 = (w_even + 1) * 2^-32 in (0, 1],
    u2 = w_odd * 2^-32 in [0, 1), rho = sqrt(-2 ln u1), theta = 2 pi u2,
    z_even = rho cos(theta), z_odd = rho sin(theta), rounded to float32;
  * x = clamp(mu + sigma * z, lo, hi) in float32, one rounding per operation
    (no fused multiply-add), mu and sigma broadcast over candidates.
"""
from __future__ import annotations

import numpy as np

from .philox import philox4x32_10, seed_key

TWO_POW_M32 = 2.0 ** -32


def raw_words(seed: int, rnd: int, plan_id: int, count: int) -> np.ndarray:
    """The Philox words of elements 0..count-1 (one word per element), uint32."""
    n_ctr = (count + 3) // 4
    ctr = np.zeros((n_ctr, 4), dtype=np.uint32)
    ctr[:, 0] = np.arange(n_ctr, dtype=np.uint64).astype(np.uint32)
    ctr[:, 1] = np.uint32(rnd & 0xFFFFFFFF)
    ctr[:, 2] = np.uint32(plan_id & 0xFFFFFFFF)
    return philox4x32_10(ctr, seed_key(seed)).reshape(-1)[:count]


def box_muller(w_even: np.ndarray, w_odd: np.ndarray):
    """float64 Box-Muller of word pairs; returns (z_even, z_odd) float64."""
    u1 = (w_even.astype(np.float64) + 1.0) * TWO_POW_M32
    u2 = w_odd.astype(np.float64) * TWO_POW_M32
    rho = np.sqrt(-2.0 * np.log(u1))
    theta = 2.0 * np.pi * u2
    return rho * np.cos(theta), rho * np.sin(theta)


def gaussian(seed: int, rnd: int, plan_id: int, count: int) -> np.ndarray:
    """Standard normal float32 values of elements 0..count-1."""
    n_ctr = (count + 3) // 4
    words = raw_words(seed, rnd, plan_id, 4 * n_ctr).reshape(n_ctr, 4)
    z = np.empty((n_ctr, 4), dtype=np.float64)
    z[:, 0], z[:, 1] = box_muller(words[:, 0], words[:, 1])
    z[:, 2], z[:, 3] = box_muller(words[:, 2], words[:, 3])
    return z.reshape(-1)[:count].astype(np.float32)


def sample_actions(mu: np.ndarray, sigma: np.ndarray, seed: int, rnd: int, plan_id: int,
                   n: int, lo: float, hi: float) -> np.ndarray:
    """Candidates X [n, H, A] float32 = clamp(mu + sigma * z, lo, hi)."""
    mu = np.asarray(mu, dtype=np.float32)
    sigma = np.asarray(sigma, dtype=np.float32)
    h, a = mu.shape
    z = gaussian(seed, rnd, plan_id, n * h * a).reshape(n, h, a)
    scaled = (sigma[None] * z).astype(np.float32)      # float32 product, rounded
    x = (mu[None] + scaled).astype(np.float32)          # float32 sum, rounded
    return np.minimum(np.maximum(x, np.float32(lo)), np.float32(hi)).astype(np.float32)

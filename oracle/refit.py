"""Refit of the sampling Gaussian on the elites.

Page "Real-Time Inference for JEPA World Model Architectures with Ray",
section 01: the Gaussian is re-centred on the kept candidates each round.
Reading taken: per (step, action dim) mean and population standard deviation
(divide by K) of the elites' clamped samples, accumulated in float64 and
rounded to float32; no floor, momentum or smoothing.
"""
from __future__ import annotations

import numpy as np


def refit(x: np.ndarray, elites: np.ndarray):
    """x [N, H, A] float32 samples, elites [K] indices -> (mu, sigma) float32 [H, A]."""
    sel = np.asarray(x, dtype=np.float64)[np.asarray(elites, dtype=np.int64)]
    mu = sel.mean(axis=0)
    sigma = np.sqrt(((sel - mu[None]) ** 2).mean(axis=0))
    return mu.astype(np.float32), sigma.astype(np.float32)

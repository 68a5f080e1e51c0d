"""L1 energy of a predicted embedding against the goal embedding.

Page "Real-Time Inference for JEPA World Model Architectures with Ray",
section 01: each rollout result is scored against the goal embedding and the
candidates closest to the goal are kept.  The distance is L1; the reading
taken for its normalisation is the mean absolute difference over the P x E
elements (a sum would only rescale; ranking is unchanged).
"""
from __future__ import annotations

import numpy as np


def energy_l1(z_pred: np.ndarray, z_goal: np.ndarray) -> np.ndarray:
    """E[n] = mean_{p,e} |z_pred[n,p,e] - z_goal[p,e]|, float64.  z_pred [n,P,E]."""
    zp = np.asarray(z_pred, dtype=np.float64)
    zg = np.asarray(z_goal, dtype=np.float64)
    return np.abs(zp - zg[None]).reshape(zp.shape[0], -1).mean(axis=1)

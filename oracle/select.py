"""Top-K elite selection.

Page "Real-Time Inference for JEPA World Model Architectures with Ray",
section 01: after scoring, the search keeps the best 80 of 800 candidates.
The pages do not say how ties or non-finite scores are ordered; the reading
taken is a total order on (energy, index) with NaN treated as +infinity and
-0.0 equal to +0.0, so the elite list is unique.  Returned ascending.
"""
from __future__ import annotations

import numpy as np


def topk_elites(energy: np.ndarray, k: int) -> np.ndarray:
    e = np.asarray(energy, dtype=np.float64).copy()
    e[np.isnan(e)] = np.inf
    order = np.argsort(e, kind="stable")        # stable: equal energies keep index order
    return order[:k].astype(np.int32)

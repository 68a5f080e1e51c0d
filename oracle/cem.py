"""The cross-entropy-method planning loop.

Page "Real-Time Inference for JEPA World Model Architectures with Ray",
section 01 ("Where the sixteen seconds actually goes"): one round draws N
candidate action sequences from a Gaussian centred on the current best guess,
pushes each through the predictor, scores it against the goal, keeps the best
K and re-centres the Gaussian on them; R rounds run one after another; only
the first action of the plan is executed.  Reading taken for "the first action
of the winning sequence": the first step of the final refit mean, mu_R[0];
the last round's best candidate index is returned alongside.
"""
from __future__ import annotations

from typing import Callable, Optional

import numpy as np

from .refit import refit
from .sampler import sample_actions
from .select import topk_elites

EnergyFn = Callable[[int, np.ndarray], np.ndarray]


def cem_plan(energy_fn: EnergyFn, n: int, k: int, rounds: int, mu0: np.ndarray,
             sigma0: np.ndarray, seed: int, plan_id: int, lo: float, hi: float,
             select_energy_fn: Optional[EnergyFn] = None):
    """Run the CEM loop.

    energy_fn(r, X) -> E [n] scores the round's samples.  When
    select_energy_fn is given, elites are chosen from its energies instead
    (used to follow another implementation's scores round by round), while
    energy_fn's values are still recorded.
    Returns dict(action, mu, sigma, best_idx, trace lists).
    """
    mu = np.asarray(mu0, dtype=np.float32).copy()
    sigma = np.asarray(sigma0, dtype=np.float32).copy()
    tr = {"x": [], "energy": [], "elites": [], "mu": [mu.copy()], "sigma": [sigma.copy()]}
    elites = None
    for r in range(rounds):
        x = sample_actions(mu, sigma, seed, r, plan_id, n, lo, hi)
        e = energy_fn(r, x)
        e_sel = select_energy_fn(r, x) if select_energy_fn is not None else e
        elites = topk_elites(e_sel, k)
        mu, sigma = refit(x, elites)
        tr["x"].append(x)
        tr["energy"].append(np.asarray(e))
        tr["elites"].append(elites)
        tr["mu"].append(mu.copy())
        tr["sigma"].append(sigma.copy())
    return {"action": mu[0].copy(), "mu": mu, "sigma": sigma,
            "best_idx": int(elites[0]) if elites is not None else -1, "trace": tr}


def predictor_energy_fn(pred, z_obs: np.ndarray, z_goal: np.ndarray, s0: np.ndarray,
                        cached: bool = True) -> EnergyFn:
    """energy_fn that rolls every candidate through the predictor and scores z_H."""
    from .energy import energy_l1

    def fn(_r: int, x: np.ndarray) -> np.ndarray:
        roll = pred.rollout_cached if cached else pred.rollout
        return energy_l1(roll(x, z_obs, s0), z_goal)

    return fn

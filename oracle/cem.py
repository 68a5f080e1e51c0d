"""The cross-entropy-method planning loop.

Page "Real-Time Inference for JEPA World Model Architectures with Ray",
section 01 ("Where the sixteen seconds actually goes"): one round draws N
candidate action sequences from a Gaussian centred on the current best guess,
pushes each through the predictor, scores it against the goal, keeps the best
K and re-centres the Gaussian on them; R rounds run one after another; only
the first action of the plan is executed.  Reading taken for "the first action
of the winning sequence": the first step of the final refit mean, mu_R[0];
the last round's best candidate index is returned alongside.

Section 06 ("Further Optimization", B. "Warm-started CEM"): receding-horizon
control throws away all but the first action; re-using the rest of the plan to
seed the next step's distribution lets each replan converge in fewer rounds.
Reading taken: the next step's mean is the plan's final mean shifted one step
earlier, the vacated last step takes the fresh (mu0, sigma0), and each carried
width is kept but not below a floor (floor = sigma0: widths reset; floor = 0:
widths carried).  The pages fix no floor; they report that on their task a
fresh 3-round search did as well as a warm-started one.
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


def warm_start(mu: np.ndarray, sigma: np.ndarray, mu_fill: float, sigma_fill: float,
               sigma_floor: float):
    """Next control step's Gaussian from a plan's final (mu, sigma) [H, A]
    (section 06 B): step t takes step t + 1 of the plan, the last step starts
    fresh.  Widths below sigma_floor (and NaN widths) become sigma_floor."""
    mu = np.asarray(mu, dtype=np.float32)
    sigma = np.asarray(sigma, dtype=np.float32)
    mu_n = np.empty_like(mu)
    sg_n = np.empty_like(sigma)
    mu_n[:-1] = mu[1:]
    sg_n[:-1] = np.fmax(sigma[1:], np.float32(sigma_floor))
    mu_n[-1] = np.float32(mu_fill)
    sg_n[-1] = np.float32(sigma_fill)
    return mu_n, sg_n


def receding_horizon(energy_for_step: Callable[[int], EnergyFn], steps: int, n: int, k: int,
                     rounds: int, horizon: int, action_dim: int, mu0: float, sigma0: float,
                     seed: int, lo: float, hi: float, warm: bool, sigma_floor: float = 0.0):
    """Closed loop over `steps` control steps (section 06 A/B): at step s plan
    with energy_for_step(s) (plan id s), execute mu_R[0]; the next plan starts
    from warm_start(mu_R, sigma_R) when `warm`, else from the fresh Gaussian.
    Returns the executed actions [steps, A] and the per-step plan results."""
    fresh_mu = np.full((horizon, action_dim), mu0, np.float32)
    fresh_sigma = np.full((horizon, action_dim), sigma0, np.float32)
    mu, sigma = fresh_mu, fresh_sigma
    actions, plans = [], []
    for s in range(steps):
        out = cem_plan(energy_for_step(s), n, k, rounds, mu, sigma, seed, s, lo, hi)
        actions.append(out["action"])
        plans.append(out)
        if warm:
            mu, sigma = warm_start(out["mu"], out["sigma"], mu0, sigma0, sigma_floor)
        else:
            mu, sigma = fresh_mu, fresh_sigma
    return np.stack(actions), plans

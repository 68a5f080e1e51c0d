"""Writes small_reachable_plan.json: the oracle's own CEM plan (float64 predictor) on
the small workload with a reachable goal -- the oracle's predicted frame for a
known action sequence a* -- as the expected value of the GPU test that plans
against the same goal.  Calls only the oracle and the seeded input generators.

    python tests/golden/make_small_reachable_plan.py     (about 5 minutes on 8 cores)

Page "Real-Time Inference for JEPA World Model Architectures with Ray", section 01
(sample, predict, score against the goal, keep the best, refit; execute the first
action of the final Gaussian)."""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from cem_jepa_predictor_amd import inputs  # noqa: E402
from oracle import cem  # noqa: E402
from oracle.predictor import Predictor  # noqa: E402

A_STAR_SEED, A_STAR_SCALE = 99, 0.6


def reachable_goal(pred, wl, z_obs, s0):
    a_star = inputs.make_actions(1, wl.plan.horizon, seed=A_STAR_SEED) * np.float32(A_STAR_SCALE)
    return a_star, pred.rollout_cached(a_star, z_obs, s0)[0].astype(np.float32)


def main():
    wl = inputs.WORKLOADS["small"]
    m, pc = wl.model, wl.plan
    w = inputs.make_weights(m, wl.weight_seed)
    z_obs, _, s0 = inputs.make_embeddings(m, wl.embed_seed)
    pred = Predictor(w, m.layers, m.heads, m.ln_eps)
    a_star, goal = reachable_goal(pred, wl, z_obs, s0)
    H, A = pc.horizon, m.action_dim
    out = cem.cem_plan(cem.predictor_energy_fn(pred, z_obs, goal, s0), pc.n_samples, pc.n_elites,
                       pc.rounds, np.full((H, A), pc.mu0), np.full((H, A), pc.sigma0), pc.seed,
                       pc.plan_id, pc.clamp_lo, pc.clamp_hi)
    rec = {"workload": "small", "a_star_seed": A_STAR_SEED, "a_star_scale": A_STAR_SCALE,
           "a_star": a_star[0].tolist(), "action": np.asarray(out["action"]).tolist(),
           "elites": [np.asarray(e).tolist() for e in out["trace"]["elites"]]}
    with open(os.path.join(HERE, "small_reachable_plan.json"), "w") as f:
        json.dump(rec, f)
    print("action", np.round(out["action"], 4).tolist())


if __name__ == "__main__":
    main()

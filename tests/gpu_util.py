"""Helpers shared by the GPU parity tests (not collected as tests)."""
from __future__ import annotations

import functools
import sys

import numpy as np

from cem_jepa_predictor_amd import _lib, inputs


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_np(t) -> np.ndarray:
    import torch

    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def workload(name: str):
    """A named workload; "sweep_<N>" is the batch-sweep point with N candidates."""
    if name.startswith("sweep_"):
        return inputs.sweep_workload(int(name[len("sweep_"):]))
    return inputs.WORKLOADS[name]


@functools.lru_cache(maxsize=None)
def workload_data(name: str):
    wl = workload(name)
    m = wl.model
    w = inputs.make_weights(m, wl.weight_seed)
    z_obs, z_goal, s0 = inputs.make_embeddings(m, wl.embed_seed)
    return wl, w, inputs.flatten_weights(m, w), z_obs, z_goal, s0


@functools.lru_cache(maxsize=None)
def oracle_predictor(name: str):
    from oracle.predictor import Predictor

    wl, w, _, _, _, _ = workload_data(name)
    return Predictor(w, wl.model.layers, wl.model.heads, wl.model.ln_eps,
                     fp8_projections=wl.model.dtype == "fp8")


_models = {}


def gpu_model(name: str, max_samples: int | None = None):
    key = (name, max_samples)
    if key not in _models:
        wl, _, flat, _, _, _ = workload_data(name)
        _models[key] = _lib.Model(wl.model, flat, max_samples or wl.plan.n_samples)
    return _models[key]


def release_models():
    for m in _models.values():
        m.close()
    _models.clear()


def run_plan(name: str, *, use_graph: bool = True, rounds: int | None = None,
             n: int | None = None, k: int | None = None, seed: int | None = None,
             plan_id: int = 0, horizon: int | None = None, mu_init=None, sigma_init=None,
             z_goal=None, first_round: int = 0):
    """Run cem_plan on the GPU and return outputs and the full trace as numpy.
    mu_init / sigma_init [H, A] replace the fresh Gaussian when given; z_goal [P, E]
    replaces the workload's goal embedding."""
    import torch

    wl, _, _, z_obs, wl_goal, s0 = workload_data(name)
    z_goal = wl_goal if z_goal is None else np.asarray(z_goal, np.float32)
    pc = wl.plan
    N, K = n or pc.n_samples, k or pc.n_elites
    R, H = rounds or pc.rounds, horizon or pc.horizon
    A = wl.model.action_dim
    model = gpu_model(name)
    mu = torch.full((H, A), pc.mu0, dtype=torch.float32, device="cuda")
    sigma = torch.full((H, A), pc.sigma0, dtype=torch.float32, device="cuda")
    if mu_init is not None:
        mu.copy_(torch.from_numpy(np.ascontiguousarray(mu_init, np.float32)))
    if sigma_init is not None:
        sigma.copy_(torch.from_numpy(np.ascontiguousarray(sigma_init, np.float32)))
    action = torch.empty(A, dtype=torch.float32, device="cuda")
    best = torch.empty(1, dtype=torch.int32, device="cuda")
    model.plan(to_dev(z_obs), to_dev(z_goal), to_dev(s0), mu, sigma, action, best, n_samples=N,
               n_elites=K, rounds=R, horizon=H, seed=pc.seed if seed is None else seed,
               plan_id=plan_id, clamp_lo=pc.clamp_lo, clamp_hi=pc.clamp_hi, use_graph=use_graph,
               first_round=first_round)
    tr = {
        "x": model.trace(_lib.TRACE_ACTIONS, torch.empty((R, N, H, A), dtype=torch.float32, device="cuda")),
        "energy": model.trace(_lib.TRACE_ENERGY, torch.empty((R, N), dtype=torch.float32, device="cuda")),
        "elites": model.trace(_lib.TRACE_ELITES, torch.empty((R, K), dtype=torch.int32, device="cuda")),
        "mu": model.trace(_lib.TRACE_MU, torch.empty((R + 1, H, A), dtype=torch.float32, device="cuda")),
        "sigma": model.trace(_lib.TRACE_SIGMA, torch.empty((R + 1, H, A), dtype=torch.float32, device="cuda")),
    }
    torch.cuda.synchronize()
    out = {"action": to_np(action), "mu_out": to_np(mu), "sigma_out": to_np(sigma),
           "best": int(best.item())}
    out.update({k2: to_np(v) for k2, v in tr.items()})   # "mu"/"sigma" are the per-round history
    out.update(N=N, K=K, R=R, H=H)
    return out


def max_rel(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), 1e-30)))

"""cem_plan_noalloc: the plan step without allocation, for callers that cannot
allocate (graph capture, serving loops).  Its plan state lives in the library's
per-device scratch array; its results must equal cem_plan's bit for bit, call
after call, including a smaller plan right after a larger one (the scratch keeps
the previous call's contents)."""
import numpy as np
import pytest

from .gpu_util import gpu_model, log, release_models, to_dev, to_np, workload_data

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _free_models():
    yield
    release_models()


def _plan(name, *, noalloc, n, k, rounds, horizon, plan_id=0, seed=None):
    import torch

    wl, _, _, z_obs, z_goal, s0 = workload_data(name)
    pc, A = wl.plan, wl.model.action_dim
    model = gpu_model(name)
    mu = torch.full((horizon, A), pc.mu0, dtype=torch.float32, device="cuda")
    sigma = torch.full((horizon, A), pc.sigma0, dtype=torch.float32, device="cuda")
    action = torch.empty(A, dtype=torch.float32, device="cuda")
    best = torch.empty(1, dtype=torch.int32, device="cuda")
    model.plan(to_dev(z_obs), to_dev(z_goal), to_dev(s0), mu, sigma, action, best, n_samples=n,
               n_elites=k, rounds=rounds, horizon=horizon, seed=pc.seed if seed is None else seed,
               plan_id=plan_id, clamp_lo=pc.clamp_lo, clamp_hi=pc.clamp_hi, noalloc=noalloc)
    torch.cuda.synchronize()
    return {"action": to_np(action), "mu": to_np(mu), "sigma": to_np(sigma), "best": int(best.item())}


@pytest.mark.parametrize("name,shapes", [
    ("small", [(256, 32, 3, 3), (64, 8, 2, 2)]),   # bf16, horizon 3 then a smaller plan
    ("tiny", [(64, 8, 3, 2), (17, 5, 1, 1)]),      # fp32
    ("vjepa2ac", [(800, 80, 2, 1), (200, 20, 1, 1)]),   # the measured shape, then a smaller plan
])
def test_noalloc_plan_equals_cem_plan(gpu_lib, name, shapes):
    for i, (n, k, r, h) in enumerate(shapes):
        log(f"{name}: call {i}: N={n} K={k} R={r} H={h}, cem_plan_noalloc vs cem_plan")
        got = _plan(name, noalloc=True, n=n, k=k, rounds=r, horizon=h, plan_id=3 + i)
        want = _plan(name, noalloc=False, n=n, k=k, rounds=r, horizon=h, plan_id=3 + i)
        for key in ("action", "mu", "sigma"):
            np.testing.assert_array_equal(got[key], want[key], err_msg=f"call {i}: {key}")
        assert got["best"] == want["best"]


def test_noalloc_plan_leaves_the_trace_of_cem_plan(gpu_lib):
    import torch

    from cem_jepa_predictor_amd import _lib

    name = "tiny"
    R, N, H, A = 2, 64, 2, 7
    _plan(name, noalloc=False, n=N, k=8, rounds=R, horizon=H, plan_id=1)
    model = gpu_model(name)
    before = to_np(model.trace(_lib.TRACE_ENERGY, torch.empty((R, N), device="cuda")))
    _plan(name, noalloc=True, n=32, k=4, rounds=3, horizon=1, plan_id=9)
    after = to_np(model.trace(_lib.TRACE_ENERGY, torch.empty((R, N), device="cuda")))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(before, after)


def test_noalloc_plan_rejects_what_the_scratch_cannot_hold(gpu_lib):
    """Host-side checks: a plan state beyond the 8 MiB scratch, or kernel timers on,
    is refused before anything is enqueued."""
    from cem_jepa_predictor_amd import _lib

    name = "tiny"
    # R N H A 4 = 4096 * 64 * 2 * 7 * 4 bytes of samples alone: 14.7 MB
    with pytest.raises(_lib.CemError) as e:
        _plan(name, noalloc=True, n=64, k=8, rounds=4096, horizon=2)
    assert e.value.status == -2 and "scratch" in str(e.value)
    model = gpu_model(name)
    model.timer_enable(True)
    try:
        with pytest.raises(_lib.CemError) as e:
            _plan(name, noalloc=True, n=64, k=8, rounds=1, horizon=2)
        assert e.value.status == -1
    finally:
        model.timer_enable(False)
    # still usable afterwards
    got = _plan(name, noalloc=True, n=64, k=8, rounds=1, horizon=2)
    want = _plan(name, noalloc=False, n=64, k=8, rounds=1, horizon=2)
    np.testing.assert_array_equal(got["action"], want["action"])

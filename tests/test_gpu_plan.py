"""GPU parity of the predictor rollout and of the full CEM plan step against the oracle.

Modes (tolerances from the method's stated bar):
  * rollout / energy parity: on the same candidate actions, GPU energies vs the
    oracle's float64 energies, max relative error <= 1e-5 for the fp32 model and
    <= 2e-2 for bf16 models;
  * lockstep plan: the oracle runs its own sampler and refit but takes each
    round's elites from the GPU's energies; elite lists must be bit-exact every
    round and the final action within 1e-2 absolute;
  * determinism: graph replay, direct enqueue and repeated runs are bitwise
    identical, and so is any split of the candidates into launches.
"""
import numpy as np
import pytest

from oracle import energy as o_energy
from oracle import refit as o_refit
from oracle import sampler as o_sampler
from oracle import select as o_select

from .gpu_util import (gpu_model, log, max_rel, oracle_predictor, release_models, run_plan, to_dev,
                       to_np, workload_data)

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 2e-2}


@pytest.fixture(scope="module", autouse=True)
def _free_models():
    yield
    release_models()


def gpu_rollout(name, actions):
    import torch

    wl, _, _, z_obs, _, s0 = workload_data(name)
    m = wl.model
    model = gpu_model(name)
    dt = torch.float32 if m.dtype == "f32" else torch.bfloat16
    zp = torch.empty((actions.shape[0], m.patches, m.enc_dim), dtype=dt, device="cuda")
    model.rollout(to_dev(actions), to_dev(z_obs), to_dev(s0), zp)
    torch.cuda.synchronize()
    return to_np(zp)


# small with n = 3 and 5 (M = 198, 330 rows): the last rows of each GEMM fill an 8-row piece only
# partly (6 and 2 rows), in the residual kind's buffer-bounded epilogue as well.  wide768 and
# wide2048: the LayerNorm statistics of d = 768 and 2048 rows in 12 and 32 pieces (small: 8, the
# V-JEPA2-AC shape: 16, oddk: a statistics pass of its own).  Horizon 1 on the bf16 and fp8
# models (small, oddk, small_fp8, wide2048): layer 0 projects each problem's shared rows once
# and the candidates' action rows once, in one compact block the attention reads from.  p256
# (17 query tiles) and p140 (9): one wave of the attention workgroup takes a third (second)
# query tile, the last, with 2 (14) rows.  p318: the longest block (B = 320, 20 tiles).
# wide4096: the widest model (d = 4096, 64 statistics pieces per row).
@pytest.mark.parametrize("name,n,horizon", [("tiny", 64, None), ("tiny", 5, None), ("small", 12, None),
                                            ("small", 3, None), ("small", 5, None), ("small", 12, 1),
                                            ("small", 3, 1), ("small", 1, 1), ("oddk", 9, None), ("oddk", 9, 1),
                                            ("small_fp8", 12, None), ("small_fp8", 12, 1),
                                            ("wide768", 12, None),
                                            ("wide2048", 9, None), ("p256", 16, None), ("p256", 300, None),
                                            ("p256", 5, None), ("p140", 16, None), ("p140", 40, 1),
                                            ("p318", 16, None), ("p318", 24, 1), ("wide4096", 5, None)])
def test_rollout_matches_oracle(gpu_lib, name, n, horizon):
    from cem_jepa_predictor_amd import inputs

    wl, _, _, z_obs, z_goal, s0 = workload_data(name)
    H = horizon or wl.plan.horizon
    log(f"rollout {name} n={n} H={H}")
    actions = inputs.make_actions(n, H, seed=n)
    got = gpu_rollout(name, actions)
    pred = oracle_predictor(name)
    want = pred.rollout_cached(actions, z_obs, s0)
    e_got = o_energy.energy_l1(got, z_goal)
    e_want = o_energy.energy_l1(want, z_goal)
    rel = max_rel(e_got, e_want)
    scale = np.abs(want).max()
    log(f"  energy max rel err {rel:.3e}; z max abs err {np.abs(got - want).max():.3e} (scale {scale:.2f})")
    assert rel <= TOL[wl.model.dtype]
    # element-wise bound on the predicted frame: fp8 models flip an e4m3 rounding of the
    # LayerNorm outputs wherever GPU (bf16 residual stream) and oracle (float64) land on
    # either side of a step, which moves single elements by up to ~7 % of the frame's
    # largest magnitude after six layers; energies average it out
    ztol = {"f32": 1e-4, "bf16": 5e-2, "fp8": 1.5e-1}[wl.model.dtype]
    assert np.abs(got - want).max() <= ztol * scale
    if n >= 8:
        # energy parity as a ranking: Pearson r of GPU vs oracle energies across the
        # candidates, next to the ratio of the candidates' energy spread to the error.
        # Gated at the page's 0.9999 for the fp32 model; for bf16 models under
        # random-init weights the spread sits near bf16 resolution (logged only).
        r = float(np.corrcoef(e_got, e_want)[0, 1])
        err = float(np.sqrt(np.mean((e_got - e_want) ** 2)))
        spread = float(np.std(e_want))
        log(f"  Pearson r {r:.6f}; energy spread {spread:.3e} vs rms error {err:.3e} (ratio {spread / max(err, 1e-30):.1f})")
        if wl.model.dtype == "f32":
            assert r >= 0.9999


def _lockstep(name, out, oracle_rows, mu_init=None, sigma_init=None, plan_id=None, problem=None,
              round0=0):
    """Follow the GPU plan round by round with the oracle.  problem = (z_obs, z_goal,
    s0) replaces the workload's own inputs; round0 is the plan's first Philox round."""
    wl, _, _, z_obs, z_goal, s0 = workload_data(name)
    if problem is not None:
        z_obs, z_goal, s0 = problem
    pc = wl.plan
    N, K, R, H = out["N"], out["K"], out["R"], out["H"]
    pred = oracle_predictor(name)
    mu = np.full((H, 7), pc.mu0, np.float32) if mu_init is None else np.asarray(mu_init, np.float32)
    sigma = np.full((H, 7), pc.sigma0, np.float32) if sigma_init is None else np.asarray(sigma_init, np.float32)
    np.testing.assert_array_equal(out["mu"][0], mu)
    np.testing.assert_array_equal(out["sigma"][0], sigma)
    pid = pc.plan_id if plan_id is None else plan_id
    worst = 0.0
    for r in range(R):
        x = o_sampler.sample_actions(mu, sigma, pc.seed, round0 + r, pid, N, pc.clamp_lo, pc.clamp_hi)
        # samples: identical up to a float32 ulp where float64 libms differ
        ulps = np.abs(out["x"][r].view(np.int32).astype(np.int64) - x.view(np.int32).astype(np.int64))
        assert ulps.max() <= 1, f"round {r}: samples differ by {ulps.max()} ulp"
        rows = oracle_rows(r, N)
        if len(rows):
            e_or = o_energy.energy_l1(pred.rollout_cached(out["x"][r][rows], z_obs, s0), z_goal)
            rel = max_rel(out["energy"][r][rows], e_or)
            worst = max(worst, rel)
            assert rel <= TOL[wl.model.dtype], f"round {r}: energy rel err {rel:.3e}"
        elites = o_select.topk_elites(out["energy"][r], K)
        np.testing.assert_array_equal(out["elites"][r], elites, err_msg=f"round {r}")
        mu, sigma = o_refit.refit(x, elites)
        np.testing.assert_allclose(out["mu"][r + 1], mu, rtol=0, atol=1e-6)
        np.testing.assert_allclose(out["sigma"][r + 1], sigma, rtol=0, atol=1e-6)
    assert np.abs(out["action"] - mu[0]).max() <= 1e-2
    np.testing.assert_array_equal(out["action"], out["mu"][R][0])
    np.testing.assert_array_equal(out["mu_out"], out["mu"][R])
    np.testing.assert_array_equal(out["sigma_out"], out["sigma"][R])
    assert out["best"] == out["elites"][R - 1][0]
    return worst


def test_plan_tiny_lockstep_all_candidates(gpu_lib):
    log("plan tiny lockstep, oracle energies for every candidate")
    out = run_plan("tiny")
    worst = _lockstep("tiny", out, lambda r, n: np.arange(n))
    log(f"  worst energy rel err {worst:.3e}")


def test_plan_tiny_independent(gpu_lib):
    """fp32: the oracle's own end-to-end plan picks the same elites."""
    from oracle import cem

    wl, _, _, z_obs, z_goal, s0 = workload_data("tiny")
    pc = wl.plan
    log("plan tiny independent")
    out = run_plan("tiny")
    pred = oracle_predictor("tiny")
    ref = cem.cem_plan(cem.predictor_energy_fn(pred, z_obs, z_goal, s0), pc.n_samples, pc.n_elites,
                       pc.rounds, np.full((pc.horizon, 7), pc.mu0), np.full((pc.horizon, 7), pc.sigma0),
                       pc.seed, pc.plan_id, pc.clamp_lo, pc.clamp_hi)
    for r in range(pc.rounds):
        gaps = np.diff(np.sort(ref["trace"]["energy"][r]))
        log(f"  round {r}: min energy gap {gaps.min():.3e}")
        np.testing.assert_array_equal(out["elites"][r], ref["trace"]["elites"][r])
    assert np.abs(out["action"] - ref["action"]).max() <= 1e-2


def test_plan_small_lockstep_sampled(gpu_lib):
    log("plan small lockstep, 6 oracle candidates per round")
    out = run_plan("small")
    worst = _lockstep("small", out, lambda r, n: np.random.default_rng(r).choice(n, 6, replace=False))
    log(f"  worst energy rel err {worst:.3e}")


def test_plan_vjepa2ac_full_size_lockstep(gpu_lib):
    """The measured configuration: 800 candidates x 10 rounds, V-JEPA2-AC-shaped predictor."""
    log("plan vjepa2ac full size (N=800, K=80, R=10, H=1) lockstep, oracle on 2 rounds x 2 candidates")
    out = run_plan("vjepa2ac")
    e = out["energy"]
    spread = float(np.median(e.std(axis=1)))
    log(f"  energy median {np.median(e):.5f}, per-round std median {spread:.3e}")
    rows = {0: [0, 517], 9: [3, 799]}
    worst = _lockstep("vjepa2ac", out, lambda r, n: np.array(rows.get(r, []), dtype=int))
    log(f"  worst energy rel err {worst:.3e}")


def test_plan_h4_kv_cache_lockstep(gpu_lib):
    """Horizon 4 with the KV cache across frame blocks at full candidate count (2 rounds)."""
    log("plan vjepa2ac_h4 (N=800, H=4) 2 rounds lockstep, oracle on 1 candidate per round")
    out = run_plan("vjepa2ac_h4", rounds=2)
    worst = _lockstep("vjepa2ac_h4", out, lambda r, n: np.array([7 + 400 * r]))
    log(f"  worst energy rel err {worst:.3e}")


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_plan_graph_equals_eager_and_is_deterministic(gpu_lib, name):
    log(f"determinism {name}")
    a = run_plan(name, use_graph=True)
    b = run_plan(name, use_graph=False)
    c = run_plan(name, use_graph=True)
    for key in ["x", "energy", "elites", "mu", "sigma", "action"]:
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
        np.testing.assert_array_equal(a[key], c[key], err_msg=key)
    # a different plan id draws different candidates
    d = run_plan(name, plan_id=5)
    assert not np.array_equal(a["x"], d["x"])


@pytest.mark.parametrize("name,horizon,n,chunk", [("small", None, 64, 16), ("small", 1, 64, 16),
                                                   ("p256", None, 300, 100), ("p140", None, 64, 24)])
def test_rollout_is_invariant_to_candidate_chunking(gpu_lib, name, horizon, n, chunk):
    """Same seeds give the same answer however candidates are grouped (cf. plans identical
    at 1, 2, 4 and 8 GPUs).  At horizon 1 the groups also change the compact layer-0 block
    (shared rows once, then each group's action rows); p256 runs the V-JEPA2-AC block
    length (B = 258) with 600 and 200 (candidate, head) attention items per launch."""
    import torch
    from cem_jepa_predictor_amd import _lib

    wl, _, _, z_obs, z_goal, s0 = workload_data(name)
    from cem_jepa_predictor_amd import inputs

    actions = inputs.make_actions(n, horizon or wl.plan.horizon, seed=11)
    full = gpu_rollout(name, actions)
    parts = np.concatenate([gpu_rollout(name, actions[i:i + chunk]) for i in range(0, n, chunk)])
    np.testing.assert_array_equal(full, parts)
    e = torch.empty(n, dtype=torch.float32, device="cuda")
    _lib.energy_l1(to_dev(full).to(torch.bfloat16), to_dev(z_goal), e)
    torch.cuda.synchronize()


def test_plan_energies_equal_rollout_then_energy(gpu_lib):
    """The plan's fused round equals the stand-alone rollout + energy calls on its samples."""
    import torch
    from cem_jepa_predictor_amd import _lib

    name = "small"
    wl, _, _, z_obs, z_goal, s0 = workload_data(name)
    out = run_plan(name, rounds=2)
    z = gpu_rollout(name, out["x"][1])
    tz = to_dev(z).to(torch.bfloat16)
    e = torch.empty(out["N"], dtype=torch.float32, device="cuda")
    _lib.energy_l1(tz, to_dev(z_goal), e)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(e), out["energy"][1])


@pytest.mark.parametrize("n,k,r", [(1, 1, 1), (17, 17, 2), (33, 5, 1)])
def test_plan_edge_shapes(gpu_lib, n, k, r):
    log(f"plan tiny edge N={n} K={k} R={r}")
    out = run_plan("tiny", n=n, k=k, rounds=r)
    _lockstep("tiny", out, lambda rr, nn: np.arange(nn))


def test_plan_shorter_horizon_than_max(gpu_lib):
    log("plan small with H=1 on a max-horizon-3 model")
    out = run_plan("small", horizon=1, rounds=2)
    _lockstep("small", out, lambda r, n: np.arange(4))


@pytest.mark.parametrize("floor", [0.0, 1.0])
def test_warm_started_closed_loop_lockstep(gpu_lib, floor):
    """Receding-horizon control (page section 06 B): each control step's plan
    starts from cem_warm_start of the previous plan (shifted one step, fresh last
    step), run in place on the device; the warm start is bit-exact against the
    oracle and every plan follows the oracle round by round."""
    import torch
    from cem_jepa_predictor_amd import _lib
    from oracle import cem

    wl = workload_data("tiny")[0]
    pc = wl.plan
    H, A = pc.horizon, wl.model.action_dim
    mu = np.full((H, A), pc.mu0, np.float32)
    sigma = np.full((H, A), pc.sigma0, np.float32)
    log(f"warm-started closed loop, tiny, 3 control steps x 2 rounds, sigma floor {floor}")
    for step in range(3):
        out = run_plan("tiny", rounds=2, plan_id=step, mu_init=mu, sigma_init=sigma)
        _lockstep("tiny", out, lambda r, n: np.arange(n), mu_init=mu, sigma_init=sigma, plan_id=step)
        mt, st = to_dev(out["mu_out"]), to_dev(out["sigma_out"])
        _lib.warm_start(mt, st, pc.mu0, pc.sigma0, floor, mt, st)
        torch.cuda.synchronize()
        mu, sigma = cem.warm_start(out["mu_out"], out["sigma_out"], pc.mu0, pc.sigma0, floor)
        np.testing.assert_array_equal(to_np(mt), mu)
        np.testing.assert_array_equal(to_np(st), sigma)
        np.testing.assert_array_equal(mu[0], out["mu_out"][1])


@pytest.mark.parametrize("name,use_graph", [("tiny", True), ("small", False), ("small", True)])
def test_plan_resume_equals_uninterrupted(gpu_lib, name, use_graph):
    """A plan stopped after r0 rounds and resumed from the Gaussian it returned, with
    first_round = r0, is the uninterrupted plan bit for bit, trace included; the
    resumed rounds also follow the oracle from that Gaussian at Philox rounds r0, ..."""
    R, r0 = 4, 2
    log(f"resume {name}: {r0} + {R - r0} rounds against {R}, graph={use_graph}")
    full = run_plan(name, rounds=R, use_graph=use_graph)
    first = run_plan(name, rounds=r0, use_graph=use_graph)
    rest = run_plan(name, rounds=R - r0, use_graph=use_graph, mu_init=first["mu_out"],
                    sigma_init=first["sigma_out"], first_round=r0)
    for key in ("x", "energy", "elites"):
        np.testing.assert_array_equal(first[key], full[key][:r0], err_msg=key)
        np.testing.assert_array_equal(rest[key], full[key][r0:], err_msg=key)
    for key in ("mu", "sigma"):
        np.testing.assert_array_equal(first[key], full[key][:r0 + 1], err_msg=key)
        np.testing.assert_array_equal(rest[key], full[key][r0:], err_msg=key)
    for key in ("action", "mu_out", "sigma_out"):
        np.testing.assert_array_equal(rest[key], full[key], err_msg=key)
    assert rest["best"] == full["best"]
    rows = (lambda r, n: np.arange(n)) if name == "tiny" else (
        lambda r, n: np.random.default_rng(50 + r).choice(n, 6, replace=False))
    worst = _lockstep(name, rest, rows, mu_init=first["mu_out"], sigma_init=first["sigma_out"], round0=r0)
    log(f"  resumed rounds in lockstep with the oracle, worst energy rel err {worst:.3e}")


def _problems(name, batch, horizon=None):
    """Per-problem inputs: problem 0 is the workload's own, the others differ in
    observation, goal, state and starting Gaussian."""
    wl, _, _, z_obs, z_goal, s0 = workload_data(name)
    pc, m = wl.plan, wl.model
    H, A = horizon or pc.horizon, m.action_dim
    rng = np.random.default_rng(17)
    zo = [z_obs] + [rng.standard_normal(z_obs.shape).astype(np.float32) for _ in range(batch - 1)]
    zg = [z_goal] + [rng.standard_normal(z_goal.shape).astype(np.float32) for _ in range(batch - 1)]
    st = [s0] + [rng.uniform(-0.5, 0.5, s0.shape).astype(np.float32) for _ in range(batch - 1)]
    mu = [np.full((H, A), pc.mu0, np.float32)] + [rng.uniform(-0.3, 0.3, (H, A)).astype(np.float32)
                                                  for _ in range(batch - 1)]
    sg = [np.full((H, A), pc.sigma0, np.float32)] + [rng.uniform(0.2, 1.0, (H, A)).astype(np.float32)
                                                     for _ in range(batch - 1)]
    return [np.stack(v) for v in (zo, zg, st, mu, sg)]


# sweep_400 x 2: two V-JEPA2-AC-shaped problems of 400 candidates in one 800-candidate batch
# (M = 206,400 rows), as the benchmark's fleet-batching rows run it.  small at horizon 1: three
# problems' shared layer-0 rows in one compact block
@pytest.mark.parametrize("name,batch,use_graph,horizon", [("tiny", 3, True, None), ("small", 2, True, None),
                                                          ("tiny", 2, False, None), ("small", 3, True, 1),
                                                          ("sweep_400", 2, True, None)])
def test_plan_batched_equals_independent_plans(gpu_lib, name, batch, use_graph, horizon):
    """Fleet batching (page section 06 C): a batched plan of several problems in one
    predictor batch gives each problem exactly its own cem_plan result (plan id
    + b), trace included."""
    import torch
    from cem_jepa_predictor_amd import _lib

    wl = workload_data(name)[0]
    pc, m = wl.plan, wl.model
    N, K, R, A = pc.n_samples, pc.n_elites, min(pc.rounds, 3), m.action_dim
    H = horizon or pc.horizon
    log(f"batched plan {name}: {batch} problems x N={N}, R={R}, H={H}, graph={use_graph}")
    zo, zg, st, mu, sg = _problems(name, batch, H)
    model = gpu_model(name, batch * N)
    kw = dict(n_samples=N, n_elites=K, rounds=R, horizon=H, seed=pc.seed, clamp_lo=pc.clamp_lo,
              clamp_hi=pc.clamp_hi, use_graph=use_graph)

    def traces(nb):
        f32, i32 = torch.float32, torch.int32
        return {
            "x": to_np(model.trace(_lib.TRACE_ACTIONS, torch.empty((R, nb * N, H, A), dtype=f32, device="cuda"))),
            "e": to_np(model.trace(_lib.TRACE_ENERGY, torch.empty((R, nb * N), dtype=f32, device="cuda"))),
            "el": to_np(model.trace(_lib.TRACE_ELITES, torch.empty((R, nb, K), dtype=i32, device="cuda"))),
            "mu": to_np(model.trace(_lib.TRACE_MU, torch.empty((R + 1, nb, H, A), dtype=f32, device="cuda"))),
            "sg": to_np(model.trace(_lib.TRACE_SIGMA, torch.empty((R + 1, nb, H, A), dtype=f32, device="cuda"))),
        }

    mu_t, sg_t = to_dev(mu), to_dev(sg)
    act = torch.empty((batch, A), dtype=torch.float32, device="cuda")
    best = torch.empty(batch, dtype=torch.int32, device="cuda")
    model.plan_batched(to_dev(zo), to_dev(zg), to_dev(st), mu_t, sg_t, act, best, plan_id=4, **kw)
    torch.cuda.synchronize()
    tb = traces(batch)
    got = {"act": to_np(act), "mu": to_np(mu_t), "sg": to_np(sg_t), "best": to_np(best)}
    for b in range(batch):
        mb, sb = to_dev(mu[b]), to_dev(sg[b])
        ab = torch.empty(A, dtype=torch.float32, device="cuda")
        bb = torch.empty(1, dtype=torch.int32, device="cuda")
        model.plan(to_dev(zo[b]), to_dev(zg[b]), to_dev(st[b]), mb, sb, ab, bb, plan_id=4 + b, **kw)
        torch.cuda.synchronize()
        t1 = traces(1)
        np.testing.assert_array_equal(got["act"][b], to_np(ab), err_msg=f"problem {b} action")
        np.testing.assert_array_equal(got["mu"][b], to_np(mb))
        np.testing.assert_array_equal(got["sg"][b], to_np(sb))
        assert got["best"][b] == int(bb.item())
        np.testing.assert_array_equal(tb["x"][:, b * N:(b + 1) * N], t1["x"])
        np.testing.assert_array_equal(tb["e"][:, b * N:(b + 1) * N], t1["e"])
        np.testing.assert_array_equal(tb["el"][:, b], t1["el"][:, 0])
        np.testing.assert_array_equal(tb["mu"][:, b], t1["mu"][:, 0])
        np.testing.assert_array_equal(tb["sg"][:, b], t1["sg"][:, 0])
    # the problems really differ
    assert not np.array_equal(tb["e"][:, :N], tb["e"][:, N:2 * N])
    # and every problem's slice follows the oracle round by round on its own inputs,
    # Gaussian and plan id (all candidates for tiny, 6 per round for small, 2 per round at
    # the V-JEPA2-AC shape)
    for b in range(batch):
        out_b = {"x": tb["x"][:, b * N:(b + 1) * N], "energy": tb["e"][:, b * N:(b + 1) * N],
                 "elites": tb["el"][:, b], "mu": tb["mu"][:, b], "sigma": tb["sg"][:, b],
                 "action": got["act"][b], "mu_out": got["mu"][b], "sigma_out": got["sg"][b],
                 "best": int(got["best"][b]), "N": N, "K": K, "R": R, "H": H}
        if name == "tiny":
            rows = lambda r, n: np.arange(n)  # noqa: E731
        else:
            per_round = 6 if name == "small" else 2
            rows = lambda r, n, b=b, k=per_round: np.random.default_rng(10 * b + r).choice(n, k, replace=False)  # noqa: E731
        worst = _lockstep(name, out_b, rows, mu_init=mu[b], sigma_init=sg[b], plan_id=4 + b,
                          problem=(zo[b], zg[b], st[b]))
        log(f"  problem {b}: lockstep with the oracle, worst energy rel err {worst:.3e}")


def test_plan_small_fp8_lockstep_sampled(gpu_lib):
    """fp8 q|k|v and MLP-up projections (model dtype CEM_FP8) against the oracle's
    fp8-projection predictor, round by round."""
    log("plan small_fp8 lockstep, 6 oracle candidates per round")
    out = run_plan("small_fp8")
    worst = _lockstep("small_fp8", out, lambda r, n: np.random.default_rng(r).choice(n, 6, replace=False))
    log(f"  worst energy rel err {worst:.3e}")


def test_plan_vjepa2ac_fp8_full_size_lockstep(gpu_lib):
    """The V-JEPA2-AC shape with fp8 projections, 800 candidates x 2 rounds."""
    log("plan vjepa2ac_fp8 (N=800, R=2) lockstep, oracle on 2 candidates")
    out = run_plan("vjepa2ac_fp8", rounds=2)
    worst = _lockstep("vjepa2ac_fp8", out, lambda r, n: np.array([5 + 300 * r, 777 - r]))
    log(f"  worst energy rel err {worst:.3e}")


def gpu_rollout_rows(name, actions, rows):
    """GPU rollout of all candidates; the predicted frames of `rows` as float64."""
    import torch

    wl, _, _, z_obs, _, s0 = workload_data(name)
    m = wl.model
    model = gpu_model(name)
    dt = torch.float32 if m.dtype == "f32" else torch.bfloat16
    zp = torch.empty((actions.shape[0], m.patches, m.enc_dim), dtype=dt, device="cuda")
    model.rollout(to_dev(actions), to_dev(z_obs), to_dev(s0), zp)
    sel = zp[torch.as_tensor(rows, device="cuda")].float().cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    return sel, zp


@pytest.mark.parametrize("name,n,rows", [("vjepa2ac", 800, [0, 413, 799]), ("vjepa2ac_h4", 800, [1, 799])])
def test_rollout_full_size_elementwise(gpu_lib, name, n, rows):
    """The measured shape, element by element: all 800 candidates in one rollout (the
    plan step's GEMM tile schedule, persistent multi-tile workgroups, 17 query tiles per
    attention workgroup with a ragged last one; at horizon 4 the several-block attention
    over the KV cache and the fed-back frames' in-projection), sampled candidates
    compared with the oracle's cached rollout."""
    from cem_jepa_predictor_amd import inputs

    wl, _, _, z_obs, z_goal, s0 = workload_data(name)
    H = wl.plan.horizon
    actions = inputs.make_actions(n, H, seed=21)
    log(f"rollout {name} n={n} H={H}, oracle on candidates {rows}")
    got, _ = gpu_rollout_rows(name, actions, rows)
    want = oracle_predictor(name).rollout_cached(actions[rows], z_obs, s0)
    scale = np.abs(want).max()
    err = np.abs(got - want)
    rel = max_rel(o_energy.energy_l1(got, z_goal), o_energy.energy_l1(want, z_goal))
    log(f"  z max abs err {err.max():.3e} (scale {scale:.2f}, {err.max() / scale:.2e} of it); "
        f"rms err {np.sqrt(np.mean(err ** 2)):.3e}; energy max rel err {rel:.3e}")
    for i, r in enumerate(rows):
        log(f"  candidate {r}: max abs err {err[i].max():.3e}")
    assert err.max() <= 5e-2 * scale
    assert rel <= TOL["bf16"]


@pytest.mark.parametrize("name", ["small", "small_fp8"])
def test_rollout_many_tiles_equals_oracle_checked_chunks(gpu_lib, name):
    """256 candidates in one rollout give more GEMM tiles than compute units, so every
    workgroup of the persistent GEMM runs several tiles (operand ring carried across
    tiles, prefetched tile constants, staging-entry reuse); the result must equal,
    bit for bit, rollouts of chunks of 12 candidates (the size compared element by
    element with the oracle elsewhere), and sampled rows must match the oracle."""
    from cem_jepa_predictor_amd import inputs

    wl, _, _, z_obs, z_goal, s0 = workload_data(name)
    m, H, n = wl.model, wl.plan.horizon, 256
    tiles = -(-n * m.block_tokens // 256) * -(-3 * m.d_model // 256)
    log(f"rollout {name} n={n}: {tiles} q|k|v tiles")
    actions = inputs.make_actions(n, H, seed=31)
    full = gpu_rollout(name, actions)
    parts = np.concatenate([gpu_rollout(name, actions[i:i + 12]) for i in range(0, n, 12)])
    np.testing.assert_array_equal(full, parts)
    rows = [0, 131, 255]
    want = oracle_predictor(name).rollout_cached(actions[rows], z_obs, s0)
    err = np.abs(full[rows] - want).max()
    log(f"  bitwise equal to 12-candidate chunks; rows {rows}: max abs err {err:.3e} (scale {np.abs(want).max():.2f})")
    ztol = {"bf16": 5e-2, "fp8": 1.5e-1}[m.dtype]
    assert err <= ztol * np.abs(want).max()


@pytest.mark.parametrize("n", [200, 1600, 3200])
def test_plan_sweep_lockstep(gpu_lib, n):
    """Batch-sweep points (N candidates, K = N / 10) for one round: sampler, rollout,
    energy, selection and refit at M = 258 N rows (825,600 at N = 3200), the oracle on
    the first and last candidates."""
    name = f"sweep_{n}"
    log(f"plan {name} 1 round lockstep, oracle on candidates 0 and {n - 1}")
    out = run_plan(name, rounds=1)
    worst = _lockstep(name, out, lambda r, nn: np.array([0, nn - 1]))
    log(f"  worst energy rel err {worst:.3e}")
    release_models()


@pytest.mark.parametrize("name", ["shallow_fp8", "small_fp8"])
def test_fp8_rollout_is_the_fp8_method(gpu_lib, name):
    """fp8 projections (page section 06, "D. Model compression") must be visible: the
    GPU rollout's rms distance from the oracle's fp8-projection mode, in units of the
    fp8 effect (fp8 mode minus plain mode), stays below the gate on the one-layer
    workload (a path without quantization sits near 1; so do the wrong matrices or
    scales, see the CPU test of the gate).  On the six-layer workload the flips of
    e4m3 rounding decisions compound, so it is held to a wider bound."""
    from cem_jepa_predictor_amd import inputs
    from oracle.predictor import Predictor

    from .bf16_storage import FP8_GATE, fp8_distance

    wl, w, _, z_obs, _, s0 = workload_data(name)
    m = wl.model
    actions = inputs.make_actions(16, wl.plan.horizon, seed=41)
    got = gpu_rollout(name, actions).astype(np.float64)
    z8 = oracle_predictor(name).rollout_cached(actions, z_obs, s0)
    z = Predictor(w, m.layers, m.heads, m.ln_eps).rollout_cached(actions, z_obs, s0)
    d8, d0 = fp8_distance(got, z8, z), fp8_distance(got, z, z8)
    log(f"  {name}: distance to the fp8 mode {d8:.3f}, to the plain mode {d0:.3f} (units of the fp8 effect)")
    assert d8 <= (FP8_GATE if m.layers == 1 else 0.9)
    assert d0 >= 0.8


@pytest.mark.parametrize("name,n,draws", [("small", 64, 4), ("vjepa2ac", 16, 1)])
def test_energy_ranking_with_reachable_goal(gpu_lib, name, n, draws):
    """Energy parity as a ranking (page section 05: the bf16 planner's energies track the
    fp32 reference, Pearson r 0.9999).  With the workload's random goal the candidates'
    energies differ by little more than bf16 storage of the residual stream moves them
    (any bf16 implementation; logged).  With a reachable goal -- the oracle's predicted
    frame for a known action sequence -- candidates differ by how far their actions are
    from it, and the GPU's energies must rank them as the oracle does.  On small, r is
    pooled over `draws` action draws of n candidates: the r of one 64-candidate draw moves
    by about 3e-4 with the bf16 rounding pattern alone."""
    from cem_jepa_predictor_amd import inputs

    wl, _, _, z_obs, z_goal, s0 = workload_data(name)
    H = wl.plan.horizon
    pred = oracle_predictor(name)
    a_star = inputs.make_actions(1, H, seed=99) * np.float32(0.6)
    goal = pred.rollout_cached(a_star, z_obs, s0)[0].astype(np.float32)
    got, want = [], []
    for k in range(draws):
        actions = inputs.make_actions(n, H, seed=51 + k)
        got.append(gpu_rollout(name, actions))
        want.append(pred.rollout_cached(actions, z_obs, s0))
    got, want = np.concatenate(got), np.concatenate(want)
    stats = {}
    for label, g in (("random goal", z_goal), ("reachable goal", goal)):
        e_got, e_want = o_energy.energy_l1(got, g), o_energy.energy_l1(want, g)
        r = float(np.corrcoef(e_got, e_want)[0, 1])
        d = e_got - e_want
        spread, err = float(np.std(e_want)), float(np.std(d))
        stats[label] = r
        log(f"  {name} {label} ({draws} x {n} candidates): mean energy {e_want.mean():.4e}, Pearson r {r:.6f}, "
            f"spread {spread:.3e}, candidate-specific rms err {err:.3e} (ratio {spread / max(err, 1e-30):.1f}), "
            f"common offset {d.mean():.3e}")
    # bf16 storage of the residual stream alone, emulated on the oracle, gives r of
    # 0.9993 on small; at 24 layers it is a larger share of the smaller effect of an
    # action on the predicted frame
    assert stats["reachable goal"] >= (0.999 if name == "small" else 0.99)


def test_plan_small_reachable_goal_independent(gpu_lib):
    """Independent plan, bf16 (page section 01: sample, predict, score, keep the best,
    refit; execute the first action of the final Gaussian).  The goal is reachable --
    the oracle's predicted frame for a known action sequence a* -- so the energies
    carry a real signal; the GPU plans on its own energies and its action must land
    near the oracle's own float64 plan, stored by tests/golden/make_small_reachable_plan.py.
    Bound: bf16 storage of the activations alone (emulated on the oracle) moves this
    plan's action by 0.058 and keeps 28-31 of the 32 elites per round, so the action is
    held to 0.15 and round 0 (same samples on both sides) to 28 shared elites."""
    import json
    import os

    path = os.path.join(os.path.dirname(__file__), "golden", "small_reachable_plan.json")
    with open(path) as f:
        rec = json.load(f)
    from cem_jepa_predictor_amd import inputs

    wl, _, _, z_obs, _, s0 = workload_data("small")
    pred = oracle_predictor("small")
    a_star = inputs.make_actions(1, wl.plan.horizon, seed=rec["a_star_seed"]) * np.float32(rec["a_star_scale"])
    np.testing.assert_array_equal(a_star[0], np.asarray(rec["a_star"], np.float32))
    goal = pred.rollout_cached(a_star, z_obs, s0)[0].astype(np.float32)
    out = run_plan("small", z_goal=goal)
    want = np.asarray(rec["action"], np.float32)
    diff = float(np.abs(out["action"] - want).max())
    shared0 = len(set(out["elites"][0].tolist()) & set(rec["elites"][0]))
    log(f"  action {np.round(out['action'], 3).tolist()} vs oracle {np.round(want, 3).tolist()} "
        f"(a* first step {np.round(a_star[0, 0], 3).tolist()}): max diff {diff:.3f}; round-0 elites shared {shared0}/32")
    assert shared0 >= 28
    assert diff <= 0.15


@pytest.mark.parametrize("d_model,patches,heads,dtype,msg", [(128, 319, 2, "bf16", "patches + 2 <= 320"),
                                                             (128, 318, 4, "bf16", "head dim 64"),
                                                             (512, 319, 8, "fp8", "patches + 2 <= 320"),
                                                             (128, 318, 2, "fp8", "d_model % 512")])
def test_model_create_rejects_shapes_beyond_the_attention(gpu_lib, d_model, patches, heads, dtype, msg):
    """One past the longest frame block (B = 321), a head dim other than 64, or an fp8 width
    that is not a multiple of 512 is refused at creation with a shape error, not launched."""
    import dataclasses

    from cem_jepa_predictor_amd import _lib, inputs

    cfg = dataclasses.replace(inputs.WORKLOADS["p318"].model, name="reject", d_model=d_model,
                              patches=patches, heads=heads, dtype=dtype)
    flat = inputs.flatten_weights(cfg, inputs.make_weights(cfg, 0))
    with pytest.raises(_lib.CemError) as e:
        _lib.Model(cfg, flat, 8)
    log(f"  {cfg.patches} patches, {cfg.heads} heads, {dtype}: {e.value}")
    assert msg in str(e.value)

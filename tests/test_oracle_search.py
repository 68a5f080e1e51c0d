"""Pins of the oracle's energy, elite selection, refit and CEM loop (CPU)."""
import statistics

import numpy as np
import pytest

from oracle import cem, energy, refit, select


def test_energy_closed_forms():
    rng = np.random.default_rng(0)
    g = rng.standard_normal((4, 6)).astype(np.float32)
    z = np.stack([g, g + 0.5, g - 2.0]).astype(np.float32)
    e = energy.energy_l1(z, g)
    np.testing.assert_allclose(e, [0.0, 0.5, 2.0], rtol=0, atol=1e-6)


def test_energy_brute_force():
    rng = np.random.default_rng(1)
    z = rng.standard_normal((3, 5, 4))
    g = rng.standard_normal((5, 4))
    e = energy.energy_l1(z, g)
    for n in range(3):
        acc = 0.0
        for p in range(5):
            for j in range(4):
                acc += abs(float(z[n, p, j]) - float(g[p, j]))
        assert e[n] == pytest.approx(acc / 20.0, rel=1e-14)


def _brute_topk(e, k):
    key = [(float("inf") if np.isnan(v) else float(v), i) for i, v in enumerate(e)]
    return [i for _, i in sorted(key)[:k]]


def test_topk_brute_force_with_ties_and_nan():
    rng = np.random.default_rng(2)
    for trial in range(50):
        n = int(rng.integers(1, 300))
        k = int(rng.integers(1, n + 1))
        e = rng.choice([0.0, -0.0, 1.0, 2.5, np.inf, np.nan, -1.0], size=n) if trial % 2 else \
            rng.standard_normal(n).astype(np.float32)
        got = select.topk_elites(e, k)
        assert list(got) == _brute_topk(e, k)


def test_refit_closed_forms():
    # two elites a, b: mean (a+b)/2, population std |a-b|/2
    x = np.zeros((4, 1, 2), np.float32)
    x[1] = [[0.25, -1.0]]
    x[3] = [[0.75, 1.0]]
    mu, sigma = refit.refit(x, np.array([3, 1]))
    np.testing.assert_array_equal(mu, [[0.5, 0.0]])
    np.testing.assert_array_equal(sigma, [[0.25, 1.0]])
    # identical elites: zero spread
    mu, sigma = refit.refit(np.ones((5, 2, 3), np.float32), np.arange(5))
    np.testing.assert_array_equal(sigma, 0)


def test_refit_matches_statistics_module():
    rng = np.random.default_rng(3)
    x = rng.uniform(-1, 1, (40, 2, 7)).astype(np.float32)
    idx = rng.permutation(40)[:9]
    mu, sigma = refit.refit(x, idx)
    for h in range(2):
        for a in range(7):
            vals = [float(x[i, h, a]) for i in idx]
            assert mu[h, a] == np.float32(statistics.fmean(vals))
            assert abs(float(sigma[h, a]) - statistics.pstdev(vals)) <= 1e-7 * max(1.0, statistics.pstdev(vals))


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_cem_converges_on_quadratic(seed):
    """E(x) = sum w (x - c)^2 has its minimum at c; CEM must find it."""
    rng = np.random.default_rng(100 + seed)
    h, a = 2, 7
    c = rng.uniform(-0.5, 0.5, (h, a))
    wq = rng.uniform(0.5, 2.0, (h, a))

    def efn(_r, x):
        return ((x.astype(np.float64) - c) ** 2 * wq).reshape(x.shape[0], -1).sum(axis=1)

    out = cem.cem_plan(efn, n=256, k=32, rounds=20, mu0=np.zeros((h, a)), sigma0=np.ones((h, a)),
                       seed=seed, plan_id=0, lo=-1.0, hi=1.0)
    assert np.abs(out["mu"] - c).max() <= 2e-3
    assert np.abs(out["action"] - c[0]).max() <= 2e-3
    assert out["sigma"].max() < 1e-2
    # the last round's best candidate is the elite list's head, and its energy is the round minimum
    tr = out["trace"]
    assert out["best_idx"] == tr["elites"][-1][0]
    assert tr["energy"][-1][out["best_idx"]] == tr["energy"][-1].min()


def test_cem_follows_supplied_selection_energies():
    """Selection can follow another implementation's scores while recording our own."""
    h, a = 1, 7

    def efn(_r, x):
        return np.abs(x).reshape(x.shape[0], -1).sum(axis=1)

    def rev(_r, x):
        return -efn(_r, x)

    out = cem.cem_plan(efn, 64, 8, 2, np.zeros((h, a)), np.ones((h, a)), 0, 0, -1.0, 1.0,
                       select_energy_fn=rev)
    e0 = out["trace"]["energy"][0]
    assert list(out["trace"]["elites"][0]) == list(select.topk_elites(-e0, 8))


def test_warm_start_closed_form():
    """Next step's Gaussian: shift one step earlier, fresh last step, width floor."""
    mu = np.array([[0.1, -0.2], [0.3, 0.4], [-0.5, 0.6]], np.float32)
    sigma = np.array([[0.9, 0.8], [0.05, np.nan], [0.2, 0.0]], np.float32)
    m, s = cem.warm_start(mu, sigma, 0.0, 1.0, 0.1)
    np.testing.assert_array_equal(m, np.array([[0.3, 0.4], [-0.5, 0.6], [0.0, 0.0]], np.float32))
    np.testing.assert_array_equal(s, np.array([[0.1, 0.1], [0.2, 0.1], [1.0, 1.0]], np.float32))
    # floor 0 carries the widths; horizon 1 is a plain reset
    _, s0 = cem.warm_start(mu, np.abs(np.nan_to_num(sigma)), 0.0, 1.0, 0.0)
    np.testing.assert_array_equal(s0[:2], np.array([[0.05, 0.0], [0.2, 0.0]], np.float32))
    m1, s1 = cem.warm_start(mu[:1], sigma[:1], 0.25, 0.5, 0.0)
    np.testing.assert_array_equal(m1, [[0.25, 0.25]])
    np.testing.assert_array_equal(s1, [[0.5, 0.5]])


def _moving_quadratic(seed, steps, h, a):
    """Target trajectory c[t] and, per control step s, the energy sum_t ||x_t - c[s + t]||^2."""
    ph = np.random.default_rng(seed).uniform(0, 2 * np.pi, a)
    c = 0.6 * np.sin(0.35 * np.arange(steps + h)[:, None] + ph)

    def for_step(s):
        tgt = c[s:s + h]
        return lambda _r, x: ((x.astype(np.float64) - tgt) ** 2).sum(axis=(1, 2)).astype(np.float32)

    return c, for_step


def test_warm_started_three_rounds_track_like_cold_ten():
    """Section 06 B on a closed-form receding-horizon task: after the first H
    steps, a warm-started 3-round search executes actions about as close to the
    target as a fresh 10-round search, and far closer than a fresh 3-round one.
    A warm start that forgot the one-step shift lags the target by a step."""
    h, a, n, k, steps = 4, 3, 64, 8, 12
    err = {"cold10": [], "cold3": [], "warm3": []}
    for seed in range(4):
        c, for_step = _moving_quadratic(seed, steps, h, a)
        for name, rounds, warm in (("cold10", 10, False), ("cold3", 3, False), ("warm3", 3, True)):
            acts, _ = cem.receding_horizon(for_step, steps, n, k, rounds, h, a, 0.0, 1.0, 7 + seed,
                                           -1.0, 1.0, warm)
            err[name].append(np.abs(acts - c[:steps])[h:].mean())
    e = {key: float(np.mean(v)) for key, v in err.items()}
    assert e["warm3"] < 0.4 * e["cold3"], e
    assert e["warm3"] < 2.5 * e["cold10"], e
    assert e["warm3"] < 0.05, e

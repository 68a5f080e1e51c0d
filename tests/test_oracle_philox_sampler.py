"""Pins of the oracle's Philox-4x32-10 generator and Gaussian sampler (CPU)."""
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

from oracle import philox, sampler

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_words(tmp_path_factory):
    """rocRAND's philox4x32_10 engine compiled for the host, as an independent reference."""
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand"):
        pytest.skip("rocRAND headers / hipcc not available")
    exe = str(tmp_path_factory.mktemp("rr") / "rr_words")
    subprocess.run([hipcc, "-x", "c++", "-std=c++17", "-O1", "-I/opt/rocm/include",
                    "-D__HIP_PLATFORM_AMD__", os.path.join(HERE, "pins", "rocrand_philox_words.cpp"),
                    "-o", exe], check=True, capture_output=True)

    def run(rows):
        text = "".join(f"{s} {p} {r} {c}\n" for s, p, r, c in rows)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        return np.array([[int(v) for v in line.split()] for line in out.strip().splitlines()],
                        dtype=np.uint64).astype(np.uint32)

    return run


def test_philox_matches_rocrand(rocrand_words):
    rng = np.random.default_rng(11)
    # rocRAND takes the round through a 64-bit word offset 4 * (round * 2^32 + counter),
    # so rounds stay below 2^30 here.
    rows = [(0, 0, 0, 0), (1, 0, 0, 0), (2, 0, 3, 5), (2**64 - 1, 2**32 - 1, 2**30 - 1, 2**32 - 1),
            (0xDEADBEEFCAFEF00D, 17, 9, 1 << 31)]
    for _ in range(200):
        rows.append((int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2)),
                     int(rng.integers(0, 2**32)), int(rng.integers(0, 2**30)),
                     int(rng.integers(0, 2**32))))
    ref = rocrand_words(rows)
    for (s, p, r, c), want in zip(rows, ref):
        got = philox.philox4x32_10(np.array([c, r, p, 0], dtype=np.uint64).astype(np.uint32),
                                   philox.seed_key(s))
        np.testing.assert_array_equal(got, want, err_msg=f"seed={s} plan={p} round={r} ctr={c}")


def test_raw_words_layout_matches_rocrand(rocrand_words):
    """Element e takes word e & 3 of counter (e >> 2, round, plan_id, 0)."""
    seed, rnd, plan = 2, 4, 9
    words = sampler.raw_words(seed, rnd, plan, 40)
    ref = rocrand_words([(seed, plan, rnd, c) for c in range(10)]).reshape(-1)
    np.testing.assert_array_equal(words, ref)


def test_philox_is_a_bijection_on_a_fixed_key():
    n = 1 << 17
    ctr = np.zeros((n, 4), dtype=np.uint32)
    ctr[:, 0] = np.arange(n, dtype=np.uint32)
    ctr[:, 2] = 5
    out = philox.philox4x32_10(ctr, (123, 456)).view(np.uint64).reshape(n, 2)
    assert np.unique(out, axis=0).shape[0] == n
    # and a different key gives a different stream
    out2 = philox.philox4x32_10(ctr[:64], (124, 456))
    assert not np.array_equal(out2, philox.philox4x32_10(ctr[:64], (123, 456)))


def test_box_muller_closed_form_special_cases():
    # u1 = 1 (w_even = 2^32 - 1): rho = 0 exactly, so both outputs are zero.
    ze, zo = sampler.box_muller(np.array([2**32 - 1], dtype=np.uint32), np.array([12345], dtype=np.uint32))
    assert ze[0] == 0.0 and zo[0] == 0.0
    # u2 = 0: theta = 0, z_even = sqrt(-2 ln u1), z_odd = 0.
    w = np.array([2**31 - 1], dtype=np.uint32)                 # u1 = 1/2
    ze, zo = sampler.box_muller(w, np.array([0], dtype=np.uint32))
    assert zo[0] == 0.0
    assert ze[0] == pytest.approx(np.sqrt(2.0 * np.log(2.0)), rel=1e-15)
    # u2 = 1/4: theta = pi/2, the even output vanishes and the odd one carries rho.
    ze, zo = sampler.box_muller(w, np.array([2**30], dtype=np.uint32))
    assert abs(ze[0]) < 1e-15 and zo[0] == pytest.approx(np.sqrt(2.0 * np.log(2.0)), rel=1e-15)
    # u2 = 1/2: theta = pi, z_even = -rho.
    ze, zo = sampler.box_muller(w, np.array([2**31], dtype=np.uint32))
    assert ze[0] == pytest.approx(-np.sqrt(2.0 * np.log(2.0)), rel=1e-15)


def test_gaussian_distribution():
    z = sampler.gaussian(seed=7, rnd=0, plan_id=0, count=1 << 20).astype(np.float64)
    n = z.size
    assert abs(z.mean()) < 5.0 / np.sqrt(n)
    assert abs(z.var() - 1.0) < 5.0 * np.sqrt(2.0 / n)
    assert stats.kstest(z, "norm").pvalue > 1e-4
    # even/odd partners are uncorrelated, and so are neighbouring counters
    zz = z.reshape(-1, 4)
    assert abs(np.corrcoef(zz[:, 0], zz[:, 1])[0, 1]) < 5.0 / np.sqrt(zz.shape[0])
    assert abs(np.corrcoef(zz[:-1, 0], zz[1:, 0])[0, 1]) < 5.0 / np.sqrt(zz.shape[0])
    # with mu = 0, sigma = 1 the clamp to [-1, 1] hits P(|z| > 1) = 0.3173
    frac = np.mean(np.abs(z) > 1.0)
    p = 2.0 * stats.norm.sf(1.0)
    assert abs(frac - p) < 5.0 * np.sqrt(p * (1 - p) / n)


def test_sample_actions_layout_and_clamp():
    h, a = 2, 7
    mu = np.zeros((h, a), np.float32)
    sigma = np.ones((h, a), np.float32)
    x40 = sampler.sample_actions(mu, sigma, 3, 1, 0, 40, -1.0, 1.0)
    x10 = sampler.sample_actions(mu, sigma, 3, 1, 0, 10, -1.0, 1.0)
    # candidate n's values depend only on its own element indices (chunk invariance)
    np.testing.assert_array_equal(x40[:10], x10)
    z = sampler.gaussian(3, 1, 0, 40 * h * a).reshape(40, h, a)
    np.testing.assert_array_equal(x40, np.clip(z, -1, 1))
    # sigma = 0 collapses every candidate onto the clamped mean
    mu2 = np.full((h, a), 0.25, np.float32)
    mu2[0, 0] = 3.0
    x = sampler.sample_actions(mu2, np.zeros_like(mu2), 3, 1, 0, 5, -1.0, 1.0)
    want = np.clip(mu2, -1, 1)
    np.testing.assert_array_equal(x, np.broadcast_to(want, x.shape))
    # round and plan id select disjoint streams
    assert not np.array_equal(sampler.gaussian(3, 1, 0, 64), sampler.gaussian(3, 2, 0, 64))
    assert not np.array_equal(sampler.gaussian(3, 1, 0, 64), sampler.gaussian(3, 1, 1, 64))


def test_sample_is_rounded_float32_sum_of_product():
    """x = fl(mu + fl(sigma * z)): one rounding per operation, checked with exact rationals."""
    from fractions import Fraction

    h, a, n = 1, 7, 50
    rng = np.random.default_rng(0)
    mu = rng.uniform(-0.5, 0.5, (h, a)).astype(np.float32)
    sigma = rng.uniform(0.0, 0.7, (h, a)).astype(np.float32)
    x = sampler.sample_actions(mu, sigma, 5, 0, 0, n, -1.0, 1.0)
    z = sampler.gaussian(5, 0, 0, n * h * a).reshape(n, h, a)

    def rn32(fr):
        """Nearest float32 to the rational fr, ties to even (exact, no double rounding)."""
        c = np.float32(float(fr))
        best = None
        for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
            err = abs(Fraction(float(cand)) - fr)
            even = (int(np.array(cand, np.float32).view(np.uint32)) & 1) == 0
            key = (err, not even)
            if best is None or key < best[0]:
                best = (key, cand)
        return best[1]

    for i in range(n):
        for j in range(a):
            prod = rn32(Fraction(float(sigma[0, j])) * Fraction(float(z[i, 0, j])))
            s = rn32(Fraction(float(mu[0, j])) + Fraction(float(prod)))
            assert x[i, 0, j] == np.clip(s, -1, 1)

"""GPU parity of the search kernels against the oracle (sampler, top-K, refit, energy)."""
import numpy as np
import pytest

from oracle import energy as o_energy
from oracle import refit as o_refit
from oracle import sampler as o_sampler
from oracle import select as o_select

from .gpu_util import log, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,h,seed,rnd,plan", [(800, 1, 2, 0, 0), (3, 1, 5, 7, 1), (3200, 4, 2, 9, 3),
                                                 (1, 2, 2**64 - 1, 2**32 - 1, 2**32 - 1), (0, 1, 1, 1, 1)])
def test_sampler_matches_oracle(gpu_lib, n, h, seed, rnd, plan):
    import torch
    from cem_jepa_predictor_amd import _lib

    log(f"sampler n={n} h={h} seed={seed} round={rnd} plan={plan}")
    a = 7
    rng = np.random.default_rng(n + h)
    mu = rng.uniform(-0.5, 0.5, (h, a)).astype(np.float32)
    sigma = rng.uniform(0.0, 1.2, (h, a)).astype(np.float32)
    x = torch.empty((max(n, 1), h, a), dtype=torch.float32, device="cuda")
    raw = torch.empty(max(n, 1) * h * a, dtype=torch.int32, device="cuda")
    _lib.cem_sample(to_dev(mu), to_dev(sigma), n, seed, rnd, plan, -1.0, 1.0, x, raw)
    torch.cuda.synchronize()
    if n == 0:
        return
    words = to_np(raw).view(np.uint32)
    np.testing.assert_array_equal(words, o_sampler.raw_words(seed, rnd, plan, n * h * a))
    want = o_sampler.sample_actions(mu, sigma, seed, rnd, plan, n, -1.0, 1.0)
    got = to_np(x)[:n]
    # float64 libm differences can move z by one float32 ulp in rare cases: count them
    diff = got != want
    ulps = np.abs(got.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64))
    log(f"  sampler mismatches: {int(diff.sum())} of {got.size}")
    assert ulps.max() <= 1
    assert diff.sum() <= max(2, got.size // 100000)


def _energies_with_specials(rng, n):
    e = rng.standard_normal(n).astype(np.float32)
    if n >= 16:
        e[rng.integers(0, n, 4)] = np.nan
        e[rng.integers(0, n, 3)] = np.inf
        e[rng.integers(0, n, 3)] = -np.inf
        e[rng.integers(0, n, 3)] = -0.0
        e[rng.integers(0, n, 3)] = 0.0
        e[rng.integers(0, n, n // 4)] = 0.5   # many ties
    return e


@pytest.mark.parametrize("n,k", [(1, 1), (7, 3), (64, 8), (800, 80), (801, 800), (3200, 320),
                                 (16384, 1638), (1000, 1000)])
def test_topk_bit_exact(gpu_lib, n, k):
    import torch
    from cem_jepa_predictor_amd import _lib

    log(f"topk n={n} k={k}")
    e = _energies_with_specials(np.random.default_rng(n), n)
    idx = torch.empty(k, dtype=torch.int32, device="cuda")
    _lib.topk_select(to_dev(e), k, idx)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(idx), o_select.topk_elites(e, k))


@pytest.mark.parametrize("n,k,h", [(800, 80, 1), (256, 32, 3), (3200, 320, 1), (9, 9, 4), (5, 1, 2)])
def test_elite_refit_matches_oracle(gpu_lib, n, k, h):
    import torch
    from cem_jepa_predictor_amd import _lib

    log(f"elite_refit n={n} k={k} h={h}")
    rng = np.random.default_rng(n * 7 + k)
    e = _energies_with_specials(rng, n)
    x = np.clip(rng.standard_normal((n, h, 7)), -1, 1).astype(np.float32)
    idx = torch.empty(k, dtype=torch.int32, device="cuda")
    mu = torch.empty((h, 7), dtype=torch.float32, device="cuda")
    sg = torch.empty((h, 7), dtype=torch.float32, device="cuda")
    _lib.elite_refit(to_dev(e), to_dev(x), k, idx, mu, sg)
    torch.cuda.synchronize()
    want_idx = o_select.topk_elites(e, k)
    np.testing.assert_array_equal(to_np(idx), want_idx)
    want_mu, want_sg = o_refit.refit(x, want_idx)
    np.testing.assert_allclose(to_np(mu), want_mu, rtol=2e-7, atol=1e-7)
    np.testing.assert_allclose(to_np(sg), want_sg, rtol=2e-7, atol=1e-7)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n,p,e", [(5, 16, 128), (3, 7, 9), (64, 66, 512), (0, 4, 8)])
def test_energy_l1_matches_oracle(gpu_lib, dtype, n, p, e):
    import torch
    from cem_jepa_predictor_amd import _lib, inputs

    log(f"energy {dtype} n={n} p={p} e={e}")
    zp, zg = inputs.make_predictions(max(n, 1), p, e, seed=n + p)
    tz = to_dev(zp[:n] if n else zp[:1])
    if dtype == "bf16":
        tz = tz.to(torch.bfloat16)
    out = torch.full((max(n, 1),), -1.0, dtype=torch.float32, device="cuda")
    if n == 0:
        _lib.load().energy_l1(tz.data_ptr(), 1 if dtype == "bf16" else 0, to_dev(zg).data_ptr(), 0, p, e,
                              out.data_ptr(), None)
    else:
        _lib.energy_l1(tz.reshape(n, p, e), to_dev(zg), out)
    torch.cuda.synchronize()
    if n == 0:
        assert to_np(out)[0] == -1.0
        return
    want = o_energy.energy_l1(to_np(tz).reshape(n, p, e), zg)
    np.testing.assert_allclose(to_np(out), want, rtol=2e-5, atol=0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_energy_l1_is_independent_of_the_batch(gpu_lib, dtype):
    """A candidate's energy is summed in the same order whether its workgroup scores
    four candidates (n divisible by 4) or only it: every sub-batch gives the same bits."""
    import torch
    from cem_jepa_predictor_amd import _lib, inputs

    zp, zg = inputs.make_predictions(12, 16, 136, seed=5)
    tz = to_dev(zp)
    if dtype == "bf16":
        tz = tz.to(torch.bfloat16)
    full = torch.empty(12, dtype=torch.float32, device="cuda")
    _lib.energy_l1(tz, to_dev(zg), full)
    for lo, hi in ((0, 7), (3, 12), (5, 6), (4, 8)):
        part = torch.empty(hi - lo, dtype=torch.float32, device="cuda")
        _lib.energy_l1(tz[lo:hi].contiguous(), to_dev(zg), part)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_np(part), to_np(full)[lo:hi], err_msg=f"candidates {lo}..{hi - 1}")


def test_energy_l1_full_size_sampled(gpu_lib):
    """N=800 candidates of [256, 1408] bf16 predictions, oracle on a sample of rows."""
    import torch
    from cem_jepa_predictor_amd import _lib

    log("energy full size 800 x 256 x 1408 bf16")
    rng = np.random.default_rng(0)
    zp_h = rng.standard_normal((800, 256, 1408), dtype=np.float32)
    zg_h = rng.standard_normal((256, 1408), dtype=np.float32)
    zp = to_dev(zp_h).to(torch.bfloat16)
    zg = to_dev(zg_h)
    torch.cuda.synchronize()
    out = torch.empty(800, dtype=torch.float32, device="cuda")
    _lib.energy_l1(zp, zg, out)
    torch.cuda.synchronize()
    got = to_np(out)
    ref_t = (zp.float() - zg).abs().mean(dim=(1, 2))
    torch.cuda.synchronize()
    log(f"  nan rows {int(np.isnan(got).sum())}, max |ours - torch| {np.nanmax(np.abs(got - to_np(ref_t))):.3e}, "
        f"stream {torch.cuda.current_stream().cuda_stream}")
    rows = np.arange(0, 800, 53)
    want = o_energy.energy_l1(zp[rows].float().cpu().numpy(), zg_h)
    np.testing.assert_allclose(got[rows], want, rtol=2e-5, atol=0)
    # deterministic on a second call
    _lib.energy_l1(zp, zg, out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(out), got)


def test_energy_l1_device_generated_inputs(gpu_lib):
    """Inputs written by torch kernels right before the call: the binding orders the
    library's stream after torch's current stream."""
    import torch
    from cem_jepa_predictor_amd import _lib

    log("energy with torch.randn inputs on the device")
    g = torch.Generator(device="cuda").manual_seed(0)
    zp = torch.randn((800, 256, 1408), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    zg = torch.randn((256, 1408), generator=g, device="cuda", dtype=torch.float32)
    out = torch.full((800,), -7.0, dtype=torch.float32, device="cuda")
    _lib.energy_l1(zp, zg, out)
    ref = (zp.float() - zg).abs().mean(dim=(1, 2))
    torch.cuda.synchronize()
    got, want = to_np(out), to_np(ref)
    log(f"  ours: nan {int(np.isnan(got).sum())}, untouched {int((got == -7.0).sum())}")
    np.testing.assert_allclose(got, want, rtol=2e-5, atol=0)


def test_mfma_ceiling_probe_is_plausible(gpu_lib):
    """The register-only MFMA probe cannot beat the part's published dense bf16
    peak (2.5 PFLOP/s at 2.4 GHz, 256 CUs x 4096 FLOP/clk) and its clock reading
    must be a real shader clock; with changing operand bits it runs no faster
    than with constant ones (the part lowers its clock under power)."""
    from cem_jepa_predictor_amd import _lib

    ct, cmhz = _lib.mfma_ceiling(False, 6)
    rt, rmhz = _lib.mfma_ceiling(True, 6)
    log(f"mfma ceiling: constant {ct:.0f} TFLOP/s @ {cmhz:.0f} MHz, random {rt:.0f} TFLOP/s @ {rmhz:.0f} MHz")
    for tf, mhz in ((ct, cmhz), (rt, rmhz)):
        assert 300.0 < mhz < 2600.0
        assert 100.0 < tf < 2600.0
        # throughput and clock agree: 256 CUs x 4096 FLOP per clock at most
        assert tf <= 256 * 4096 * mhz * 1e6 / 1e12 * 1.05
    assert rt <= ct * 1.05


@pytest.mark.parametrize("h,a,floor", [(1, 7, 0.0), (2, 7, 0.5), (8, 32, 0.0), (32, 32, 1.0)])
def test_warm_start_bit_exact(gpu_lib, h, a, floor):
    """cem_warm_start against the oracle's warm_start, out of place and in place
    (h * a = 1024 is the largest accepted size)."""
    import torch
    from cem_jepa_predictor_amd import _lib
    from oracle import cem

    log(f"warm start h={h} a={a} floor={floor}")
    rng = np.random.default_rng(h * 100 + a)
    mu = rng.uniform(-1, 1, (h, a)).astype(np.float32)
    sigma = rng.uniform(0, 1.5, (h, a)).astype(np.float32)
    if h > 1:
        sigma[1, 0] = np.nan
        sigma[-1, -1] = 0.0
    want_mu, want_sigma = cem.warm_start(mu, sigma, 0.125, 0.75, floor)
    mt, st = to_dev(mu), to_dev(sigma)
    mo = torch.full((h, a), 7.0, dtype=torch.float32, device="cuda")
    so = torch.full((h, a), 7.0, dtype=torch.float32, device="cuda")
    _lib.warm_start(mt, st, 0.125, 0.75, floor, mo, so)
    _lib.warm_start(mt, st, 0.125, 0.75, floor, mt, st)   # in place
    torch.cuda.synchronize()
    for got_mu, got_sigma in ((mo, so), (mt, st)):
        np.testing.assert_array_equal(to_np(got_mu), want_mu)
        np.testing.assert_array_equal(to_np(got_sigma), want_sigma)


@pytest.mark.parametrize("rows,cols", [(37, 1024), (5, 8), (64, 512)])
def test_fp8_quantize_rows_bit_exact(gpu_lib, rows, cols):
    """The device's e4m3 row quantization (scale and every code) equals the oracle's."""
    import torch
    from cem_jepa_predictor_amd import _lib
    from oracle import fp8

    log(f"fp8 quantize rows={rows} cols={cols}")
    rng = np.random.default_rng(rows * cols)
    x = (rng.standard_normal((rows, cols)) * rng.choice([1e-3, 1.0, 50.0], (rows, 1))).astype(np.float32)
    x[0] = 0.0
    if rows > 3:
        x[3, :4] = [448.0, -1e-9, 2.0 ** -12, 3.0]
    codes = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    scale = torch.empty(rows, dtype=torch.float32, device="cuda")
    _lib.fp8_quantize_rows(to_dev(x), codes, scale)
    torch.cuda.synchronize()
    want_codes, want_scale = fp8.quantize_rows(x)
    np.testing.assert_array_equal(to_np(scale), want_scale)
    np.testing.assert_array_equal(to_np(codes), want_codes)

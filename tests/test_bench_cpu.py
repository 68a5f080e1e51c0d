"""Host-side pieces of bench.py: the plan-step roofline and the one-GPU contract."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from cem_jepa_predictor_amd import inputs  # noqa: E402


def test_plan_roofline_matches_hand_count():
    """V-JEPA2-AC shape, 800 x 10, H = 1, counted by hand per round at 2.5 PFLOP/s and
    8 TB/s: the four projections per layer are MFMA-bound, attention and the energy
    are HBM-bound."""
    wl = inputs.WORKLOADS["vjepa2ac"]
    M, d, F, P, E, N = 800 * 258, 1024, 4096, 256, 1408, 800
    gemm_ms = 2 * M * d * (3 * d + d + F + F) / 2.5e15 * 1e3
    attn_ms = 2 * N * (258 * d + 2 * 258 * d + 258 * d) / 8e12 * 1e3
    out_ms = 2 * N * P * E * d / 2.5e15 * 1e3
    energy_ms = (N * P * E * 2 + P * E * 4) / 8e12 * 1e3
    in_ms = 2 * P * d * E / 2.5e15 * 1e3
    want = in_ms + 10 * (24 * (gemm_ms + attn_ms) + out_ms + energy_ms)
    got = bench.plan_roofline_ms(wl.model, wl.plan, 2500.0)
    assert got == pytest.approx(want, rel=1e-3)
    assert 540 < got < 560


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr

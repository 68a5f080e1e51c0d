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


# --- counter and trace summaries (the tables under profiles/ come from these) -------------

GEMM2 = "void cem::(anonymous namespace)::gemm_bf16_kernel<2, false, false>(void const*, int)"
ATTN = "void cem::(anonymous namespace)::attn_bf16_single_kernel<17>(cem::AttnArgs)"


def _write_csv(path, header, rows):
    import csv

    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)
    return str(path)


def _table(out):
    """{kernel: [cells after the name]} from a printed markdown table."""
    rows = {}
    for line in out.splitlines():
        if line.startswith("| `"):
            cells = [c.strip() for c in line.strip("|").split("|")]
            rows[cells[0].strip("`")] = cells[1:]
    return rows


def test_summarize_stats_shares_and_gemm_mean(tmp_path, capsys):
    p = _write_csv(tmp_path / "stats.csv", ["Name", "Calls", "TotalDurationNs", "AverageNs"],
                   [[GEMM2, 4, 4_000_000, 1_000_000], [ATTN, 2, 1_000_000, 500_000],
                    ["void cem::(anonymous namespace)::gemm_bf16_kernel<1, false, true>(x)", 1, 3_000_000, 3_000_000]])
    bench.summarize_stats(p)
    out = capsys.readouterr().out
    t = _table(out)
    assert t["cem::gemm_bf16_kernel<2, false, false>"] == ["4", "1000.0", "4.0", "50.0%"]
    assert t["cem::attn_bf16_single_kernel<17>"] == ["2", "500.0", "1.0", "12.5%"]
    # (4 + 3) ms over 5 GEMM launches
    assert "gemm_bf16_kernel, all kinds: 5 launches, mean 1.4000 ms per launch" in out


def test_summarize_traffic_scales_by_the_copy(tmp_path, capsys):
    hdr = ["Kernel_Name", "Counter_Value"]
    # the copy of 1 MiB reads as 512 KiB of FETCH_SIZE and 1024 KiB of WRITE_SIZE
    cf = _write_csv(tmp_path / "cf.csv", hdr, [["__amd_rocclr_copyBuffer", 512.0]] * 3)
    cw = _write_csv(tmp_path / "cw.csv", hdr, [["__amd_rocclr_copyBuffer", 1024.0]] * 3)
    f = _write_csv(tmp_path / "f.csv", hdr, [[GEMM2, 100.0], [GEMM2, 300.0]])
    w = _write_csv(tmp_path / "w.csv", hdr, [[GEMM2, 50.0], [GEMM2, 50.0]])
    st = _write_csv(tmp_path / "st.csv", ["Name", "AverageNs"], [[GEMM2, 1000.0]])
    bench.summarize_traffic(f, w, cf, cw, copy_bytes=1 << 20, stats=st)
    out = capsys.readouterr().out
    assert "FETCH_SIZE x 2.0000, WRITE_SIZE x 1.0000" in out
    row = _table(out)["cem::gemm_bf16_kernel<2, false, false>"]
    want = (200.0 * 2 + 50.0) * 1024                       # mean KiB, scaled, in bytes
    assert row[:3] == ["2", "200.0", "50.0"]
    assert float(row[3]) == pytest.approx(want, rel=1e-3)
    assert float(row[4]) == pytest.approx(1.0)               # 1000 ns
    assert float(row[5]) == pytest.approx(want / 1000.0, rel=1e-3)   # bytes per ns = GB/s
    assert f"2 dispatches, {want:.0f} bytes per launch" in out


def _pmc_rows(kernel, dispatch, counters, start=0, end=1000):
    return [[dispatch, kernel, name, value, start, end] for name, value in counters.items()]


PMC_HDR = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def test_summarize_sq_fractions(tmp_path, capsys):
    # one dispatch of 1000 cycles per XCD: GRBM_GUI_ACTIVE sums the 8 XCDs
    c = {"GRBM_GUI_ACTIVE": 8000.0, "SQ_ACTIVE_INST_VALU": 128_000.0, "SQ_VALU_MFMA_BUSY_CYCLES": 512_000.0,
         "SQ_WAVE_CYCLES": 10_000.0, "SQ_WAIT_INST_ANY": 4_000.0, "SQ_WAIT_INST_LDS": 250.0,
         "SQ_LDS_BANK_CONFLICT": 300.0, "SQ_BUSY_CYCLES": 1.0, "SQ_ACTIVE_INST_LDS": 1.0}
    p = _write_csv(tmp_path / "sq.csv", PMC_HDR, _pmc_rows(GEMM2, 1, c))
    bench.summarize_sq(p)
    row = _table(capsys.readouterr().out)["cem::gemm_bf16_kernel<2, false, false>"]
    # VALU: 4 x 128000 / (1024 x 1000) = 0.5; MFMA: 512000 / 1024000 = 0.5
    assert row == ["1", "0.50", "0.50", "0.40", "0.025", "300"]


def test_summarize_path_fractions_and_bytes_per_clock(tmp_path, capsys):
    wl = inputs.WORKLOADS["vjepa2ac"]
    M, d = wl.plan.n_samples * wl.model.block_tokens, wl.model.d_model
    cyc = 1_000_000.0                                       # per-XCD cycles of the one dispatch
    c = {"GRBM_GUI_ACTIVE": 8 * cyc, "TCC_HIT_sum": 75.0, "TCC_MISS_sum": 25.0,
         "TCP_TCC_READ_REQ_LATENCY_sum": 30_000.0, "TCP_TCC_READ_REQ_sum": 100.0,
         "TA_TA_BUSY_sum": 0.25 * 256 * cyc, "TD_TD_BUSY_sum": 0.5 * 256 * cyc,
         "TD_TC_STALL_sum": 0.2 * 256 * cyc, "TCP_PENDING_STALL_CYCLES_sum": 0.1 * 256 * cyc,
         "TA_BUFFER_READ_LDS_WAVEFRONTS_sum": 1_000_000.0}
    p = _write_csv(tmp_path / "path.csv", PMC_HDR, _pmc_rows(GEMM2, 7, c, start=0, end=500_000))
    bench.summarize_path(p, "vjepa2ac")
    row = _table(capsys.readouterr().out)["cem::gemm_bf16_kernel<2, false, false>"]
    # 500 us; 1e6 cycles in 500 us = 2000 MHz
    assert row[:9] == ["1", "500.0", "2000", "0.75", "300", "0.25", "0.50", "0.20", "0.10"]
    # LDS-DMA bytes + residual read + result write + row statistics (M d / 8)
    want = (1_000_000 * 1024 + 2 * M * d * 2 + M * d // 8) / (cyc * 256)
    assert float(row[9]) == pytest.approx(want, abs=0.05)

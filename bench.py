#!/usr/bin/env python3
"""Benchmark of the CEM plan step on one MI355X.

Workload: the V-JEPA2-AC-shaped predictor (24 layers, d 1024, 16 heads, MLP 4096,
256 patch tokens, encoder width 1408, horizon 1) under the search settings of
page "Real-Time Inference for JEPA World Model Architectures with Ray"
(section 01: 800 candidates, best 80 kept, 10 rounds).  Random-init weights and
N(0, 1) embeddings from fixed seeds (the pages ship neither weights nor frames).

One step = one full cem_plan call (sample, rollout, L1 energy, top-K, refit for
all 10 rounds), inputs resident in HBM.  Prints ONE JSON line:
  value       = candidate evaluations per second = N * R / plan time
  ms_per_step = milliseconds per plan step (graph replay)
  roofline    = the dense-GEMM kernel (the dominant kernel), useful FLOPs over
                its HIP-event-timed launch durations, against bf16 dense MFMA peak;
                next to it the part's own sustained register-only MFMA ceiling
                (cem_mfma_ceiling), measured in the same run
  cpu_baseline= the oracle (NumPy float64) on the host cores, on a bounded
                sample of candidates, extrapolated to the metric's unit

--batch B times fleet batching (section 06 C): B independent problems of N
candidates each, planned by one cem_plan_batched call (value = B * N * R / time).
--rounds R and --warm-start time the receding-horizon variant of section 06 B
("Warm-started CEM"): every timed plan starts from cem_warm_start of the
previous plan's final Gaussian (one step earlier, fresh last step, widths kept
down to --sigma-floor) instead of the fresh Gaussian, with R rounds.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
MFMA_F32_PEAK_TFLOPS = 157.3     # MI355X fp32 (reference for fp32 models)
MFMA_FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8

# HBM-side bytes per dense-GEMM launch, from two rocprofv3 --pmc passes over
# `bench.py --steps 1 --warmup 0 --no-cpu-baseline` (FETCH_SIZE, then WRITE_SIZE,
# KiB per dispatch, launch-weighted mean over every gemm_bf16_kernel dispatch),
# each scaled by what the same counter reads for a 1 GiB device copy
# (`bench.py --copy-bytes 1073741824`): FETCH_SIZE x 2.0, WRITE_SIZE x 1.0.
# Valid only for the GEMM sources they were taken on (sha256 below); reported
# as null once those change.
GEMM_COUNTERS = {
    "sources_sha256": "b906aec90b033743e46b254b684258b3272ca8a7081afd5b9e100b824296d042",
    "bytes_per_launch": 3434899121,
}
GEMM_SOURCES = ("cem_jepa_predictor_amd/csrc/gemm.hip", "cem_jepa_predictor_amd/csrc/common.hpp")


def gemm_sources_sha256() -> str:
    import hashlib

    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def summarize_stats(path: str, top: int = 12) -> None:
    """Markdown table of a rocprofv3 --stats kernel_stats.csv, plus the
    launch-weighted mean duration of the dense-GEMM kernel (all epilogue kinds)."""
    import csv

    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    print("| kernel | calls | avg (us) | total (ms) | share |")
    print("|---|---:|---:|---:|---:|")
    for r in rows[:top]:
        name = r["Name"].replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
        print(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
              f"{float(r['TotalDurationNs']) / 1e6:.1f} | {float(r['TotalDurationNs']) / total:.1%} |")
    g = [r for r in rows if "gemm_bf16_kernel" in r["Name"]]
    calls = sum(int(r["Calls"]) for r in g)
    ns = sum(float(r["TotalDurationNs"]) for r in g)
    if calls:
        print(f"\ngemm_bf16_kernel, all kinds: {calls} launches, mean {ns / calls / 1e6:.4f} ms per launch")


def summarize_traffic(fetch: str, write: str, copy_fetch: str, copy_write: str,
                      copy_bytes: int, stats: str | None = None) -> None:
    """Per-kernel FETCH_SIZE / WRITE_SIZE means (KiB per dispatch) of two
    rocprofv3 --pmc passes, scaled by the copy calibration; with the
    --kernel-trace --stats CSV of the same command, also each kernel's mean
    duration and the HBM-side GB/s it reaches."""
    import collections
    import csv

    def per_kernel(path):
        d = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            d[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return d

    def copy_mean(path):
        d = per_kernel(path)
        v = [x for k, xs in d.items() if "copyBuffer" in k or "copy" in k.lower() for x in xs]
        return sum(v) / len(v)

    kib = copy_bytes / 1024
    ff, fw = kib / copy_mean(copy_fetch), kib / copy_mean(copy_write)
    print(f"copy calibration ({copy_bytes} bytes): FETCH_SIZE x {ff:.4f}, WRITE_SIZE x {fw:.4f}\n")
    df, dw = per_kernel(fetch), per_kernel(write)
    short = lambda k: k.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")  # noqa: E731
    avg_ns = {}
    if stats:
        for r in csv.DictReader(open(stats)):
            avg_ns[short(r["Name"])] = float(r["AverageNs"])
    print("| kernel | dispatches | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | scaled bytes / dispatch"
          + (" | mean duration (us) | HBM-side GB/s |" if stats else " |"))
    print("|---|---:|---:|---:|---:|" + ("---:|---:|" if stats else ""))
    keys = sorted(df, key=lambda k: -sum(df[k]))
    for k in keys:
        f = sum(df[k]) / len(df[k])
        w = sum(dw.get(k, [0.0])) / max(len(dw.get(k, [])), 1)
        name = short(k)
        b = (f * ff + w * fw) * 1024
        row = f"| `{name}` | {len(df[k])} | {f:.1f} | {w:.1f} | {b:.4g} |"
        if stats:
            ns = avg_ns.get(name)
            row += f" {ns / 1e3:.1f} | {b / ns:.0f} |" if ns else " - | - |"
        print(row)
    gf = [x for k, xs in df.items() if "gemm_bf16_kernel" in k for x in xs]
    gw = [x for k, xs in dw.items() if "gemm_bf16_kernel" in k for x in xs]
    if gf and gw:
        b = (sum(gf) / len(gf) * ff + sum(gw) / len(gw) * fw) * 1024
        print(f"\ngemm_bf16_kernel, all kinds: {len(gf)} dispatches, {b:.0f} bytes per launch; "
              f"GEMM sources sha256 {gemm_sources_sha256()}")


def summarize_sq(path: str) -> None:
    """Per-kernel shader-engine utilization from one rocprofv3 --pmc pass over
    SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_WAIT_INST_LDS
    SQ_WAIT_INST_ANY SQ_VALU_MFMA_BUSY_CYCLES SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE (sums over
    each kernel's dispatches; 256 CUs of 4 SIMDs, GRBM_GUI_ACTIVE summed over the 8 XCDs):
    VALU busy = 4 SQ_ACTIVE_INST_VALU / (1024 GRBM_GUI_ACTIVE / 8), MFMA busy =
    SQ_VALU_MFMA_BUSY_CYCLES / (1024 GRBM_GUI_ACTIVE / 8), waiting = SQ_WAIT_INST_ANY /
    SQ_WAVE_CYCLES."""
    import collections
    import csv

    agg = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(set)
    short = lambda k: k.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")  # noqa: E731
    for r in csv.DictReader(open(path)):
        k = short(r["Kernel_Name"])
        agg[k][r["Counter_Name"]] += float(r["Counter_Value"])
        disp[k].add(r["Dispatch_Id"])
    print("| kernel | dispatches | VALU busy | MFMA busy | wave cycles waiting (any) | of which on LDS "
          "| LDS bank-conflict cycles per dispatch |")
    print("|---|---:|---:|---:|---:|---:|---:|")
    for k in sorted(agg, key=lambda k: -agg[k]["GRBM_GUI_ACTIVE"]):
        a, n = agg[k], len(disp[k])
        g = 1024 * a["GRBM_GUI_ACTIVE"] / 8
        if g <= 0:
            continue
        wc = a["SQ_WAVE_CYCLES"] or 1.0
        print(f"| `{k}` | {n} | {4 * a['SQ_ACTIVE_INST_VALU'] / g:.2f} | {a['SQ_VALU_MFMA_BUSY_CYCLES'] / g:.2f} "
              f"| {a['SQ_WAIT_INST_ANY'] / wc:.2f} | {a['SQ_WAIT_INST_LDS'] / wc:.3f} "
              f"| {a['SQ_LDS_BANK_CONFLICT'] / n:.3g} |")


def summarize_path(path: str, workload: str = "vjepa2ac") -> None:
    """Per-kernel memory-path figures from one rocprofv3 --pmc pass over
    TCP_TCC_READ_REQ_LATENCY_sum TCP_TCC_READ_REQ_sum TCP_PENDING_STALL_CYCLES_sum TCC_HIT_sum
    TCC_MISS_sum TA_TA_BUSY_sum TA_BUFFER_READ_LDS_WAVEFRONTS_sum TD_TD_BUSY_sum TD_TC_STALL_sum
    GRBM_GUI_ACTIVE (sums over each kernel's dispatches; durations from the dispatches' own
    timestamps).  L2 hit rate = hits / (hits + misses); L1->L2 read latency = latency sum / read
    requests; TA, TD and TCP figures = their cycles / (256 units x GRBM_GUI_ACTIVE / 8); clock =
    GRBM_GUI_ACTIVE / 8 per dispatch over its duration.  For the layer GEMMs of `workload` (M = N B
    rows), bytes per clock per CU = (LDS-DMA wavefronts x 1 KB + residual rows read + bf16 results
    and row statistics written) / (cycles x 256)."""
    import collections
    import csv

    from cem_jepa_predictor_amd import inputs

    wl = inputs.WORKLOADS[workload]
    m = wl.model
    M = wl.plan.n_samples * m.block_tokens
    d, F = m.d_model, m.d_mlp
    # results written + residual rows read per dispatch, averaged over the launches of each kind
    # output / down: residual read + result write + the LayerNorm piece statistics (M d / 8 bytes;
    # every residual launch but the last layer's MLP down writes them)
    extra = {"gemm_bf16_kernel<2, false, false>": 2 * (M * d * 2) + (M * d // 8 if m.dtype == "bf16" and d % 256 == 0 else 0),
             "gemm_bf16_kernel<1, false, true>": M * F * 2,               # MLP up
             "gemm_bf16_kernel<0, false, true>": M * 3 * d * 2}           # q|k|v
    agg = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(dict)
    short = lambda k: k.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")  # noqa: E731
    for r in csv.DictReader(open(path)):
        k = short(r["Kernel_Name"])
        agg[k][r["Counter_Name"]] += float(r["Counter_Value"])
        disp[k][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    print("| kernel | dispatches | mean duration (us) | clock (MHz) | L2 hit rate | L1→L2 read latency (cycles) "
          "| TA busy | TD busy | TD waiting for L2 data | L1 stalled on pending L2 data "
          "| operand + residual + result bytes per clock per CU |")
    print("|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|")
    for k in sorted(agg, key=lambda k: -agg[k]["GRBM_GUI_ACTIVE"]):
        a, n = agg[k], len(disp[k])
        cyc = a["GRBM_GUI_ACTIVE"] / 8                       # per-XCD cycles, all dispatches
        if cyc <= 0:
            continue
        dur = sum(disp[k].values())
        hits, miss = a["TCC_HIT_sum"], a["TCC_MISS_sum"]
        reqs = a["TCP_TCC_READ_REQ_sum"] or 1.0
        units = 256 * cyc
        bpc = "—"
        for kind, eb in extra.items():
            if k.endswith(kind):
                bpc = f"{(a['TA_BUFFER_READ_LDS_WAVEFRONTS_sum'] * 1024 + eb * n) / units:.1f}"
        print(f"| `{k}` | {n} | {dur / n * 1e6:.1f} | {cyc / dur / 1e6:.0f} | {hits / max(hits + miss, 1):.2f} "
              f"| {a['TCP_TCC_READ_REQ_LATENCY_sum'] / reqs:.0f} | {a['TA_TA_BUSY_sum'] / units:.2f} "
              f"| {a['TD_TD_BUSY_sum'] / units:.2f} | {a['TD_TC_STALL_sum'] / units:.2f} "
              f"| {a['TCP_PENDING_STALL_CYCLES_sum'] / units:.2f} | {bpc} |")


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


HBM_PEAK_BYTES_PER_S = 8.0e12


def plan_roofline_ms(m, pc, peak_tflops: float) -> float:
    """Per-kernel roofline of one plan step: the sum over kernels of
    max(FLOPs / MFMA peak, bytes / HBM peak), each activation read or written once
    per kernel, LayerNorm folded into the projections (no separate pass), KV-cached
    block-causal attention counted on its unmasked part only.  fp8 models: the
    q|k|v and MLP-up projections at the fp8 peak with 1-byte operands."""
    es = 4 if m.dtype == "f32" else 2
    peak = peak_tflops * 1e12
    N, R, H = pc.n_samples, pc.rounds, pc.horizon
    B, P, E, d, F, L = m.patches + 2, m.patches, m.enc_dim, m.d_model, m.d_mlp, m.layers
    M = N * B

    def gemm(rows, n, k, residual=False, f8=False):
        flop = 2.0 * rows * n * k
        ein = 1 if f8 else es
        byts = ein * (rows * k + n * k) + es * rows * n * (2 if residual else 1)
        return max(flop / (MFMA_FP8_PEAK_TFLOPS * 1e12 if f8 else peak), byts / HBM_PEAK_BYTES_PER_S)

    total = gemm(P, d, E)                                   # frame in-projection, once per plan
    per_round = 0.0
    for t in range(H):
        if t > 0:
            per_round += gemm(N * P, d, E)                  # in-projection of the fed-back frame
        for _ in range(L):
            f8 = m.dtype == "fp8"
            per_round += (gemm(M, 3 * d, d, f8=f8) + gemm(M, d, d, True) + gemm(M, F, d, f8=f8)
                          + gemm(M, d, F, True))
            kv = (t + 1) * B
            flop = 4.0 * N * B * kv * d
            byts = es * N * (B * d + 2 * kv * d + B * d)
            per_round += max(flop / peak, byts / HBM_PEAK_BYTES_PER_S)
        per_round += gemm(N * P, E, d)                      # out-projection
    per_round += (N * P * E * es + P * E * 4) / HBM_PEAK_BYTES_PER_S   # L1 energy
    return (total + R * per_round) * 1e3


def host_cpu():
    """(CPU model name, logical CPUs this process may run on)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = os.cpu_count() or 1
    return model, avail


def cpu_baseline(wl, sample_seconds: float):
    """Time the oracle on the host: whole candidates through the predictor + energy,
    then the per-round search bookkeeping, extrapolated to candidate-evals/s."""
    import numpy as np

    from cem_jepa_predictor_amd import inputs
    from oracle import energy as o_energy
    from oracle import predictor as o_pred
    from oracle import refit as o_refit
    from oracle import sampler as o_sampler
    from oracle import select as o_select

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    m, pc = wl.model, wl.plan
    w = inputs.make_weights(m, wl.weight_seed)
    z_obs, z_goal, s0 = inputs.make_embeddings(m, wl.embed_seed)
    pred = o_pred.Predictor(w, m.layers, m.heads, m.ln_eps)
    del w
    mu = np.zeros((pc.horizon, m.action_dim), np.float32)
    sg = np.ones_like(mu)
    x = o_sampler.sample_actions(mu, sg, pc.seed, 0, pc.plan_id, pc.n_samples, pc.clamp_lo, pc.clamp_hi)
    done, t0 = 0, time.perf_counter()
    while done < 64:
        o_energy.energy_l1(pred.rollout_cached(x[done:done + 1], z_obs, s0), z_goal)
        done += 1
        if time.perf_counter() - t0 >= sample_seconds:
            break
    t_eval = time.perf_counter() - t0
    evals_per_s = done / t_eval
    # the same rollout on one thread (at least one candidate)
    one_core = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1):
            t2 = time.perf_counter()
            o_energy.energy_l1(pred.rollout_cached(x[:1], z_obs, s0), z_goal)
            one_core = 1.0 / (time.perf_counter() - t2)
    except ImportError:  # pragma: no cover
        pass
    # search bookkeeping of one full plan (sample + select + refit for every round)
    t1 = time.perf_counter()
    e = np.random.default_rng(0).standard_normal(pc.n_samples)
    for r in range(pc.rounds):
        xr = o_sampler.sample_actions(mu, sg, pc.seed, r, pc.plan_id, pc.n_samples, pc.clamp_lo, pc.clamp_hi)
        el = o_select.topk_elites(e, pc.n_elites)
        o_refit.refit(xr, el)
    t_book = time.perf_counter() - t1
    plan_s = pc.n_samples * pc.rounds / evals_per_s + t_book
    cpu_model, host_cpus = host_cpu()
    return {"value": round(evals_per_s, 6), "unit": "candidate-evals/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": cpu_model, "host_cpus": host_cpus,
            "one_core_value": round(one_core, 6) if one_core else None,
            "sample": (f"{done} candidate rollouts + L1 energies of the {wl.name} workload in "
                       f"{t_eval:.1f} s (NumPy float64), plus one plan's sampling/top-K/refit "
                       f"({t_book * 1e3:.1f} ms); extrapolated plan step {plan_s:.0f} s")}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--timer-steps", type=int, default=5,
                    help="eager steps with the library's GEMM timers (roofline.achieved)")
    ap.add_argument("--workload", default="vjepa2ac")
    ap.add_argument("--samples", type=int, default=0, help="override N (sweep); K = N / 10")
    ap.add_argument("--rounds", type=int, default=0, help="override R (rounds per plan)")
    ap.add_argument("--batch", type=int, default=1,
                    help="plan this many independent problems together (cem_plan_batched)")
    ap.add_argument("--warm-start", action="store_true",
                    help="each plan starts from cem_warm_start of the previous one")
    ap.add_argument("--sigma-floor", type=float, default=0.0,
                    help="with --warm-start: carried widths are kept down to this value")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timers", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the register-only MFMA ceiling measurement")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="calibration only: run a plain device copy of this many bytes 3 times "
                         "(reference for rocprofv3 FETCH_SIZE / WRITE_SIZE) and exit")
    ap.add_argument("--summarize-stats", metavar="KERNEL_STATS_CSV",
                    help="print a markdown summary of a rocprofv3 --stats CSV and exit")
    ap.add_argument("--summarize-traffic", nargs="+",
                    metavar="CSV",
                    help="print per-kernel HBM bytes from rocprofv3 --pmc CSVs: FETCH_SIZE, "
                         "WRITE_SIZE of the bench, the same of the --copy-bytes run, and "
                         "optionally the --kernel-trace --stats CSV of the bench (mean duration, "
                         "GB/s), then exit")
    ap.add_argument("--summarize-sq", metavar="COUNTER_CSV",
                    help="print per-kernel VALU / MFMA busy and wait shares from a rocprofv3 --pmc "
                         "pass over the SQ counters (see summarize_sq), then exit")
    ap.add_argument("--summarize-path", metavar="COUNTER_CSV",
                    help="print per-kernel memory-path figures from a rocprofv3 --pmc pass over the "
                         "TCP / TCC / TA / TD counters (see summarize_path) for --workload, then exit")
    args = ap.parse_args()
    if args.summarize_path:
        summarize_path(args.summarize_path, args.workload)
        return 0
    if args.summarize_sq:
        summarize_sq(args.summarize_sq)
        return 0
    if args.summarize_stats:
        summarize_stats(args.summarize_stats)
        return 0
    if args.summarize_traffic:
        if len(args.summarize_traffic) not in (4, 5):
            ap.error("--summarize-traffic takes 4 or 5 CSV paths")
        summarize_traffic(*args.summarize_traffic[:4], copy_bytes=args.copy_bytes or (1 << 30),
                          stats=(args.summarize_traffic[4:] or [None])[0])
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        eprint("bench.py measures one GPU: the plan step runs on a single MI355X, and "
               "several GPUs are not supported (--gpus must be 1).")
        return 2

    import numpy as np
    import torch

    from cem_jepa_predictor_amd import _lib, inputs

    if not torch.cuda.is_available():
        eprint("no GPU available")
        return 1
    torch.cuda.set_device(0)
    if args.copy_bytes:
        src = torch.ones(args.copy_bytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        eprint(f"[bench] copied {args.copy_bytes} bytes 3 times")
        return 0
    if args.samples:
        wl = inputs.sweep_workload(args.samples)
    else:
        wl = inputs.WORKLOADS[args.workload]
    if args.rounds:
        wl = dataclasses.replace(wl, plan=dataclasses.replace(wl.plan, rounds=args.rounds))
    m, pc = wl.model, wl.plan
    N, K, R, H, A = pc.n_samples, pc.n_elites, pc.rounds, pc.horizon, m.action_dim
    eprint(f"[bench] workload {wl.name}: N={N} K={K} R={R} H={H} L={m.layers} d={m.d_model} "
           f"dtype={m.dtype}")
    t0 = time.perf_counter()
    w = inputs.make_weights(m, wl.weight_seed)
    flat = inputs.flatten_weights(m, w)
    del w
    z_obs, z_goal, s0 = inputs.make_embeddings(m, wl.embed_seed)
    NB = max(1, args.batch)
    model = _lib.Model(m, flat, N * NB)
    del flat
    eprint(f"[bench] model ready in {time.perf_counter() - t0:.1f} s")

    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    zo, zg, st = dev(z_obs), dev(z_goal), dev(s0)
    shp = (NB, H, A) if NB > 1 else (H, A)
    mu0 = torch.full(shp, pc.mu0, device="cuda")
    sg0 = torch.full(shp, pc.sigma0, device="cuda")
    mu, sg = mu0.clone(), sg0.clone()
    action = torch.empty((NB, A) if NB > 1 else (A,), device="cuda")
    best = torch.empty(NB, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    if NB > 1:   # every problem sees the same observation and goal (timing does not depend on them)
        zo, zg, st = (t.unsqueeze(0).repeat(NB, *([1] * t.dim())).contiguous() for t in (zo, zg, st))

    def step(i: int, use_graph: bool = True):
        if args.warm_start:
            if NB > 1:
                raise SystemExit("--warm-start with --batch is not supported")
            _lib.warm_start(mu, sg, pc.mu0, pc.sigma0, args.sigma_floor, mu, sg, stream=stream)
        else:
            mu.copy_(mu0)
            sg.copy_(sg0)
        kw = dict(n_samples=N, n_elites=K, rounds=R, horizon=H, seed=pc.seed, plan_id=i * NB,
                  clamp_lo=pc.clamp_lo, clamp_hi=pc.clamp_hi, use_graph=use_graph, stream=stream)
        if NB > 1:
            model.plan_batched(zo, zg, st, mu, sg, action, best, **kw)
        else:
            model.plan(zo, zg, st, mu, sg, action, best, **kw)

    for i in range(args.warmup):
        step(i)
        torch.cuda.synchronize()
        eprint(f"[bench] warmup {i + 1}/{args.warmup} done")

    # ---- timed region: K plan steps replayed from the captured graph
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        marks[i].record(stream)
        step(1000 + i)
    marks[args.steps].record(stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = ev0.elapsed_time(ev1) / args.steps
    per_step = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)])
    p10, p50, p90 = (float(np.percentile(per_step, q)) for q in (10, 50, 90))
    eprint(f"[bench] timed {args.steps} steps: {ms:.2f} ms/step (median {p50:.2f}, p10 {p10:.2f}, "
           f"p90 {p90:.2f}; wall {wall:.2f} s)")

    # ---- kernel timers: the same K steps enqueued directly with HIP events around
    # every dense-GEMM launch, on the stream the kernels run on
    roof = None
    eager_ms = None
    if not args.no_kernel_timers:
        model.timer_enable(True)
        nt = max(1, min(args.steps, args.timer_steps))
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(nt):
            step(1000 + i, use_graph=False)
        ev1.record(stream)
        torch.cuda.synchronize()
        eager_ms = ev0.elapsed_time(ev1) / nt
        launches, gemm_ms, flop = model.timer_read()
        model.timer_enable(False)
        peak = MFMA_F32_PEAK_TFLOPS if m.dtype == "f32" else MFMA_BF16_PEAK_TFLOPS
        peak_note = None
        if m.dtype == "fp8":
            # q|k|v and MLP-up (7 of the 12 d^2 per layer, per token) run at the fp8 peak:
            # the launches' combined peak weights each kind by its FLOPs
            f8, b16 = 7.0 * m.d_model * m.d_model, 5.0 * m.d_model * m.d_model
            peak = round((f8 + b16) / (f8 / MFMA_FP8_PEAK_TFLOPS + b16 / MFMA_BF16_PEAK_TFLOPS), 1)
            peak_note = ("FLOP-weighted: q|k|v and MLP-up at the fp8 peak 5000, output and MLP-down "
                         "at the bf16 peak 2500 (frame projections ~1 % of FLOPs, counted as bf16)")
        achieved = flop / (gemm_ms * 1e-3) / 1e12
        traffic = None
        if m.dtype == "bf16" and gemm_sources_sha256() == GEMM_COUNTERS["sources_sha256"]:
            traffic = GEMM_COUNTERS["bytes_per_launch"]
        ceiling = None
        if m.dtype == "bf16" and not args.no_ceiling:
            # the part's own sustained MFMA ceiling, register-only: with changing operand
            # bits it lowers its clock to stay within its power limit
            rt, rmhz = _lib.mfma_ceiling(True, 40)
            ct, cmhz = _lib.mfma_ceiling(False, 20)
            ceiling = {"random_operands_tflops": round(rt, 1), "random_operands_mhz": round(rmhz),
                       "constant_operands_tflops": round(ct, 1), "constant_operands_mhz": round(cmhz),
                       "achieved_frac_of_random": round(achieved / rt, 4)}
            eprint(f"[bench] MFMA ceiling: {rt:.0f} TFLOP/s at {rmhz:.0f} MHz (random operands), "
                   f"{ct:.0f} TFLOP/s at {cmhz:.0f} MHz (constant operands)")
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic,
                "traffic_unit": "HBM-side bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                "copy-calibrated)",
                "kernel": "gemm_f32_kernel" if m.dtype == "f32" else "gemm_bf16_kernel",
                "launches": launches, "avg_launch_ms": round(gemm_ms / max(launches, 1), 4),
                "gemm_share_of_step": round(gemm_ms / nt / eager_ms, 4),
                "sustained_mfma_ceiling": ceiling}
        if peak_note:
            roof["peak_note"] = peak_note
        eprint(f"[bench] GEMMs: {launches} launches, {gemm_ms / nt:.2f} ms/step, "
               f"{achieved:.1f} TFLOP/s; eager step {eager_ms:.2f} ms")

    cpu = None
    if not args.no_cpu_baseline:
        eprint(f"[bench] timing the oracle on the host (~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline(wl, args.cpu_seconds)

    value = NB * N * R / (ms * 1e-3)
    pc_all = dataclasses.replace(pc, n_samples=N * NB)   # a batch rolls out NB * N candidates a round
    plan_ms_roof = plan_roofline_ms(m, pc_all, MFMA_F32_PEAK_TFLOPS if m.dtype == "f32" else MFMA_BF16_PEAK_TFLOPS)
    out = {
        "metric": "predictor candidate-evals/sec + ms per CEM plan step (800x10) on 1 MI355X",
        "value": round(value, 2), "unit": "candidate-evals/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8 e4m3 (q|k|v, MLP-up) + bf16" if m.dtype == "fp8" else m.dtype,
        "data": "synthetic: random-init weights N(0,0.02) (seed 0), N(0,1) embeddings (seed 1), "
                "CEM seed 2",
        "config": {"workload": wl.name, "n_samples": N, "n_elites": K, "rounds": R, "horizon": H,
                   "warm_start": bool(args.warm_start), "batch": NB,
                   "layers": m.layers, "d_model": m.d_model, "heads": m.heads, "d_mlp": m.d_mlp,
                   "patches": m.patches, "enc_dim": m.enc_dim, "graph_replay": True,
                   "eager_ms_per_step": round(eager_ms, 3) if eager_ms else None},
        "ms_per_step_p10": round(p10, 3), "ms_per_step_median": round(p50, 3),
        "ms_per_step_p90": round(p90, 3),
        "plan_roofline_ms": round(plan_ms_roof, 1),
        "plan_roofline_frac": round(plan_ms_roof / ms, 4),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    model.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())

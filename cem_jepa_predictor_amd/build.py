"""Build libcem_jepa.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m cem_jepa_predictor_amd.build

Every source in csrc/ is compiled for gfx950 only.  Packed-FP32 instruction
selection is disabled for all device code (-packed-fp32-ops); the sampler and
the refit are built without floating-point contraction so their float32
arithmetic rounds once per operation.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libcem_jepa.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# the measurement probe (cem_probe.h) is a library of its own
PROBE_LIB_PATH = os.path.join(PKG, "libcem_probe.so")
ARCH = "gfx950"

SOURCES = ["sampler.hip", "embed.hip", "layernorm.hip", "gemm.hip", "attention.hip",
           "energy.hip", "select_refit.hip", "model.hip", "abi.hip"]
PROBE_SOURCES = ["probe.hip"]
NO_CONTRACT = {"sampler.hip", "select_refit.hip"}
# attention keeps its MFMA accumulators in VGPRs: its softmax rescales them with VALU ops
EXTRA = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _flags(src: str):
    f = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-x", "hip",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]
    if src in NO_CONTRACT:
        f.append("-ffp-contract=off")
    f += EXTRA.get(src, [])
    return f


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
    cmd = [hipcc()] + _flags(src) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, path: str) -> None:
    tmp = path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = True, jobs: int = 8) -> str:
    """Compile every source and link the plan library and the probe library;
    returns the plan library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB_PATH)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} and {PROBE_LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build()
    sys.exit(0)

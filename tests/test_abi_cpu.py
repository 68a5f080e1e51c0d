"""The C-ABI library loads, exports what include/cem_jepa.h declares, and
rejects bad arguments on the host before any device work (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from cem_jepa_predictor_amd import _lib, inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cem_jepa.h")
PROBE_HEADER = os.path.join(ROOT, "include", "cem_probe.h")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libcem_jepa.so is not built (python -m cem_jepa_predictor_amd.build)")
    return _lib.load()


def test_header_declares_the_boundary():
    fns = declared_functions()
    for name in ["cem_plan", "predictor_rollout", "energy_l1", "elite_refit", "cem_model_create",
                 "cem_model_destroy", "cem_last_error", "cem_sample", "topk_select"]:
        assert name in fns
    assert set(fns) == set(_lib.EXPORTS)


def _exported(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True,
                         text=True, check=True).stdout
    return {line.split()[-1] for line in out.splitlines() if " T " in line}


def test_library_exports_every_declared_symbol(lib):
    exported = _exported(_lib.LIB_PATH)
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_probe_library_exports_its_header_and_the_plan_library_none_of_it(lib):
    probe = _lib.load_probe()
    fns = declared_functions(PROBE_HEADER)
    assert set(fns) == set(_lib.PROBE_EXPORTS)
    exported = _exported(_lib.PROBE_LIB_PATH)
    for name in fns:
        assert name in exported, name
        assert hasattr(probe, name)
    assert not set(fns) & _exported(_lib.LIB_PATH)


def test_weights_count_matches_canonical_layout(lib):
    for name in ["tiny", "small", "vjepa2ac", "vjepa2ac_h4", "small_fp8"]:
        m = inputs.WORKLOADS[name].model
        desc = _lib.model_desc(m, 8)
        assert _lib.weights_count(desc) == inputs.weight_count(m)


@pytest.mark.parametrize("field,value,status", [
    ("d_model", 100, -2), ("heads", 3, -2), ("d_mlp", 100, -2), ("enc_dim", 30, -2),
    ("max_horizon", 9, -2), ("max_samples", 0, -2), ("max_samples", 20000, -2), ("dtype", 7, -3),
    ("layers", 0, -2), ("patches", 0, -2), ("ln_eps", 0.0, -1), ("action_dim", 0, -2),
])
def test_model_desc_validation(lib, field, value, status):
    m = inputs.WORKLOADS["tiny"].model
    desc = _lib.model_desc(m, 8)
    setattr(desc, field, value)
    n = ctypes.c_size_t(0)
    assert lib.cem_weights_count(ctypes.byref(desc), ctypes.byref(n)) == status
    assert lib.cem_last_error().decode() != ""


def test_bf16_gemm_takes_one_slab_contractions(lib):
    """The bf16 GEMM's operand ring runs across tiles for any number of 64-wide
    K-slabs, so bf16 models with a 64-wide MLP or encoder are accepted."""
    m = inputs.WORKLOADS["small"].model
    n = ctypes.c_size_t(0)
    for field in ("d_mlp", "enc_dim"):
        desc = _lib.model_desc(m, 8)
        setattr(desc, field, 64)
        assert lib.cem_weights_count(ctypes.byref(desc), ctypes.byref(n)) == 0
        setattr(desc, field, 96)   # not a whole number of slabs
        assert lib.cem_weights_count(ctypes.byref(desc), ctypes.byref(n)) == -2


def test_bf16_attention_shape_limits(lib):
    m = inputs.WORKLOADS["small"].model
    desc = _lib.model_desc(m, 8)
    desc.heads = 4   # head dim 128: the bf16 attention kernel takes 64
    n = ctypes.c_size_t(0)
    assert lib.cem_weights_count(ctypes.byref(desc), ctypes.byref(n)) == -2
    desc = _lib.model_desc(m, 8)
    desc.patches = 400   # 402 tokens per block exceeds the per-wave query tiles
    assert lib.cem_weights_count(ctypes.byref(desc), ctypes.byref(n)) == -2


def test_create_rejects_wrong_weight_count_and_nonfinite(lib):
    m = inputs.WORKLOADS["tiny"].model
    desc = _lib.model_desc(m, 8)
    w = np.zeros(inputs.weight_count(m) - 1, np.float32)
    h = ctypes.c_void_p()
    assert lib.cem_model_create(ctypes.byref(desc), w.ctypes.data, w.size, 0, ctypes.byref(h)) == -2
    w = np.zeros(inputs.weight_count(m), np.float32)
    w[5] = np.nan
    assert lib.cem_model_create(ctypes.byref(desc), w.ctypes.data, w.size, 0, ctypes.byref(h)) == -1
    assert "non-finite" in lib.cem_last_error().decode()
    assert lib.cem_model_create(None, w.ctypes.data, w.size, 0, ctypes.byref(h)) == -1


def test_model_free_calls_validate_before_launch(lib):
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    assert lib.energy_l1(None, 0, fake, 1, 1, 1, fake, None) == -1
    assert lib.energy_l1(fake, 5, fake, 1, 1, 1, fake, None) == -3
    assert lib.energy_l1(fake, 0, fake, -1, 1, 1, fake, None) == -2
    assert lib.elite_refit(fake, fake, 10, 11, 1, 7, fake, fake, fake, None) == -2
    assert lib.elite_refit(fake, fake, 20000, 10, 1, 7, fake, fake, fake, None) == -2
    assert lib.elite_refit(fake, fake, 10, 0, 1, 7, fake, fake, fake, None) == -2
    assert lib.topk_select(fake, 0, 1, fake, None) == -2
    assert lib.cem_sample(fake, fake, 4, 1, 7, 0, 0, 0, 1.0, -1.0, fake, None, None) == -1
    assert lib.cem_sample(fake, fake, 4, 1, 7, 0, 0, 0, float("nan"), 1.0, fake, None, None) == -1
    assert lib.energy_l1(ctypes.c_void_p(0x1001), 0, fake, 1, 1, 1, fake, None) == -1   # misaligned


def test_plan_calls_validate_null_model(lib):
    p = _lib.Params(8, 2, 1, 1, -1.0, 1.0, 0, 0, 1)
    fake = ctypes.c_void_p(0x1000)
    assert lib.cem_plan(None, ctypes.byref(p), fake, fake, fake, fake, fake, fake, None, None) == -1
    assert lib.predictor_rollout(None, fake, 1, 1, fake, fake, fake, None) == -1
    assert lib.cem_plan_trace(None, 0, fake, 4, None) == -1
    assert lib.cem_timer_enable(None, 1) == -1


def test_mfma_ceiling_validates_before_launch(lib):
    probe = _lib.load_probe()
    tf, mhz = ctypes.c_double(), ctypes.c_double()
    assert probe.cem_mfma_ceiling(1, 1, ctypes.byref(tf), ctypes.byref(mhz)) == -1
    assert probe.cem_mfma_ceiling(2, 10, ctypes.byref(tf), ctypes.byref(mhz)) == -1
    assert probe.cem_mfma_ceiling(1, 10, None, ctypes.byref(mhz)) == -1


def test_binding_rejects_bad_tensors_before_the_library():
    """dtype, shape, device and layout are checked in the binding, before any pointer
    crosses the ABI (a float64 goal read as float32 would give garbage energies)."""
    import torch

    zp = torch.zeros((2, 3, 8), dtype=torch.bfloat16)
    out = torch.zeros(2, dtype=torch.float32)
    with pytest.raises(TypeError, match="z_goal: dtype torch.float64"):
        _lib.energy_l1(zp, torch.zeros((3, 8), dtype=torch.float64), out)
    with pytest.raises(ValueError, match=r"z_goal: shape \(8, 3\)"):
        _lib.energy_l1(zp, torch.zeros((8, 3), dtype=torch.float32), out)
    with pytest.raises(ValueError, match="must be a device"):
        _lib.energy_l1(zp, torch.zeros((3, 8), dtype=torch.float32), out)
    with pytest.raises(TypeError, match="idx: dtype torch.int64"):
        _lib.topk_select(torch.zeros(4), 2, torch.zeros(2, dtype=torch.int64))
    with pytest.raises(TypeError, match="out: dtype torch.float32"):
        _lib.Model.trace(None, _lib.TRACE_ELITES, torch.zeros(4))


def test_warm_start_validates_before_launch(lib):
    fake = ctypes.c_void_p(0x1000)
    assert lib.cem_warm_start(None, fake, 2, 7, 0.0, 1.0, 0.0, fake, fake, None) == -1
    assert lib.cem_warm_start(fake, fake, 0, 7, 0.0, 1.0, 0.0, fake, fake, None) == -2
    assert lib.cem_warm_start(fake, fake, 200, 7, 0.0, 1.0, 0.0, fake, fake, None) == -2
    assert lib.cem_warm_start(fake, fake, 2, 7, 0.0, 0.0, 0.0, fake, fake, None) == -1
    assert lib.cem_warm_start(fake, fake, 2, 7, 0.0, 1.0, -0.5, fake, fake, None) == -1
    assert lib.cem_warm_start(fake, fake, 2, 7, float("inf"), 1.0, 0.0, fake, fake, None) == -1
    assert lib.cem_warm_start(fake, ctypes.c_void_p(0x1002), 2, 7, 0.0, 1.0, 0.0, fake, fake, None) == -1


def test_plan_batched_validates_null_model(lib):
    p = _lib.Params(8, 2, 1, 1, -1.0, 1.0, 0, 0, 1)
    fake = ctypes.c_void_p(0x1000)
    assert lib.cem_plan_batched(None, ctypes.byref(p), 2, fake, fake, fake, fake, fake, fake, None,
                                None) == -1



def test_fp8_models_need_d_model_multiple_of_512(lib):
    n = ctypes.c_size_t(0)
    desc = _lib.model_desc(inputs.WORKLOADS["small_fp8"].model, 8)
    assert lib.cem_weights_count(ctypes.byref(desc), ctypes.byref(n)) == 0
    desc = _lib.model_desc(inputs.WORKLOADS["oddk"].model, 8)
    desc.dtype = 2
    assert lib.cem_weights_count(ctypes.byref(desc), ctypes.byref(n)) == -2
    assert "512" in lib.cem_last_error().decode()
    fake = ctypes.c_void_p(0x1000)
    assert lib.cem_fp8_quantize_rows(fake, 4, 12, fake, fake, None) == -2
    assert lib.cem_fp8_quantize_rows(None, 4, 16, fake, fake, None) == -1


def test_binding_structs_match_the_header_layout(tmp_path):
    """The ctypes mirrors of cem_params and cem_model_desc have the size and field
    offsets the C compiler gives the header's structs."""
    structs = {"cem_params": _lib.Params, "cem_model_desc": _lib.ModelDesc}
    lines = ['#include "cem_jepa.h"', "#include <stddef.h>", "#include <stdio.h>", "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for field, _ in py._fields_:
            lines.append(f'  printf("{cname} {field} %zu\\n", offsetof({cname}, {field}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    got = {}
    for line in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.splitlines():
        cname, field, value = line.split()
        got[(cname, field)] = int(value)
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for field, _ in py._fields_:
            assert got[(cname, field)] == getattr(py, field).offset, (cname, field)

"""ctypes binding of libcem_jepa.so: argument marshalling only.

Every function here forwards torch tensors' device pointers and the current
HIP stream to the C ABI declared in include/cem_jepa.h; all computation runs
in the library's HIP kernels.  There is no fallback: if the library is not
built, load() raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

from .inputs import ModelConfig

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcem_jepa.so")
PROBE_LIB_PATH = os.path.join(_PKG, "libcem_probe.so")   # measurement only (cem_probe.h)

CEM_F32, CEM_BF16, CEM_FP8 = 0, 1, 2
_MODEL_DTYPES = {"f32": CEM_F32, "bf16": CEM_BF16, "fp8": CEM_FP8}
TRACE_ACTIONS, TRACE_ENERGY, TRACE_ELITES, TRACE_MU, TRACE_SIGMA = range(5)
STATUS_NAMES = {0: "CEM_OK", -1: "CEM_E_ARG", -2: "CEM_E_SHAPE", -3: "CEM_E_DTYPE",
                -4: "CEM_E_OOM", -5: "CEM_E_HIP", -6: "CEM_E_INTERNAL"}

EXPORTS = ["cem_last_error", "cem_weights_count", "cem_model_create", "cem_model_destroy",
           "cem_plan", "cem_plan_batched", "cem_plan_noalloc", "cem_plan_trace", "predictor_rollout", "energy_l1", "elite_refit",
           "cem_sample", "topk_select", "cem_warm_start", "cem_fp8_quantize_rows", "cem_timer_enable", "cem_timer_read"]
PROBE_EXPORTS = ["cem_mfma_ceiling"]


class CemError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class ModelDesc(ctypes.Structure):
    _fields_ = [("layers", ctypes.c_int32), ("d_model", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("d_mlp", ctypes.c_int32), ("patches", ctypes.c_int32), ("enc_dim", ctypes.c_int32),
                ("action_dim", ctypes.c_int32), ("state_dim", ctypes.c_int32),
                ("max_horizon", ctypes.c_int32), ("max_samples", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("ln_eps", ctypes.c_float)]


class Params(ctypes.Structure):
    _fields_ = [("n_samples", ctypes.c_int32), ("n_elites", ctypes.c_int32),
                ("rounds", ctypes.c_int32), ("horizon", ctypes.c_int32),
                ("clamp_lo", ctypes.c_float), ("clamp_hi", ctypes.c_float),
                ("seed", ctypes.c_uint64), ("plan_id", ctypes.c_uint32),
                ("use_graph", ctypes.c_int32), ("first_round", ctypes.c_uint32)]


_lib: Optional[ctypes.CDLL] = None
P = ctypes.c_void_p
I32, U32, U64, F32, SZ = ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_float, ctypes.c_size_t


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m cem_jepa_predictor_amd.build`")
    # torch ships its own HIP runtime; importing it first makes the library bind to
    # that same runtime (same SONAME), so both share one device context and streams.
    import torch  # noqa: F401

    lib = ctypes.CDLL(path)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise RuntimeError("two HIP runtimes are mapped in this process (" + ", ".join(runtimes)
                           + "): import torch before anything that loads libamdhip64")
    lib.cem_last_error.restype = ctypes.c_char_p
    lib.cem_last_error.argtypes = []
    sigs = {
        "cem_weights_count": [ctypes.POINTER(ModelDesc), ctypes.POINTER(SZ)],
        "cem_model_create": [ctypes.POINTER(ModelDesc), P, SZ, I32, ctypes.POINTER(P)],
        "cem_model_destroy": [P],
        "cem_plan": [P, ctypes.POINTER(Params), P, P, P, P, P, P, P, P],
        "cem_plan_batched": [P, ctypes.POINTER(Params), I32, P, P, P, P, P, P, P, P],
        "cem_plan_noalloc": [P, ctypes.POINTER(Params), P, P, P, P, P, P, P, P],
        "cem_plan_trace": [P, I32, P, SZ, P],
        "predictor_rollout": [P, P, I32, I32, P, P, P, P],
        "energy_l1": [P, I32, P, I32, I32, I32, P, P],
        "elite_refit": [P, P, I32, I32, I32, I32, P, P, P, P],
        "cem_sample": [P, P, I32, I32, I32, U64, U32, U32, F32, F32, P, P, P],
        "topk_select": [P, I32, I32, P, P],
        "cem_warm_start": [P, P, I32, I32, F32, F32, F32, P, P, P],
        "cem_fp8_quantize_rows": [P, I32, I32, P, P, P],
        "cem_timer_enable": [P, I32],
        "cem_timer_read": [P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double),
                           ctypes.POINTER(ctypes.c_double)],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    _lib = lib
    return lib


def _hip_runtimes_mapped():
    """Distinct libamdhip64 files mapped into this process (Linux /proc)."""
    try:
        with open("/proc/self/maps") as f:
            paths = {line.split()[-1] for line in f if "libamdhip64.so" in line}
    except OSError:
        return []
    return sorted({os.path.realpath(p) for p in paths})


def _check(status: int) -> None:
    if status != 0:
        raise CemError(status, load().cem_last_error().decode())


def _args(*specs):
    """Device pointers of tensor arguments after checking what the C ABI assumes of
    them; raises before any library call.  Each spec is (tensor, name, dtypes[, shape
    [, optional]]).  dtype and shape of every argument are checked before device
    residency and contiguity, so a wrong dtype is reported as such even for host
    tensors."""
    import torch

    full = [tuple(sp) + (None, False)[len(sp) - 3:] for sp in specs]
    for t, name, dtypes, shape, optional in full:
        if t is None:
            if optional:
                continue
            raise ValueError(f"{name} is required")
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
        if t.dtype not in dtypes:
            raise TypeError(f"{name}: dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    ptrs = []
    for t, name, _, _, _ in full:
        if t is None:
            ptrs.append(None)
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device (cuda) tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        ptrs.append(t.data_ptr())
    return ptrs


def _f32():
    import torch
    return (torch.float32,)


def _i32():
    import torch
    return (torch.int32,)


_side_streams = {}


class _OnStream:
    """Run library calls on an explicit HIP stream ordered with torch's work.

    An explicit torch stream with a real handle is used as is.  torch's default
    stream reports handle 0, which the library would read as HIP's legacy null
    stream -- not necessarily the stream torch launched its own kernels on.  So
    library calls then go to a torch-created side stream that first waits for
    torch's current stream, and torch's current stream waits for it afterwards.
    """

    def __init__(self, stream):
        import torch

        self.cur = stream if stream is not None else torch.cuda.current_stream()
        self.side = None
        if self.cur.cuda_stream == 0:
            dev = self.cur.device
            key = dev.index if dev.index is not None else torch.cuda.current_device()
            if key not in _side_streams:
                _side_streams[key] = torch.cuda.Stream(device=key)
            self.side = _side_streams[key]

    def __enter__(self) -> int:
        if self.side is None:
            return self.cur.cuda_stream
        self.side.wait_stream(self.cur)
        return self.side.cuda_stream

    def __exit__(self, *exc):
        if self.side is not None:
            self.cur.wait_stream(self.side)
        return False


def model_desc(m: ModelConfig, max_samples: int, max_horizon: Optional[int] = None) -> ModelDesc:
    return ModelDesc(m.layers, m.d_model, m.heads, m.d_mlp, m.patches, m.enc_dim, m.action_dim,
                     m.state_dim, max_horizon or m.max_horizon, max_samples,
                     _MODEL_DTYPES[m.dtype], m.ln_eps)


def weights_count(desc: ModelDesc) -> int:
    n = SZ(0)
    _check(load().cem_weights_count(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


class Model:
    """A model handle on one device (cem_model_create / cem_model_destroy)."""

    def __init__(self, cfg: ModelConfig, flat_weights: np.ndarray, max_samples: int,
                 device: int = 0, max_horizon: Optional[int] = None):
        lib = load()
        self.cfg = cfg
        self.desc = model_desc(cfg, max_samples, max_horizon)
        w = np.ascontiguousarray(flat_weights, dtype=np.float32)
        h = P()
        _check(lib.cem_model_create(ctypes.byref(self.desc), w.ctypes.data, w.size, device,
                                    ctypes.byref(h)))
        self.handle = h
        self._last = None

    def close(self) -> None:
        if self.handle:
            _check(load().cem_model_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def plan(self, z_obs, z_goal, s0, mu, sigma, action, best_idx=None, *, n_samples: int,
             n_elites: int, rounds: int, horizon: int, seed: int, plan_id: int = 0,
             clamp_lo: float = -1.0, clamp_hi: float = 1.0, use_graph: bool = True, stream=None,
             noalloc: bool = False, first_round: int = 0):
        """cem_plan (or, with noalloc, cem_plan_noalloc: the plan state in the library's
        per-device scratch, nothing allocated, kernels enqueued directly, the model's
        trace untouched).  first_round > 0 resumes a plan after that many rounds from
        the mu and sigma it returned."""
        c = self.cfg
        pe, ha = (c.patches, c.enc_dim), (horizon, c.action_dim)
        ptrs = _args((z_obs, "z_obs", _f32(), pe), (z_goal, "z_goal", _f32(), pe),
                     (s0, "s0", _f32(), (c.state_dim,)), (mu, "mu", _f32(), ha),
                     (sigma, "sigma", _f32(), ha), (action, "action", _f32(), (c.action_dim,)),
                     (best_idx, "best_idx", _i32(), (1,), True))
        p = Params(n_samples, n_elites, rounds, horizon, clamp_lo, clamp_hi, seed, plan_id,
                   1 if use_graph else 0, first_round)
        with _OnStream(stream) as st:
            if noalloc:
                _check(load().cem_plan_noalloc(self.handle, ctypes.byref(p), *ptrs, st))
            else:
                _check(load().cem_plan(self.handle, ctypes.byref(p), *ptrs, st))
                self._last = p

    def plan_batched(self, z_obs, z_goal, s0, mu, sigma, action, best_idx=None, *, n_samples: int,
                     n_elites: int, rounds: int, horizon: int, seed: int, plan_id: int = 0,
                     clamp_lo: float = -1.0, clamp_hi: float = 1.0, use_graph: bool = True,
                     stream=None, first_round: int = 0):
        """cem_plan_batched: z_obs/z_goal [b, P, E], s0 [b, S], mu/sigma [b, H, A],
        action [b, A], best_idx [b]; problem i plans with plan id plan_id + i."""
        c = self.cfg
        if z_obs.dim() != 3:
            raise ValueError(f"z_obs: expected [batch, P, E], got {tuple(z_obs.shape)}")
        b = z_obs.shape[0]
        pe, ha = (b, c.patches, c.enc_dim), (b, horizon, c.action_dim)
        ptrs = _args((z_obs, "z_obs", _f32(), pe), (z_goal, "z_goal", _f32(), pe),
                     (s0, "s0", _f32(), (b, c.state_dim)), (mu, "mu", _f32(), ha),
                     (sigma, "sigma", _f32(), ha), (action, "action", _f32(), (b, c.action_dim)),
                     (best_idx, "best_idx", _i32(), (b,), True))
        p = Params(n_samples, n_elites, rounds, horizon, clamp_lo, clamp_hi, seed, plan_id,
                   1 if use_graph else 0, first_round)
        with _OnStream(stream) as st:
            _check(load().cem_plan_batched(self.handle, ctypes.byref(p), b, *ptrs, st))
        self._last = p

    def trace(self, kind: int, out, stream=None):
        """Copies one per-round record of the last plan into `out` (int32 for the
        elite indices, float32 otherwise; the library checks the byte size)."""
        ptr, = _args((out, "out", _i32() if kind == TRACE_ELITES else _f32()))
        with _OnStream(stream) as st:
            _check(load().cem_plan_trace(self.handle, kind, ptr, out.numel() * out.element_size(), st))
        return out

    def rollout(self, actions, z_obs, s0, z_pred, stream=None):
        import torch

        c = self.cfg
        if actions.dim() != 3:
            raise ValueError(f"actions: expected [n, h, {c.action_dim}], got {tuple(actions.shape)}")
        n, h = actions.shape[0], actions.shape[1]
        zdt = torch.float32 if c.dtype == "f32" else torch.bfloat16
        ptrs = _args((actions, "actions", _f32(), (n, h, c.action_dim)),
                     (z_obs, "z_obs", _f32(), (c.patches, c.enc_dim)),
                     (s0, "s0", _f32(), (c.state_dim,)),
                     (z_pred, "z_pred", (zdt,), (n, c.patches, c.enc_dim)))
        with _OnStream(stream) as st:
            _check(load().predictor_rollout(self.handle, ptrs[0], n, h, ptrs[1], ptrs[2], ptrs[3], st))
        return z_pred

    def timer_enable(self, on: bool = True):
        _check(load().cem_timer_enable(self.handle, 1 if on else 0))

    def timer_read(self):
        n, ms, fl = ctypes.c_int64(0), ctypes.c_double(0), ctypes.c_double(0)
        _check(load().cem_timer_read(self.handle, ctypes.byref(n), ctypes.byref(ms), ctypes.byref(fl)))
        return n.value, ms.value, fl.value


def energy_l1(z_pred, z_goal, energy, stream=None):
    import torch

    if z_pred.dim() != 3:
        raise ValueError(f"z_pred: expected [n, p, e], got {tuple(z_pred.shape)}")
    n, p, e = z_pred.shape
    zp, zg, en = _args((z_pred, "z_pred", (torch.bfloat16, torch.float32)),
                       (z_goal, "z_goal", _f32(), (p, e)), (energy, "energy", _f32(), (n,)))
    dt = CEM_BF16 if z_pred.dtype == torch.bfloat16 else CEM_F32
    with _OnStream(stream) as st:
        _check(load().energy_l1(zp, dt, zg, n, p, e, en, st))
    return energy


def elite_refit(energy, actions, k, elite_idx, mu, sigma, stream=None):
    if actions.dim() != 3:
        raise ValueError(f"actions: expected [n, h, a], got {tuple(actions.shape)}")
    n, h, a = actions.shape
    ptrs = _args((energy, "energy", _f32(), (n,)), (actions, "actions", _f32()),
                 (elite_idx, "elite_idx", _i32(), (k,)), (mu, "mu", _f32(), (h, a)),
                 (sigma, "sigma", _f32(), (h, a)))
    with _OnStream(stream) as st:
        _check(load().elite_refit(ptrs[0], ptrs[1], n, k, h, a, ptrs[2], ptrs[3], ptrs[4], st))


def cem_sample(mu, sigma, n, seed, rnd, plan_id, lo, hi, actions, raw_words=None, stream=None):
    import torch

    if mu.dim() != 2:
        raise ValueError(f"mu: expected [h, a], got {tuple(mu.shape)}")
    h, a = mu.shape
    if actions.dim() != 3 or tuple(actions.shape[1:]) != (h, a) or actions.shape[0] < n:
        raise ValueError(f"actions: shape {tuple(actions.shape)}, expected [>= {n}, {h}, {a}]")
    if raw_words is not None and raw_words.numel() < n * h * a:
        raise ValueError(f"raw_words: {raw_words.numel()} elements, need {n * h * a}")
    mp, sp, xp, raw = _args((mu, "mu", _f32()), (sigma, "sigma", _f32(), (h, a)),
                            (actions, "actions", _f32()),
                            (raw_words, "raw_words", (torch.int32, torch.uint32), None, True))
    ptrs = (mp, sp, xp)
    with _OnStream(stream) as st:
        _check(load().cem_sample(ptrs[0], ptrs[1], n, h, a, seed, rnd, plan_id, lo, hi, ptrs[2], raw,
                                 st))


def topk_select(energy, k, idx, stream=None):
    if energy.dim() != 1:
        raise ValueError(f"energy: expected 1-d, got {tuple(energy.shape)}")
    ptrs = _args((energy, "energy", _f32()), (idx, "idx", _i32(), (k,)))
    with _OnStream(stream) as st:
        _check(load().topk_select(ptrs[0], energy.numel(), k, ptrs[1], st))


def warm_start(mu_prev, sigma_prev, mu_fill, sigma_fill, sigma_floor, mu_next, sigma_next,
               stream=None):
    """Seeds the next control step's Gaussian from a plan's final one
    (cem_warm_start); outputs may be the inputs."""
    if mu_prev.dim() != 2:
        raise ValueError(f"mu_prev: expected [h, a], got {tuple(mu_prev.shape)}")
    h, a = mu_prev.shape
    ptrs = _args((mu_prev, "mu_prev", _f32()), (sigma_prev, "sigma_prev", _f32(), (h, a)),
                 (mu_next, "mu_next", _f32(), (h, a)), (sigma_next, "sigma_next", _f32(), (h, a)))
    with _OnStream(stream) as st:
        _check(load().cem_warm_start(ptrs[0], ptrs[1], h, a, mu_fill, sigma_fill, sigma_floor,
                                     ptrs[2], ptrs[3], st))


def fp8_quantize_rows(x, codes, scale, stream=None):
    """Per-row OCP e4m3 quantization of fp32 rows (cem_fp8_quantize_rows)."""
    import torch

    if x.dim() != 2:
        raise ValueError(f"x: expected [rows, cols], got {tuple(x.shape)}")
    r, c = x.shape
    ptrs = _args((x, "x", _f32()), (codes, "codes", (torch.uint8,), (r, c)), (scale, "scale", _f32(), (r,)))
    with _OnStream(stream) as st:
        _check(load().cem_fp8_quantize_rows(ptrs[0], r, c, ptrs[1], ptrs[2], st))


_probe: Optional[ctypes.CDLL] = None


def load_probe(path: str = PROBE_LIB_PATH) -> ctypes.CDLL:
    """The measurement probe library (raises if it has not been built)."""
    global _probe
    if _probe is not None:
        return _probe
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m cem_jepa_predictor_amd.build`")
    load()   # same HIP runtime as the plan library (torch's)
    lib = ctypes.CDLL(path)
    lib.cem_mfma_ceiling.argtypes = [I32, I32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    lib.cem_mfma_ceiling.restype = ctypes.c_int
    _probe = lib
    return lib


def mfma_ceiling(random_operands: bool = True, launches: int = 40):
    """Sustained dense bf16 MFMA TFLOP/s and shader clock (MHz) of the current
    device, register-only (cem_mfma_ceiling in the probe library); synchronous."""
    tf, mhz = ctypes.c_double(), ctypes.c_double()
    st = load_probe().cem_mfma_ceiling(1 if random_operands else 0, int(launches), ctypes.byref(tf),
                                       ctypes.byref(mhz))
    if st != 0:
        raise CemError(st, "cem_mfma_ceiling failed (arguments or HIP runtime)")
    return tf.value, mhz.value

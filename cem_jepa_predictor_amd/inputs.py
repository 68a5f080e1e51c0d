"""Seeded synthetic inputs shared by the HIP path, the oracle and the benchmark.

This module holds data only: the workload shapes and the seeded generators that
draw weights and embeddings for them. It contains none of the planning
method's arithmetic, and it imports neither the HIP binding nor the oracle.

Workload shapes follow the CEM plan step described on the page "Real-Time
Inference for JEPA World Model Architectures with Ray" (section 01, "Where the
sixteen seconds actually goes": 800 candidates, best 80 kept, ten rounds) and
the predictor sizes of the V-JEPA2-AC-shaped predictor used there (24 layers,
width 1024, 16 heads, MLP 4096, 256 patch tokens, encoder width 1408, 7-D
actions and states).

Random-init recipe (the pages ship no weights):
  * every Linear weight and bias ~ N(0, 0.02^2);
  * LayerNorm gain = 1 + N(0, 0.02^2), LayerNorm shift ~ N(0, 0.02^2);
  * observation and goal embeddings ~ N(0, 1), shape [P, E]; s0 ~ N(0, 1), [S];
  * tensors drawn from numpy PCG64(seed) in the canonical order below;
  * for bf16 models every parameter is rounded to the nearest bf16 value
    (ties to even) and kept as float32, so both sides see the same model.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple

import numpy as np

ACTION_DIM = 7
STATE_DIM = 7


@dataclasses.dataclass(frozen=True)
class ModelConfig:
    """Shape of the action-conditioned predictor."""

    name: str
    layers: int
    d_model: int
    heads: int
    d_mlp: int
    patches: int          # P, patch tokens per frame block
    enc_dim: int          # E, encoder embedding width (projected in and out)
    dtype: str            # "f32", "bf16", or "fp8" (bf16 with e4m3 LayerNorm-fed projections)
    max_horizon: int
    action_dim: int = ACTION_DIM
    state_dim: int = STATE_DIM
    ln_eps: float = 1e-5

    @property
    def head_dim(self) -> int:
        return self.d_model // self.heads

    @property
    def block_tokens(self) -> int:
        """B = P + 2: one action token, one state token, P frame tokens."""
        return self.patches + 2


@dataclasses.dataclass(frozen=True)
class PlanConfig:
    """CEM search settings."""

    n_samples: int
    n_elites: int
    rounds: int
    horizon: int
    clamp_lo: float = -1.0
    clamp_hi: float = 1.0
    mu0: float = 0.0
    sigma0: float = 1.0
    seed: int = 2
    plan_id: int = 0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    model: ModelConfig
    plan: PlanConfig
    weight_seed: int = 0
    embed_seed: int = 1


def _vj(name: str, horizon: int, max_horizon: int) -> ModelConfig:
    return ModelConfig(name=name, layers=24, d_model=1024, heads=16, d_mlp=4096,
                       patches=256, enc_dim=1408, dtype="bf16", max_horizon=max_horizon)


WORKLOADS: Dict[str, Workload] = {
    # Tiny fp32 case that the oracle finishes in seconds.
    "tiny": Workload("tiny", ModelConfig("tiny", 2, 128, 4, 512, 16, 128, "f32", 2),
                     PlanConfig(64, 8, 3, 2)),
    # Small bf16 case with a 3-step autoregressive rollout (KV cache).
    "small": Workload("small", ModelConfig("small", 6, 512, 8, 2048, 64, 512, "bf16", 3),
                      PlanConfig(256, 32, 5, 3)),
    # Small bf16 case with odd and single K-slab counts (64-wide slabs: d_mlp 320
    # -> 5, d_model 128 -> 2, enc_dim 64 -> 1) and ragged or split-straddling
    # output tiles in every projection.
    "oddk": Workload("oddk", ModelConfig("oddk", 2, 128, 2, 320, 16, 64, "bf16", 2),
                     PlanConfig(16, 4, 2, 2)),
    # The small case with the fp8 (e4m3) q|k|v and MLP-up projections.
    "small_fp8": Workload("small_fp8", ModelConfig("small_fp8", 6, 512, 8, 2048, 64, 512, "fp8", 3),
                          PlanConfig(256, 32, 5, 3)),
    # One layer of the small shape with the fp8 projections, horizon 1: shallow
    # enough that the e4m3 quantization, not the bf16 activation rounding, sets the
    # difference from the plain model.
    "shallow_fp8": Workload("shallow_fp8", ModelConfig("shallow_fp8", 1, 512, 8, 2048, 64, 512, "fp8", 1),
                            PlanConfig(16, 4, 2, 1)),
    # bf16 at d_model 768 (12 heads): three 256-column output tiles per residual
    # GEMM, so the LayerNorm statistics come in 12 pieces of 64 columns per row.
    "wide768": Workload("wide768", ModelConfig("wide768", 2, 768, 12, 3072, 16, 128, "bf16", 2),
                        PlanConfig(32, 4, 2, 2)),
    # One bf16 layer at d_model 2048 (32 heads): the MLP-up LayerNorm's statistics
    # from the output projection's epilogue in 32 pieces per row.
    "wide2048": Workload("wide2048", ModelConfig("wide2048", 1, 2048, 32, 2048, 16, 64, "bf16", 1),
                         PlanConfig(16, 4, 2, 1)),
    # The V-JEPA2-AC frame-block length (256 patches, B = 258: 17 query tiles, the last
    # holding 2 rows) on a two-layer, two-head model the oracle runs in seconds, with up
    # to 320 candidates: the attention at that block length in both of its input modes
    # (layer 0 reads the compact layer-0 block, layer 1 the full rows).
    "p256": Workload("p256", ModelConfig("p256", 2, 128, 2, 256, 256, 128, "bf16", 1),
                     PlanConfig(320, 32, 2, 1)),
    # 140 patches (B = 142: 9 query tiles over the attention workgroup's eight waves, the
    # ninth holding 14 rows), horizon 2 so the second frame block runs the cached-keys
    # kernel at that length too.
    "p140": Workload("p140", ModelConfig("p140", 2, 128, 2, 256, 140, 128, "bf16", 2),
                     PlanConfig(64, 8, 2, 2)),
    # One bf16 layer at the widest d_model the library takes (4096, 64 heads): statistics
    # in 64 pieces per row, K = 4096 in every projection.
    "wide4096": Workload("wide4096", ModelConfig("wide4096", 1, 4096, 64, 4096, 16, 64, "bf16", 1),
                         PlanConfig(16, 4, 2, 1)),
    # The longest frame block the bf16 attention takes: 318 patches, B = 320 (20 query and
    # key tiles, K and V of a block filling half of a CU's LDS), horizon 2.
    "p318": Workload("p318", ModelConfig("p318", 2, 128, 2, 256, 318, 128, "bf16", 2),
                     PlanConfig(64, 8, 2, 2)),
    # V-JEPA2-AC-shaped predictor, horizon 1: the measured plan step.
    "vjepa2ac": Workload("vjepa2ac", _vj("vjepa2ac", 1, 1), PlanConfig(800, 80, 10, 1)),
    # Same predictor and search with the fp8 (e4m3) q|k|v and MLP-up projections.
    "vjepa2ac_fp8": Workload("vjepa2ac_fp8", dataclasses.replace(_vj("vjepa2ac_fp8", 1, 1), dtype="fp8"),
                             PlanConfig(800, 80, 10, 1)),
    # Same predictor, horizon 4 with a KV cache across frame blocks.
    "vjepa2ac_h4": Workload("vjepa2ac_h4", _vj("vjepa2ac_h4", 4, 4), PlanConfig(800, 80, 10, 4)),
}

SWEEP_SAMPLES = (200, 400, 800, 1600, 3200)


def sweep_workload(n: int) -> Workload:
    """Batch-sweep point on the V-JEPA2-AC-shaped predictor (horizon 1, K = N/10)."""
    return Workload(f"sweep_{n}", _vj(f"sweep_{n}", 1, 1), PlanConfig(n, n // 10, 10, 1))


def weight_layout(m: ModelConfig) -> List[Tuple[str, Tuple[int, ...]]]:
    """Canonical parameter order of the flat weight buffer.

    Matrices are stored [in, out] (row-major), so a layer computes x @ W + b.
    W_qkv's columns are [q | k | v], each d wide; head h owns columns
    h*dh .. (h+1)*dh-1 inside each part.
    """
    d, f, e, a, s = m.d_model, m.d_mlp, m.enc_dim, m.action_dim, m.state_dim
    out: List[Tuple[str, Tuple[int, ...]]] = [
        ("w_in", (e, d)), ("b_in", (d,)),
        ("w_a", (a, d)), ("b_a", (d,)),
        ("w_s", (s, d)), ("b_s", (d,)),
    ]
    for l in range(m.layers):
        out += [
            (f"l{l}.ln1_g", (d,)), (f"l{l}.ln1_b", (d,)),
            (f"l{l}.w_qkv", (d, 3 * d)), (f"l{l}.b_qkv", (3 * d,)),
            (f"l{l}.w_o", (d, d)), (f"l{l}.b_o", (d,)),
            (f"l{l}.ln2_g", (d,)), (f"l{l}.ln2_b", (d,)),
            (f"l{l}.w_1", (d, f)), (f"l{l}.b_1", (f,)),
            (f"l{l}.w_2", (f, d)), (f"l{l}.b_2", (d,)),
        ]
    out += [("lnf_g", (d,)), ("lnf_b", (d,)), ("w_out", (d, e)), ("b_out", (e,))]
    return out


def weight_count(m: ModelConfig) -> int:
    return int(sum(int(np.prod(s)) for _, s in weight_layout(m)))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (ties to even) of finite float32 data, kept as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def make_weights(m: ModelConfig, seed: int = 0) -> Dict[str, np.ndarray]:
    """Random-init parameters, drawn in canonical order from PCG64(seed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out: Dict[str, np.ndarray] = {}
    for name, shape in weight_layout(m):
        v = rng.standard_normal(shape, dtype=np.float32) * np.float32(0.02)
        if name.endswith("_g"):
            v = v + np.float32(1.0)
        v = v.astype(np.float32)
        if m.dtype in ("bf16", "fp8"):
            v = round_to_bf16(v)
        out[name] = v
    return out


def flatten_weights(m: ModelConfig, w: Dict[str, np.ndarray]) -> np.ndarray:
    parts = []
    for name, shape in weight_layout(m):
        arr = np.asarray(w[name], dtype=np.float32)
        if arr.shape != shape:
            raise ValueError(f"{name}: shape {arr.shape} != {shape}")
        parts.append(arr.reshape(-1))
    return np.concatenate(parts).astype(np.float32, copy=False)


def make_embeddings(m: ModelConfig, seed: int = 1) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(z_obs [P,E], z_goal [P,E], s0 [S]) ~ N(0,1), float32."""
    rng = np.random.Generator(np.random.PCG64(seed))
    z_obs = rng.standard_normal((m.patches, m.enc_dim), dtype=np.float32)
    z_goal = rng.standard_normal((m.patches, m.enc_dim), dtype=np.float32)
    s0 = rng.standard_normal((m.state_dim,), dtype=np.float32)
    return z_obs, z_goal, s0


def make_actions(n: int, horizon: int, action_dim: int = ACTION_DIM, seed: int = 3) -> np.ndarray:
    """Stand-alone candidate actions in [-1, 1] for rollout-only cases."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.clip(rng.standard_normal((n, horizon, action_dim), dtype=np.float32), -1, 1)


def make_predictions(n: int, p: int, e: int, seed: int = 4) -> Tuple[np.ndarray, np.ndarray]:
    """Stand-alone (z_pred [n,P,E], z_goal [P,E]) ~ N(0,1) for energy-only cases."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.standard_normal((n, p, e), dtype=np.float32),
            rng.standard_normal((p, e), dtype=np.float32))

"""The oracle's predictor with bf16 storage of activations (test infrastructure).

A bf16 model stores its activations in bf16: the residual stream after the
embedding and after every residual add, the q/k/v projections, the attention
output, the MLP hidden layer and the predicted frame (statistics, softmax,
GELU and every accumulation stay wide).  The oracle itself computes in float64
throughout; this subclass rounds to the nearest bf16 value (ties to even) at
those storage points and nowhere else, so tests can tell how much of a
GPU-vs-oracle difference the method's own bf16 storage explains.  It uses only
the oracle and the input module's bf16 rounding.

Also here: the fp8 discrimination measure, i.e. how far a rollout lies from the
oracle's fp8-projection mode, in units of the whole fp8 effect
(fp8 mode minus plain mode).
"""
from __future__ import annotations

import numpy as np

from cem_jepa_predictor_amd import inputs
from oracle.predictor import Predictor, gelu, layer_norm

# A rollout counts as "fp8" when its rms distance to the oracle's fp8 mode is at
# most this fraction of the fp8 effect.  With bf16 storage the method itself sits
# near 0.45 after one layer (about 1 % of the LayerNorm outputs land on the other
# side of an e4m3 rounding boundary and move by a whole step); a rollout without
# fp8, or with the wrong matrices or scales quantized, sits at 1.0 or above.
FP8_GATE = 0.6


def round_bf16(x) -> np.ndarray:
    return inputs.round_to_bf16(np.asarray(x, np.float32)).astype(np.float64)


class Bf16Storage(Predictor):
    """Predictor whose stored activations are rounded to bf16."""

    def embed_block(self, a_t, s_t, f_t):
        return round_bf16(super().embed_block(a_t, s_t, f_t))

    def qkv(self, l, x):
        q, k, v = super().qkv(l, x)
        return round_bf16(q), round_bf16(k), round_bf16(v)

    def attn_out_and_mlp(self, l, x, o_heads):
        w = self.w
        o = round_bf16(o_heads)
        x = round_bf16(x + self.merge_heads(o) @ w[f"l{l}.w_o"] + w[f"l{l}.b_o"])
        h = self._proj_input(layer_norm(x, w[f"l{l}.ln2_g"], w[f"l{l}.ln2_b"], self.eps))
        u = round_bf16(gelu(h @ w[f"l{l}.w_1"] + w[f"l{l}.b_1"]))
        return round_bf16(x + u @ w[f"l{l}.w_2"] + w[f"l{l}.b_2"])

    def out_project(self, patch_rows):
        return round_bf16(super().out_project(patch_rows))


def rms(d) -> float:
    return float(np.sqrt(np.mean(np.square(np.asarray(d, np.float64)))))


def fp8_distance(z, z_fp8, z_plain) -> float:
    """rms(z - z_fp8) / rms(z_fp8 - z_plain)."""
    return rms(np.asarray(z, np.float64) - z_fp8) / rms(z_fp8 - z_plain)

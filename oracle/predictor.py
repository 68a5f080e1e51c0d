"""Action-conditioned, block-causal transformer predictor in float64.

Page "Real-Time Inference for JEPA World Model Architectures with Ray":
section 01 ("Where the sixteen seconds actually goes") pushes every candidate
action sequence through the predictor; section 05 ("Measured on 8x A100")
notes the predictor is frame-causal, so earlier frames never need recomputing
and a KV cache across rollout steps is exact.  The pages give no layer
equations; the readings taken (the plainest a transformer predictor with the
stated sizes supports) are:

  * frame block t holds B = P + 2 tokens, in this order: action token
    a_t W_a + b_a, state token s_t W_s + b_s, then P frame tokens
    f_t W_in + b_in.  No positional encoding (none is given), so the order
    inside a block does not matter;
  * f_0 = z_obs; f_{t+1} = LN_f(patch rows of block t) W_out + b_out;
    s_{t+1} = s_t + a_t;
  * pre-LN blocks: x += Attn(LN1 x) W_o + b_o; x += GELU(LN2 x W_1 + b_1) W_2 + b_2,
    fused q|k|v projection, softmax scale 1/sqrt(dh), exact (erf) GELU,
    LayerNorm with biased variance and eps from the model config;
  * block-causal mask: query i may attend key j iff block(j) <= block(i);
  * the rollout's output is the last predicted frame z_H [P, E].

Weights are the same dict the input generator draws; for bf16 models they are
already bf16-representable, and this module still computes in float64.

fp8 projections (page section 06, "D. Model compression": quantizing the
predictor shrinks the compute term; the OCP E4M3 format of the gfx950 matrix
cores): with fp8_projections the two LayerNorm-fed projections (fused q|k|v and
MLP up) see their weights quantized per tensor and their LayerNorm outputs
quantized per token row to E4M3 (oracle/fp8.py), then dequantized; every other
step is unchanged.
"""
from __future__ import annotations

from typing import Dict, List

import numpy as np
from scipy.special import erf

F64 = np.float64


def layer_norm(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float) -> np.ndarray:
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    return (x - mean) / np.sqrt(var + eps) * gamma + beta


def gelu(x: np.ndarray) -> np.ndarray:
    """Exact GELU: x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2))."""
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def block_causal_allowed(q_blocks: np.ndarray, k_blocks: np.ndarray) -> np.ndarray:
    """allowed[i, j] = block(key j) <= block(query i)."""
    return k_blocks[None, :] <= q_blocks[:, None]


def token_blocks(n_blocks: int, block_tokens: int) -> np.ndarray:
    return np.repeat(np.arange(n_blocks), block_tokens)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, allowed: np.ndarray) -> np.ndarray:
    """Masked softmax attention; q [.., Lq, dh], k/v [.., Lk, dh], allowed [Lq, Lk]."""
    dh = q.shape[-1]
    s = (q @ np.swapaxes(k, -1, -2)) / np.sqrt(F64(dh))
    s = np.where(allowed, s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return p @ v


class Predictor:
    """The predictor with float64 copies of the weights."""

    def __init__(self, weights: Dict[str, np.ndarray], layers: int, heads: int, eps: float,
                 fp8_projections: bool = False):
        self.w = {k: np.asarray(v, dtype=F64) for k, v in weights.items()}
        self.layers = layers
        self.heads = heads
        self.eps = eps
        self.d = self.w["b_in"].shape[0]
        self.dh = self.d // heads
        self.fp8 = fp8_projections
        if self.fp8:
            from .fp8 import dequantize, quantize_tensor

            for l in range(layers):
                for name in (f"l{l}.w_qkv", f"l{l}.w_1"):
                    codes, scale = quantize_tensor(np.asarray(weights[name], dtype=np.float32))
                    self.w[name] = dequantize(codes, scale)

    def _proj_input(self, h: np.ndarray) -> np.ndarray:
        """Input of a LayerNorm-fed projection: itself, or in fp8 mode its per-row
        E4M3 quantization (float32 rows), dequantized."""
        if not self.fp8:
            return h
        from .fp8 import dequantize, quantize_rows

        rows = h.reshape(-1, h.shape[-1]).astype(np.float32)
        codes, scale = quantize_rows(rows)
        return dequantize(codes, scale[:, None]).reshape(h.shape)

    # -- pieces -------------------------------------------------------------
    def embed_block(self, a_t: np.ndarray, s_t: np.ndarray, f_t: np.ndarray) -> np.ndarray:
        """Tokens of one frame block: [n, B, d] from a_t [n,A], s_t [n,S], f_t [n,P,E]."""
        w = self.w
        act = a_t @ w["w_a"] + w["b_a"]
        st = s_t @ w["w_s"] + w["b_s"]
        fr = f_t @ w["w_in"] + w["b_in"]
        return np.concatenate([act[:, None, :], st[:, None, :], fr], axis=1)

    def split_heads(self, x: np.ndarray) -> np.ndarray:
        n, t, _ = x.shape
        return x.reshape(n, t, self.heads, self.dh).transpose(0, 2, 1, 3)

    def merge_heads(self, x: np.ndarray) -> np.ndarray:
        n, _, t, _ = x.shape
        return x.transpose(0, 2, 1, 3).reshape(n, t, self.d)

    def qkv(self, l: int, x: np.ndarray):
        w = self.w
        h = self._proj_input(layer_norm(x, w[f"l{l}.ln1_g"], w[f"l{l}.ln1_b"], self.eps))
        y = h @ w[f"l{l}.w_qkv"] + w[f"l{l}.b_qkv"]
        d = self.d
        return (self.split_heads(y[..., :d]), self.split_heads(y[..., d:2 * d]),
                self.split_heads(y[..., 2 * d:]))

    def attn_out_and_mlp(self, l: int, x: np.ndarray, o_heads: np.ndarray) -> np.ndarray:
        w = self.w
        x = x + self.merge_heads(o_heads) @ w[f"l{l}.w_o"] + w[f"l{l}.b_o"]
        h = self._proj_input(layer_norm(x, w[f"l{l}.ln2_g"], w[f"l{l}.ln2_b"], self.eps))
        u = gelu(h @ w[f"l{l}.w_1"] + w[f"l{l}.b_1"])
        return x + u @ w[f"l{l}.w_2"] + w[f"l{l}.b_2"]

    def layer(self, l: int, x: np.ndarray, allowed: np.ndarray) -> np.ndarray:
        q, k, v = self.qkv(l, x)
        return self.attn_out_and_mlp(l, x, attention(q, k, v, allowed))

    def out_project(self, patch_rows: np.ndarray) -> np.ndarray:
        w = self.w
        h = layer_norm(patch_rows, w["lnf_g"], w["lnf_b"], self.eps)
        return h @ w["w_out"] + w["b_out"]

    # -- rollouts -------------------------------------------------------------
    def rollout(self, actions: np.ndarray, z_obs: np.ndarray, s0: np.ndarray,
                return_all: bool = False):
        """Autoregressive rollout by full block-causal recompute at every step.

        actions [n, H, A]; z_obs [P, E]; s0 [S].  Returns z_H [n, P, E]
        (or the list z_1..z_H when return_all).
        """
        actions = np.asarray(actions, dtype=F64)
        n, horizon, _ = actions.shape
        p = z_obs.shape[0]
        bt = p + 2
        f = np.broadcast_to(np.asarray(z_obs, dtype=F64), (n,) + z_obs.shape)
        s = np.broadcast_to(np.asarray(s0, dtype=F64), (n, s0.shape[0]))
        blocks: List[np.ndarray] = []
        frames = []
        for t in range(horizon):
            blocks.append(self.embed_block(actions[:, t], s, f))
            x = np.concatenate(blocks, axis=1)
            tb = token_blocks(t + 1, bt)
            allowed = block_causal_allowed(tb, tb)
            for l in range(self.layers):
                x = self.layer(l, x, allowed)
            f = self.out_project(x[:, t * bt + 2:(t + 1) * bt])
            frames.append(f)
            s = s + actions[:, t]
        return frames if return_all else frames[-1]

    def rollout_cached(self, actions: np.ndarray, z_obs: np.ndarray, s0: np.ndarray,
                       return_all: bool = False):
        """The same rollout with per-layer K/V of earlier blocks kept in a cache."""
        actions = np.asarray(actions, dtype=F64)
        n, horizon, _ = actions.shape
        f = np.broadcast_to(np.asarray(z_obs, dtype=F64), (n,) + z_obs.shape)
        s = np.broadcast_to(np.asarray(s0, dtype=F64), (n, s0.shape[0]))
        cache_k: List[List[np.ndarray]] = [[] for _ in range(self.layers)]
        cache_v: List[List[np.ndarray]] = [[] for _ in range(self.layers)]
        frames = []
        for t in range(horizon):
            x = self.embed_block(actions[:, t], s, f)
            for l in range(self.layers):
                q, k, v = self.qkv(l, x)
                cache_k[l].append(k)
                cache_v[l].append(v)
                kk = np.concatenate(cache_k[l], axis=2)
                vv = np.concatenate(cache_v[l], axis=2)
                # every cached key belongs to an earlier or the same block
                allowed = np.ones((q.shape[2], kk.shape[2]), dtype=bool)
                x = self.attn_out_and_mlp(l, x, attention(q, kk, vv, allowed))
            f = self.out_project(x[:, 2:])
            frames.append(f)
            s = s + actions[:, t]
        return frames if return_all else frames[-1]

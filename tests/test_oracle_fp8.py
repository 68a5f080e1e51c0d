"""Pins of the oracle's OCP E4M3 arithmetic (oracle/fp8.py) against the format's
definition: exact values of the specification, every finite code, ties to even,
nearest rounding by brute force, and the per-row / per-tensor scalings."""
import numpy as np
import pytest

from oracle import fp8


def _finite_codes():
    codes = np.arange(256, dtype=np.uint8)
    return codes[(codes & 0x7F) != 0x7F]


def test_known_values():
    enc = fp8.e4m3_encode
    assert enc([448.0])[0] == 0x7E and enc([-448.0])[0] == 0xFE      # largest finite
    assert enc([1.0])[0] == 0x38 and enc([-2.0])[0] == 0xC0
    assert enc([2.0 ** -6])[0] == 0x08                                 # smallest normal
    assert enc([2.0 ** -9])[0] == 0x01                                 # smallest subnormal
    assert enc([7 * 2.0 ** -9])[0] == 0x07                             # largest subnormal
    assert enc([0.0])[0] == 0x00 and enc([-0.0])[0] == 0x80
    dec = fp8.e4m3_decode
    assert dec(0x7E) == 448.0 and dec(0x01) == 2.0 ** -9 and np.isnan(dec(0x7F)) and np.isnan(dec(0xFF))
    with pytest.raises(ValueError):
        enc([449.0])


def test_every_finite_code_round_trips():
    codes = _finite_codes()
    vals = fp8.e4m3_decode(codes)
    np.testing.assert_array_equal(fp8.e4m3_encode(vals), codes)
    pos = np.sort(vals[vals > 0])
    assert len(pos) == 126 and np.all(np.diff(pos) > 0)


def test_ties_go_to_even_mantissa_and_rounding_is_nearest():
    pos = np.sort(np.unique(fp8.e4m3_decode(_finite_codes())[fp8.e4m3_decode(_finite_codes()) >= 0]))
    mids = (pos[:-1] + pos[1:]) / 2                      # exact in float64
    got = fp8.e4m3_encode(mids)
    assert np.all((got & 1) == 0)                        # the even neighbour
    np.testing.assert_array_equal(np.isin(fp8.e4m3_decode(got), pos[:-1]) | np.isin(fp8.e4m3_decode(got), pos[1:]), True)
    rng = np.random.default_rng(0)
    x = rng.uniform(-448, 448, 20000) * rng.choice([1.0, 1e-2, 1e-4], 20000)
    q = fp8.e4m3_decode(fp8.e4m3_encode(x))
    allv = np.concatenate([-pos[::-1], pos])
    best = np.min(np.abs(allv[None, :] - x[:, None]), axis=1)     # brute-force nearest distance
    np.testing.assert_allclose(np.abs(q - x), best, rtol=0, atol=0)


def test_quantize_rows_scaling():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64)).astype(np.float32) * np.float32(3.0)
    x[2] = 0.0
    codes, scale = fp8.quantize_rows(x)
    assert scale.dtype == np.float32 and scale[2] == 1.0 and np.all(codes[2] == 0)
    for r in (0, 1, 3, 4):
        j = np.argmax(np.abs(x[r]))
        assert codes[r, j] & 0x7F == 0x7E                # the row's largest magnitude maps to 448
        assert scale[r] == np.float32(np.abs(x[r, j]) / np.float32(448.0))
    deq = fp8.dequantize(codes, scale[:, None])
    big = np.abs(x) >= 2.0 ** -6 * scale[:, None]
    rel = np.abs(deq - x)[big] / np.abs(x)[big]
    assert rel.max() <= 2.0 ** -4 + 1e-7                 # half a step of a 3-bit mantissa


def test_quantize_tensor_scaling():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((48, 32)) * 0.02).astype(np.float32)
    codes, s = fp8.quantize_tensor(w)
    assert s == np.float32(np.abs(w).max() / np.float32(448.0))
    assert np.sum((codes & 0x7F) == 0x7E) >= 1
    deq = fp8.dequantize(codes, s)
    assert np.abs(deq - w).max() <= 2.0 ** -4 * np.abs(w).max()
    c0, s0 = fp8.quantize_tensor(np.zeros((3, 3), np.float32))
    assert s0 == 1.0 and np.all(c0 == 0)


def test_fp8_projections_perturb_the_rollout_slightly():
    """The fp8 predictor differs from the float64 one by the quantization of two
    projections: present, and small against the prediction itself."""
    from cem_jepa_predictor_amd import inputs
    from oracle.predictor import Predictor

    wl = inputs.WORKLOADS["small"]
    m = wl.model
    w = inputs.make_weights(m, wl.weight_seed)
    z_obs, _, s0 = inputs.make_embeddings(m, wl.embed_seed)
    acts = inputs.make_actions(3, 1, seed=3)
    ref = Predictor(w, m.layers, m.heads, m.ln_eps).rollout_cached(acts, z_obs, s0)
    q8 = Predictor(w, m.layers, m.heads, m.ln_eps, fp8_projections=True).rollout_cached(acts, z_obs, s0)
    d = np.abs(q8 - ref).max() / np.abs(ref).max()
    assert 1e-4 < d < 0.1, d


def _fp8_layer_case():
    m = inputs_mod().ModelConfig("pin8", 1, 64, 4, 128, 6, 48, "fp8", 1)
    w = inputs_mod().make_weights(m, 5)
    rng = np.random.default_rng(7)
    x = rng.standard_normal((3, m.block_tokens, m.d_model)) * 0.8 + 0.3
    o_heads = rng.standard_normal((3, m.heads, m.block_tokens, m.head_dim)) * 0.5
    return m, w, x, o_heads


def inputs_mod():
    from cem_jepa_predictor_amd import inputs

    return inputs


def test_fp8_layer_matches_independent_composition():
    """Pin of the fp8-projection mode's placement (page section 06, "D. Model
    compression"), written independently with torch: LayerNorm with its gain and
    shift, then the per-row E4M3 quantization of that output (as float32), then the
    product with the per-tensor-quantized w_qkv / w_1; w_o and w_2 are untouched.
    Quantizing another matrix, quantizing before the gain and shift, or per-column
    weight scales all change the result far beyond 1e-12."""
    import torch

    from oracle.predictor import Predictor

    m, w, x, o_heads = _fp8_layer_case()
    d, H, dh = m.d_model, m.heads, m.head_dim
    pred = Predictor(w, 1, H, m.ln_eps, fp8_projections=True)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))  # noqa: E731

    def ln_then_rows(v, g, b):
        h = torch.nn.functional.layer_norm(t(v), (d,), t(g), t(b), eps=m.ln_eps).numpy()
        codes, scale = fp8.quantize_rows(h.reshape(-1, d).astype(np.float32))
        return t(fp8.dequantize(codes, scale[:, None]).reshape(v.shape))

    def per_tensor(name):
        codes, s = fp8.quantize_tensor(np.asarray(w[name], np.float32))
        return t(fp8.dequantize(codes, s))

    # q|k|v
    y = ln_then_rows(x, w["l0.ln1_g"], w["l0.ln1_b"]) @ per_tensor("l0.w_qkv") + t(w["l0.b_qkv"])
    heads = lambda z: z.reshape(z.shape[0], z.shape[1], H, dh).permute(0, 2, 1, 3).numpy()  # noqa: E731
    for got, want in zip(pred.qkv(0, x), (heads(y[..., :d]), heads(y[..., d:2 * d]), heads(y[..., 2 * d:]))):
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    # output projection (plain), MLP up (fp8) with exact GELU, MLP down (plain)
    o = t(o_heads).permute(0, 2, 1, 3).reshape(x.shape)
    x1 = t(x) + o @ t(w["l0.w_o"]) + t(w["l0.b_o"])
    u = torch.nn.functional.gelu(ln_then_rows(x1.numpy(), w["l0.ln2_g"], w["l0.ln2_b"]) @ per_tensor("l0.w_1")
                                 + t(w["l0.b_1"]), approximate="none")
    want = (x1 + u @ t(w["l0.w_2"]) + t(w["l0.b_2"])).numpy()
    np.testing.assert_allclose(pred.attn_out_and_mlp(0, x, o_heads), want, rtol=0, atol=1e-12)
    for name in ("l0.w_o", "l0.w_2", "w_in", "w_out"):
        np.testing.assert_array_equal(pred.w[name], np.asarray(w[name], np.float64))


def test_fp8_gate_separates_the_method_from_its_mutants():
    """The GPU fp8 gate (distance to the oracle's fp8 mode, in units of the fp8
    effect) on the one-layer fp8 workload: the method with bf16 activation storage,
    as the device runs it, passes; the same with no fp8, with w_o / w_2 quantized
    in place of w_qkv / w_1, with quantization before the LayerNorm gain and shift,
    or with per-column weight scales fails."""
    from oracle.predictor import Predictor, gelu, layer_norm

    from .bf16_storage import FP8_GATE, Bf16Storage, fp8_distance, round_bf16

    inputs = inputs_mod()
    wl = inputs.WORKLOADS["shallow_fp8"]
    m = wl.model
    w = inputs.make_weights(m, wl.weight_seed)
    z_obs, _, s0 = inputs.make_embeddings(m, wl.embed_seed)
    acts = inputs.make_actions(4, wl.plan.horizon, seed=3)
    args = (w, m.layers, m.heads, m.ln_eps)
    z8 = Predictor(*args, fp8_projections=True).rollout_cached(acts, z_obs, s0)
    z = Predictor(*args).rollout_cached(acts, z_obs, s0)

    def quantized(names):
        out = {}
        for name in names:
            codes, s = fp8.quantize_tensor(np.asarray(w[name], np.float32))
            out[name] = fp8.dequantize(codes, s)
        return out

    class WrongMatrices(Bf16Storage):
        def __init__(self):
            super().__init__(*args, fp8_projections=True)
            for l in range(m.layers):
                for name in (f"l{l}.w_qkv", f"l{l}.w_1"):
                    self.w[name] = np.asarray(w[name], np.float64)
                self.w.update(quantized([f"l{l}.w_o", f"l{l}.w_2"]))

    class BeforeAffine(Bf16Storage):
        """Both LayerNorm-fed inputs quantized before the LayerNorm gain and shift."""

        def _ln_q(self, x, g, b):
            return self._proj_input(layer_norm(x, np.ones_like(g), np.zeros_like(b), self.eps)) * g + b

        def qkv(self, l, x):
            y = self._ln_q(x, self.w[f"l{l}.ln1_g"], self.w[f"l{l}.ln1_b"]) @ self.w[f"l{l}.w_qkv"] \
                + self.w[f"l{l}.b_qkv"]
            d = self.d
            return tuple(round_bf16(self.split_heads(y[..., i * d:(i + 1) * d])) for i in range(3))

        def attn_out_and_mlp(self, l, x, o_heads):
            w = self.w
            x = round_bf16(x + self.merge_heads(round_bf16(o_heads)) @ w[f"l{l}.w_o"] + w[f"l{l}.b_o"])
            u = round_bf16(gelu(self._ln_q(x, w[f"l{l}.ln2_g"], w[f"l{l}.ln2_b"]) @ w[f"l{l}.w_1"]
                                + w[f"l{l}.b_1"]))
            return round_bf16(x + u @ w[f"l{l}.w_2"] + w[f"l{l}.b_2"])

    class PerColumn(Bf16Storage):
        def __init__(self):
            super().__init__(*args, fp8_projections=True)
            for l in range(m.layers):
                for name in (f"l{l}.w_qkv", f"l{l}.w_1"):
                    W = np.asarray(w[name], np.float32)
                    self.w[name] = np.concatenate(
                        [fp8.dequantize(*fp8.quantize_tensor(W[:, j:j + 1])) for j in range(W.shape[1])], axis=1)

    method = fp8_distance(Bf16Storage(*args, fp8_projections=True).rollout_cached(acts, z_obs, s0), z8, z)
    assert method <= FP8_GATE - 0.05, method
    mutants = {
        "no fp8": Bf16Storage(*args),
        "w_o and w_2 quantized": WrongMatrices(),
        "quantized before gain and shift": BeforeAffine(*args, fp8_projections=True),
        "per-column weight scales": PerColumn(),
    }
    for name, pred in mutants.items():
        dist = fp8_distance(pred.rollout_cached(acts, z_obs, s0), z8, z)
        assert dist >= FP8_GATE + 0.25, (name, dist)

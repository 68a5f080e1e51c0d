"""Pins of the oracle's predictor against independent library routines (CPU, float64)."""
import numpy as np
import pytest
import torch

from cem_jepa_predictor_amd import inputs
from oracle import predictor as P



@pytest.fixture(autouse=True, scope="module")
def _float64_modules():
    """torch.nn modules built here get float64 parameters; the global default is
    restored afterwards so other test modules keep float32."""
    prev = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(prev)


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))


def test_layer_norm_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 7, 96)) * 3 + 1.5
    g = 1 + 0.1 * rng.standard_normal(96)
    b = 0.1 * rng.standard_normal(96)
    want = torch.nn.functional.layer_norm(_t(x), (96,), _t(g), _t(b), eps=1e-5).numpy()
    np.testing.assert_allclose(P.layer_norm(x, g, b, 1e-5), want, rtol=1e-12, atol=1e-12)
    # normalised rows (unit gain, zero shift) have mean 0 and variance 1 - eps/(var+eps)
    y = P.layer_norm(x, np.ones(96), np.zeros(96), 0.0)
    np.testing.assert_allclose(y.mean(-1), 0, atol=1e-12)
    np.testing.assert_allclose(y.var(-1), 1, atol=1e-12)


def test_gelu_matches_torch_exact():
    x = np.linspace(-8, 8, 4001)
    want = torch.nn.functional.gelu(_t(x), approximate="none").numpy()
    np.testing.assert_allclose(P.gelu(x), want, rtol=1e-14, atol=1e-15)
    assert P.gelu(np.array([0.0]))[0] == 0.0


def test_block_causal_mask_by_enumeration():
    B, T = 5, 3
    tb = P.token_blocks(T, B)
    allowed = P.block_causal_allowed(tb, tb)
    for i in range(T * B):
        for j in range(T * B):
            assert allowed[i, j] == (j // B <= i // B)


def test_attention_matches_torch_sdpa_with_mask():
    rng = np.random.default_rng(1)
    B, T, dh = 6, 3, 16
    tb = P.token_blocks(T, B)
    allowed = P.block_causal_allowed(tb, tb)
    q, k, v = (rng.standard_normal((2, 4, T * B, dh)) for _ in range(3))
    want = torch.nn.functional.scaled_dot_product_attention(
        _t(q), _t(k), _t(v), attn_mask=torch.from_numpy(allowed)).numpy()
    np.testing.assert_allclose(P.attention(q, k, v, allowed), want, rtol=1e-12, atol=1e-12)


def test_attention_mask_probe_recovers_mask():
    """Q = 0 gives uniform weights over allowed keys; one-hot V reads them back."""
    B, T = 4, 3
    L = T * B
    tb = P.token_blocks(T, B)
    allowed = P.block_causal_allowed(tb, tb)
    q = np.zeros((1, 1, L, L))
    k = np.random.default_rng(2).standard_normal((1, 1, L, L))
    v = np.eye(L)[None, None]
    out = P.attention(q, k, v, allowed)[0, 0]
    want = allowed / allowed.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(out, want, rtol=1e-14, atol=1e-15)


def _small_model(layers=2, d=32, heads=4, f=64, p=5, e=24, seed=0):
    m = inputs.ModelConfig("t", layers, d, heads, f, p, e, "f32", 3)
    w = inputs.make_weights(m, seed)
    # larger weights than the random-init recipe so every term matters numerically
    rng = np.random.default_rng(seed + 100)
    w = {k: (v + 0.2 * rng.standard_normal(v.shape)).astype(np.float64) for k, v in w.items()}
    return m, w


def _torch_layer(w, l, d, heads, f):
    layer = torch.nn.TransformerEncoderLayer(d, heads, f, dropout=0.0, activation="gelu",
                                             layer_norm_eps=1e-5, batch_first=True, norm_first=True)
    with torch.no_grad():
        layer.self_attn.in_proj_weight.copy_(_t(w[f"l{l}.w_qkv"]).T)
        layer.self_attn.in_proj_bias.copy_(_t(w[f"l{l}.b_qkv"]))
        layer.self_attn.out_proj.weight.copy_(_t(w[f"l{l}.w_o"]).T)
        layer.self_attn.out_proj.bias.copy_(_t(w[f"l{l}.b_o"]))
        layer.linear1.weight.copy_(_t(w[f"l{l}.w_1"]).T)
        layer.linear1.bias.copy_(_t(w[f"l{l}.b_1"]))
        layer.linear2.weight.copy_(_t(w[f"l{l}.w_2"]).T)
        layer.linear2.bias.copy_(_t(w[f"l{l}.b_2"]))
        layer.norm1.weight.copy_(_t(w[f"l{l}.ln1_g"]))
        layer.norm1.bias.copy_(_t(w[f"l{l}.ln1_b"]))
        layer.norm2.weight.copy_(_t(w[f"l{l}.ln2_g"]))
        layer.norm2.bias.copy_(_t(w[f"l{l}.ln2_b"]))
    return layer.eval()


def test_layer_matches_torch_transformer_encoder_layer():
    m, w = _small_model()
    pred = P.Predictor(w, m.layers, m.heads, m.ln_eps)
    B, T = m.block_tokens, 2
    tb = P.token_blocks(T, B)
    allowed = P.block_causal_allowed(tb, tb)
    x = np.random.default_rng(3).standard_normal((3, T * B, m.d_model))
    layer = _torch_layer(w, 1, m.d_model, m.heads, m.d_mlp)
    with torch.no_grad():
        want = layer(_t(x), src_mask=torch.from_numpy(~allowed)).numpy()   # True = masked out
    np.testing.assert_allclose(pred.layer(1, x, allowed), want, rtol=1e-10, atol=1e-10)


def _torch_rollout(w, m, actions, z_obs, s0):
    """Independent composition from torch.nn modules (recompute at each step)."""
    layers = [_torch_layer(w, l, m.d_model, m.heads, m.d_mlp) for l in range(m.layers)]
    n, H, _ = actions.shape
    B = m.block_tokens
    f = _t(np.broadcast_to(z_obs, (n,) + z_obs.shape))
    s = _t(np.broadcast_to(s0, (n, s0.shape[0])))
    a = _t(actions)
    lin = torch.nn.functional.linear
    blocks = []
    with torch.no_grad():
        for t in range(H):
            tok_a = lin(a[:, t], _t(w["w_a"]).T, _t(w["b_a"]))[:, None]
            tok_s = lin(s, _t(w["w_s"]).T, _t(w["b_s"]))[:, None]
            tok_f = lin(f, _t(w["w_in"]).T, _t(w["b_in"]))
            blocks.append(torch.cat([tok_a, tok_s, tok_f], dim=1))
            x = torch.cat(blocks, dim=1)
            blk = torch.arange((t + 1) * B) // B
            masked = blk[None, :] > blk[:, None]
            for layer in layers:
                x = layer(x, src_mask=masked)
            pr = torch.nn.functional.layer_norm(x[:, t * B + 2:(t + 1) * B], (m.d_model,),
                                                _t(w["lnf_g"]), _t(w["lnf_b"]), eps=m.ln_eps)
            f = lin(pr, _t(w["w_out"]).T, _t(w["b_out"]))
            s = s + a[:, t]
    return f.numpy()


def test_rollout_matches_torch_module_composition():
    m, w = _small_model(layers=2)
    pred = P.Predictor(w, m.layers, m.heads, m.ln_eps)
    rng = np.random.default_rng(4)
    actions = rng.uniform(-1, 1, (3, 3, m.action_dim))
    z_obs = rng.standard_normal((m.patches, m.enc_dim))
    s0 = rng.standard_normal(m.state_dim)
    want = _torch_rollout(w, m, actions, z_obs, s0)
    np.testing.assert_allclose(pred.rollout(actions, z_obs, s0), want, rtol=1e-10, atol=1e-10)


def test_kv_cached_rollout_equals_recompute():
    m, w = _small_model(layers=3)
    pred = P.Predictor(w, m.layers, m.heads, m.ln_eps)
    rng = np.random.default_rng(5)
    actions = rng.uniform(-1, 1, (4, 3, m.action_dim))
    z_obs = rng.standard_normal((m.patches, m.enc_dim))
    s0 = rng.standard_normal(m.state_dim)
    full = pred.rollout(actions, z_obs, s0, return_all=True)
    cached = pred.rollout_cached(actions, z_obs, s0, return_all=True)
    for a, b in zip(full, cached):
        np.testing.assert_allclose(b, a, rtol=1e-11, atol=1e-11)


def test_rollout_is_frame_causal_and_patch_equivariant():
    m, w = _small_model(layers=2)
    pred = P.Predictor(w, m.layers, m.heads, m.ln_eps)
    rng = np.random.default_rng(6)
    actions = rng.uniform(-1, 1, (2, 3, m.action_dim))
    z_obs = rng.standard_normal((m.patches, m.enc_dim))
    s0 = rng.standard_normal(m.state_dim)
    base = pred.rollout(actions, z_obs, s0, return_all=True)
    # changing the last step's action leaves the earlier predicted frames alone
    a2 = actions.copy()
    a2[:, 2] = -a2[:, 2]
    alt = pred.rollout(a2, z_obs, s0, return_all=True)
    np.testing.assert_array_equal(alt[0], base[0])
    np.testing.assert_array_equal(alt[1], base[1])
    assert np.abs(alt[2] - base[2]).max() > 1e-6
    # and it does reach the output through the action token
    a3 = actions.copy()
    a3[:, 0] = -a3[:, 0]
    assert np.abs(pred.rollout(a3, z_obs, s0) - base[2]).max() > 1e-6
    # no positional encoding: permuting patch rows permutes the prediction's rows
    perm = rng.permutation(m.patches)
    permuted = pred.rollout(actions, z_obs[perm], s0, return_all=True)
    np.testing.assert_allclose(permuted[2], base[2][:, perm], rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_workload_shapes_roll_out(name):
    wl = inputs.WORKLOADS[name]
    m = wl.model
    w = inputs.make_weights(m, wl.weight_seed)
    z_obs, z_goal, s0 = inputs.make_embeddings(m, wl.embed_seed)
    pred = P.Predictor(w, m.layers, m.heads, m.ln_eps)
    actions = inputs.make_actions(2, wl.plan.horizon)
    z = pred.rollout_cached(actions, z_obs, s0)
    assert z.shape == (2, m.patches, m.enc_dim) and np.isfinite(z).all()

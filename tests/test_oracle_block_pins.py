"""Pins for the oracle's transformer block against an independent library
implementation and closed forms.

The block is the pre-norm Llama block of the benchmark's model families
(Llama-2-7B / 13B, Yi-34B): RMSNorm, q/k/v projections with RoPE, causal
attention with grouped-query heads, O projection and residual, RMSNorm,
SwiGLU MLP and residual.  The CacheBlend explainer (0h-n0), section
"選択的再計算", Step 4 finishes every layer with this standard computation on
the recomputed rows.  `transformers`' LlamaMLP / LlamaRMSNorm /
LlamaDecoderLayer (run in float64 on the CPU) is the library it is pinned to:
it shares no code with the oracle.

The library rotates pairs (i, i + d_head/2); the oracle rotates interleaved
pairs (2i, 2i+1) (CacheBlend explainer (0h-n0), section "RoPE（Rotary
Position Embedding）との整合性").  Permuting the output rows of W_q and W_k
within each head maps one convention onto the other without changing any
attention score, so the layer outputs must agree.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import ModelShape
from tests.helpers import rel_err

transformers = pytest.importorskip("transformers")
from transformers import LlamaConfig  # noqa: E402
from transformers.models.llama import modeling_llama as hf  # noqa: E402


def _shape(hq=4, hkv=2, dh=16, d=64, f=96):
    return ModelShape(1, d, hq, hkv, dh, f, vocab=64)


def _weights(shape, seed, scale=0.2):
    rng = np.random.default_rng(seed)
    d, qd, kvd, f = shape.d_model, shape.q_dim, shape.kv_dim, shape.ffn_dim
    return {
        "attn_norm": 1.0 + 0.1 * rng.standard_normal(d),
        "wq": scale * rng.standard_normal((qd, d)),
        "wk": scale * rng.standard_normal((kvd, d)),
        "wv": scale * rng.standard_normal((kvd, d)),
        "wo": scale * rng.standard_normal((d, qd)),
        "mlp_norm": 1.0 + 0.1 * rng.standard_normal(d),
        "w_gate": scale * rng.standard_normal((f, d)),
        "w_up": scale * rng.standard_normal((f, d)),
        "w_down": scale * rng.standard_normal((d, f)),
    }


def _hf_config(shape):
    cfg = LlamaConfig(hidden_size=shape.d_model, intermediate_size=shape.ffn_dim,
                      num_attention_heads=shape.n_q_heads,
                      num_key_value_heads=shape.n_kv_heads, head_dim=shape.head_dim,
                      rms_norm_eps=shape.rms_eps, attention_bias=False, mlp_bias=False,
                      hidden_act="silu", max_position_embeddings=4096,
                      rope_parameters={"rope_type": "default", "rope_theta": shape.rope_base})
    cfg._attn_implementation = "sdpa"     # eager softmax would run in float32
    return cfg


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


class _RMSNorm64(torch.nn.Module):
    """torch.nn.functional.rms_norm in float64 (LlamaRMSNorm computes its
    mean square in float32, which would cap the pin near 1e-7)."""

    def __init__(self, d, eps):
        super().__init__()
        self.weight = torch.nn.Parameter(torch.ones(d, dtype=torch.float64))
        self.eps = eps

    def forward(self, x):
        return torch.nn.functional.rms_norm(x, (x.shape[-1],), self.weight, eps=self.eps)


def _half_split_rows(w, n_heads, dh):
    """Output rows of a q/k projection reordered per head from interleaved
    pairs (2i, 2i+1) to the library's (i, i + dh/2) pairs."""
    perm = np.concatenate([np.arange(0, dh, 2), np.arange(1, dh, 2)])
    idx = np.concatenate([h * dh + perm for h in range(n_heads)])
    return w[idx]


def _hf_mlp_tail(shape, w, x, att):
    """O projection + residual, RMSNorm, LlamaMLP, residual, all from the
    library's modules."""
    cfg = _hf_config(shape)
    mlp = hf.LlamaMLP(cfg).double()
    norm = _RMSNorm64(shape.d_model, shape.rms_eps)
    with torch.no_grad():
        mlp.gate_proj.weight.copy_(_t(w["w_gate"]))
        mlp.up_proj.weight.copy_(_t(w["w_up"]))
        mlp.down_proj.weight.copy_(_t(w["w_down"]))
        norm.weight.copy_(_t(w["mlp_norm"]))
        h = _t(x) + torch.nn.functional.linear(_t(att).reshape(x.shape[0], -1), _t(w["wo"]))
        return (h + mlp(norm(h))).numpy()


# ---------------------------------------------------------------- block tail
@pytest.mark.parametrize("hq,hkv,dh", [(4, 4, 16), (4, 2, 16), (6, 1, 8)])
def test_finish_rows_vs_llama_mlp(hq, hkv, dh):
    """O projection + residual, then RMSNorm + SwiGLU MLP + residual, equals
    the library's linear / LlamaRMSNorm / LlamaMLP with explicit residuals
    (non-square O projection when Hq*dh != d)."""
    shape = _shape(hq, hkv, dh, d=48, f=80)
    w = _weights(shape, seed=hq * 10 + hkv)
    rng = np.random.default_rng(7)
    x = rng.standard_normal((9, shape.d_model))
    att = rng.standard_normal((9, hq, dh))
    got = oracle.finish_rows(w, shape, x, att)
    assert rel_err(got, _hf_mlp_tail(shape, w, x, att)) < 1e-13


def test_finish_rows_detects_swapped_gate_and_up():
    """A plausible slip (SiLU applied to the up projection instead of the
    gate) moves the result far outside the tolerance of the pin above, so
    that pin would catch it."""
    shape = _shape(d=48, f=80)
    w = _weights(shape, seed=3)
    rng = np.random.default_rng(8)
    x = rng.standard_normal((5, shape.d_model))
    att = rng.standard_normal((5, shape.n_q_heads, shape.head_dim))
    ref = _hf_mlp_tail(shape, w, x, att)
    swapped = dict(w, w_gate=w["w_up"], w_up=w["w_gate"])
    assert rel_err(oracle.finish_rows(swapped, shape, x, att), ref) > 1e-3
    # residual taken from the wrong tensor: the MLP residual must be h, not x
    h = x + att.reshape(5, -1) @ w["wo"].T
    wrong = x + (oracle.finish_rows(w, shape, x, att) - h)
    assert rel_err(wrong, ref) > 1e-3


def test_finish_rows_closed_forms():
    """W_up = 0: SiLU(gate)*0 = 0, so the output is h = x + att W_o^T exactly.
    W_o = 0: h = x exactly, so the output is x + MLP(x).  Both zero: x."""
    shape = _shape(d=48, f=80)
    w = _weights(shape, seed=4)
    rng = np.random.default_rng(9)
    x = rng.standard_normal((6, shape.d_model))
    att = rng.standard_normal((6, shape.n_q_heads, shape.head_dim))
    h = x + att.reshape(6, -1) @ w["wo"].T
    no_up = dict(w, w_up=np.zeros_like(w["w_up"]))
    assert np.array_equal(oracle.finish_rows(no_up, shape, x, att), h)
    no_o = dict(w, wo=np.zeros_like(w["wo"]))
    mlp_x = oracle.finish_rows(no_o, shape, x, att) - x
    want = _hf_mlp_tail(shape, no_o, x, np.zeros_like(att)) - x
    assert rel_err(mlp_x, want) < 1e-13
    both = dict(no_up, wo=np.zeros_like(w["wo"]))
    assert np.array_equal(oracle.finish_rows(both, shape, x, att), x)


# ---------------------------------------------------------------- whole layer
def _hf_layer(shape, w, x, pos0):
    """One LlamaDecoderLayer in float64 with cos/sin of the oracle's angles
    (float64, theta_i = base^(-2i/d_head)) in the library's half-split
    layout, causal additive mask."""
    cfg = _hf_config(shape)
    layer = hf.LlamaDecoderLayer(cfg, layer_idx=0).double()
    layer.input_layernorm = _RMSNorm64(shape.d_model, shape.rms_eps)
    layer.post_attention_layernorm = _RMSNorm64(shape.d_model, shape.rms_eps)
    dh = shape.head_dim
    with torch.no_grad():
        a = layer.self_attn
        a.q_proj.weight.copy_(_t(_half_split_rows(w["wq"], shape.n_q_heads, dh)))
        a.k_proj.weight.copy_(_t(_half_split_rows(w["wk"], shape.n_kv_heads, dh)))
        a.v_proj.weight.copy_(_t(w["wv"]))
        a.o_proj.weight.copy_(_t(w["wo"]))
        layer.mlp.gate_proj.weight.copy_(_t(w["w_gate"]))
        layer.mlp.up_proj.weight.copy_(_t(w["w_up"]))
        layer.mlp.down_proj.weight.copy_(_t(w["w_down"]))
        layer.input_layernorm.weight.copy_(_t(w["attn_norm"]))
        layer.post_attention_layernorm.weight.copy_(_t(w["mlp_norm"]))
        n = x.shape[0]
        pos = np.arange(pos0, pos0 + n, dtype=np.float64)
        theta = shape.rope_base ** (-2.0 * np.arange(dh // 2) / dh)
        ang = pos[:, None] * theta[None, :]
        cos = _t(np.concatenate([np.cos(ang), np.cos(ang)], axis=1))[None]
        sin = _t(np.concatenate([np.sin(ang), np.sin(ang)], axis=1))[None]
        mask = torch.full((n, n), float("-inf"), dtype=torch.float64).triu(1)[None, None]
        y = layer(_t(x)[None], attention_mask=mask,
                  position_ids=torch.arange(pos0, pos0 + n)[None],
                  position_embeddings=(cos, sin))
        y = y[0] if isinstance(y, tuple) else y
        # keys as the library computes them, mapped back to interleaved pairs
        hn = layer.input_layernorm(_t(x)[None])
        k = a.k_proj(hn).view(1, n, shape.n_kv_heads, dh).transpose(1, 2)
        k = hf.apply_rotary_pos_emb(k, k, cos, sin)[0].transpose(1, 2)[0].numpy()
        inter = np.empty_like(k)
        inter[..., 0::2] = k[..., :dh // 2]
        inter[..., 1::2] = k[..., dh // 2:]
    return y[0].numpy(), inter


@pytest.mark.parametrize("hq,hkv,dh,pos0", [(4, 4, 16, 0), (4, 2, 16, 37), (8, 2, 8, 500)])
def test_prefill_layer_vs_llama_decoder_layer(hq, hkv, dh, pos0):
    """One oracle prefill layer (rows at positions pos0..) equals the
    library's LlamaDecoderLayer: output rows and RoPE'd keys."""
    shape = _shape(hq, hkv, dh, d=64, f=112)
    w = _weights(shape, seed=100 + hq + hkv + dh)
    x = np.random.default_rng(11).standard_normal((21, shape.d_model))
    k, v, outs = oracle.prefill([w], shape, x, pos0=pos0)
    y_ref, k_ref = _hf_layer(shape, w, x, pos0)
    assert rel_err(outs[0], y_ref) < 1e-12
    assert rel_err(k[0], k_ref) < 1e-12


def test_prefill_layer_transposed_o_projection_is_caught():
    """With Hq*dh = d the O projection's orientation is not fixed by shapes;
    the library comparison catches W_o used transposed."""
    shape = _shape(4, 4, 16, d=64, f=112)
    w = _weights(shape, seed=5)
    x = np.random.default_rng(12).standard_normal((13, shape.d_model))
    y_ref, _ = _hf_layer(shape, w, x, 0)
    bad = dict(w, wo=w["wo"].T.copy())
    _, _, outs = oracle.prefill([bad], shape, x)
    assert rel_err(outs[0], y_ref) > 1e-3


# ---------------------------------------------------------------- rank correlation
def test_layer_rank_correlation_vs_scipy():
    """Insight 2 of the CacheBlend explainer (0h-n0), "HKVD（High KV
    Deviation）トークン選定": Spearman's rho between consecutive layers'
    deviations over the tokens measured at both layers, against
    scipy.stats.spearmanr on the same masked pairs (NaN = not measured)."""
    import scipy.stats
    rng = np.random.default_rng(21)
    L, n = 6, 50
    dev = rng.standard_normal((L, n)).cumsum(axis=0)
    dev[2, rng.choice(n, 20, replace=False)] = np.nan   # narrowed sets
    dev[3, :] = np.nan
    dev[3, :2] = [1.0, 2.0]                             # fewer than 3 shared: NaN
    dev[4, rng.choice(n, 5, replace=False)] = 7.0       # ties
    got = oracle.layer_rank_correlation(dev)
    assert len(got) == L - 1
    for l in range(L - 1):
        m = ~np.isnan(dev[l]) & ~np.isnan(dev[l + 1])
        if m.sum() < 3:
            assert math.isnan(got[l])
        else:
            want = scipy.stats.spearmanr(dev[l][m], dev[l + 1][m])[0]
            assert got[l] == pytest.approx(want, abs=1e-12), l
    # identical rankings give 1, reversed give -1
    x = rng.standard_normal(30)
    assert oracle.layer_rank_correlation(np.stack([x, 3 * x + 1, -x]))[0] == pytest.approx(1.0)
    assert oracle.layer_rank_correlation(np.stack([x, -x]))[0] == pytest.approx(-1.0)

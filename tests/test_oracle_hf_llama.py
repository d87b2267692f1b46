"""Independent pin of the oracle's whole layer composition: the oracle's forward
against the Llama decoder of the `transformers` library (built from a config,
random weights copied in, no download).

The oracle follows CS349E Lecture 6 ("Optimizing Autoregressive Decode"),
section 6.2 step 2 (one target forward over the window gives every row's
next-token distribution) and section 4.2 (the per-token layers over the
flattened rows, attention per sequence over its own cache).  The library's
decoder is an implementation of the same Llama-style model written by
others: pre-norm RMSNorm, rotate-half rotary embedding, grouped-query
attention, SwiGLU MLP, a final RMSNorm and an untied output head.  Agreement
to ~1e-7 relative pins the order and wiring of every sub-layer (which half of
the fused gate/up matrix is the gate, where each norm sits, which residual
each sub-layer reads), which the oracle's own consistency tests cannot see.

The library normalises in fp32 inside its RMSNorm even for an fp64 model, so
the bar is 1e-6 of the largest logit, far below what any wiring mistake moves
(those change logits by O(1) of their scale).
"""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

transformers = pytest.importorskip("transformers")

from oracle import model as M  # noqa: E402


def _shape(L=2, d=64, Hq=4, Hkv=2, D=16, F=96, V=97, theta=10000.0):
    return SimpleNamespace(n_layers=L, d_model=d, n_heads=Hq, n_kv_heads=Hkv, head_dim=D,
                           d_ffn=F, vocab=V, rms_eps=1e-5, rope_theta=theta)


def _weights(sh, seed):
    """Random weights with non-unit norm gains (so a misplaced gain shows)."""
    rng = np.random.default_rng(seed)
    d, F, V = sh.d_model, sh.d_ffn, sh.vocab
    qkv = (sh.n_heads + 2 * sh.n_kv_heads) * sh.head_dim
    std = 0.3
    names, arrs = ["embed"], [rng.normal(size=(V, d))]
    for l in range(sh.n_layers):
        names += [f"l{l}.attn_norm", f"l{l}.w_qkv", f"l{l}.w_o", f"l{l}.ffn_norm",
                  f"l{l}.w_gate_up", f"l{l}.w_down"]
        arrs += [1 + 0.3 * rng.normal(size=d), rng.normal(size=(qkv, d)) * std,
                 rng.normal(size=(d, sh.n_heads * sh.head_dim)) * std, 1 + 0.3 * rng.normal(size=d),
                 rng.normal(size=(2 * F, d)) * std, rng.normal(size=(d, F)) * std]
    names += ["final_norm", "lm_head"]
    arrs += [1 + 0.3 * rng.normal(size=d), rng.normal(size=(V, d)) * std]
    return names, arrs


def _hf_model(sh, names, arrs):
    """The library's decoder with the oracle's weights: w_qkv rows are q, then
    k, then v; w_gate_up rows are the gate, then up."""
    cfg = transformers.LlamaConfig(
        vocab_size=sh.vocab, hidden_size=sh.d_model, intermediate_size=sh.d_ffn,
        num_hidden_layers=sh.n_layers, num_attention_heads=sh.n_heads,
        num_key_value_heads=sh.n_kv_heads, head_dim=sh.head_dim, rms_norm_eps=sh.rms_eps,
        rope_theta=sh.rope_theta, max_position_embeddings=1024, tie_word_embeddings=False,
        attention_bias=False, mlp_bias=False, attn_implementation="eager")
    torch.manual_seed(0)
    m = transformers.LlamaForCausalLM(cfg).double().eval()
    w = dict(zip(names, arrs))
    Hq, Hkv, D, F = sh.n_heads, sh.n_kv_heads, sh.head_dim, sh.d_ffn
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))  # noqa: E731
    with torch.no_grad():
        m.model.embed_tokens.weight.copy_(t(w["embed"]))
        for l, layer in enumerate(m.model.layers):
            qkv = w[f"l{l}.w_qkv"]
            layer.input_layernorm.weight.copy_(t(w[f"l{l}.attn_norm"]))
            layer.self_attn.q_proj.weight.copy_(t(qkv[: Hq * D]))
            layer.self_attn.k_proj.weight.copy_(t(qkv[Hq * D: (Hq + Hkv) * D]))
            layer.self_attn.v_proj.weight.copy_(t(qkv[(Hq + Hkv) * D:]))
            layer.self_attn.o_proj.weight.copy_(t(w[f"l{l}.w_o"]))
            layer.post_attention_layernorm.weight.copy_(t(w[f"l{l}.ffn_norm"]))
            gu = w[f"l{l}.w_gate_up"]
            layer.mlp.gate_proj.weight.copy_(t(gu[:F]))
            layer.mlp.up_proj.weight.copy_(t(gu[F:]))
            layer.mlp.down_proj.weight.copy_(t(w[f"l{l}.w_down"]))
        m.model.norm.weight.copy_(t(w["final_norm"]))
        m.lm_head.weight.copy_(t(w["lm_head"]))
    return m


def _rel(a, b):
    return float(np.abs(a - b).max() / np.abs(b).max())


@pytest.mark.parametrize("Hkv", [2, 4])
def test_forward_from_empty_cache_matches_library_llama(Hkv):
    """A window from an empty cache (kv_len = 0): every row's logits agree with
    the library's decoder run over the same tokens (grouped-query and plain
    multi-head attention)."""
    sh = _shape(Hkv=Hkv)
    names, arrs = _weights(sh, seed=11 + Hkv)
    hf = _hf_model(sh, names, arrs)
    B, T = 2, 7
    toks = np.random.default_rng(1).integers(0, sh.vocab, size=(B, T))
    kc = np.zeros((sh.n_layers, B, sh.n_kv_heads, 16, sh.head_dim))
    vc = np.zeros((sh.n_layers, B, sh.n_kv_heads, sh.head_dim, 16))
    z, _, _ = M.forward(sh, M.Weights(names, arrs), toks, np.zeros(B, int), kc, vc)
    with torch.no_grad():
        ref = hf(torch.from_numpy(toks)).logits.numpy()
    assert _rel(z, ref) < 1e-6


def test_forward_over_a_cached_prefix_matches_library_llama():
    """A verify window over a non-empty cache: the library prefills a prompt,
    its cached (rotated) keys and values become the oracle's context cache,
    and the window's logits at positions kv_len .. kv_len + T - 1 agree with
    the library's cached decode of the same window.  The oracle's own
    suffix keys and values for the prompt agree with the library's cache."""
    sh = _shape()
    names, arrs = _weights(sh, seed=5)
    hf = _hf_model(sh, names, arrs)
    W = M.Weights(names, arrs)
    B, P, T, ctx = 2, 11, 5, 32
    rng = np.random.default_rng(2)
    prompt = rng.integers(0, sh.vocab, size=(B, P))
    window = rng.integers(0, sh.vocab, size=(B, T))
    with torch.no_grad():
        out = hf(torch.from_numpy(prompt), use_cache=True)
        cache = out.past_key_values
        ref = hf(torch.from_numpy(window), past_key_values=cache, use_cache=True).logits.numpy()
    kc = np.zeros((sh.n_layers, B, sh.n_kv_heads, ctx, sh.head_dim))
    vc = np.zeros((sh.n_layers, B, sh.n_kv_heads, sh.head_dim, ctx))
    kp = np.zeros((sh.n_layers, B, sh.n_kv_heads, P, sh.head_dim))
    vp = np.zeros_like(kp)
    for l in range(sh.n_layers):
        k_l, v_l = cache.layers[l].keys[:, :, :P].numpy(), cache.layers[l].values[:, :, :P].numpy()
        kp[l], vp[l] = k_l, v_l
        kc[l, :, :, :P, :] = k_l
        vc[l, :, :, :, :P] = np.swapaxes(v_l, 2, 3)
    z, _, _ = M.forward(sh, W, window, np.full(B, P), kc, vc)
    assert _rel(z, ref) < 1e-6
    # the oracle's prefill produces the keys / values the library cached
    kc0 = np.zeros_like(kc)
    vc0 = np.zeros_like(vc)
    zp, kn, vn = M.forward(sh, W, prompt, np.zeros(B, int), kc0, vc0)
    assert _rel(zp, out.logits.numpy()) < 1e-6
    assert _rel(np.swapaxes(kn, 2, 3), kp) < 1e-6
    assert _rel(np.swapaxes(vn, 2, 3), vp) < 1e-6

"""Pins of the oracle's decoder forward (oracle/model.py).

* building blocks against PyTorch's fp64 CPU library routines;
* the RoPE invariants (norm preserved, scores depend on relative position);
* the whole OPT-style and Qwen3-style forward against the transformers
  library's implementations of those architectures, run in fp64 with the
  oracle's weights.  That library computes attention softmax and RMSNorm in
  fp32 internally, so the bound is 1e-6 absolute on log-probs of size ~5,
  far below what a dropped term, a wrong sign or a transposed operand moves;
* the closed form log p = -ln V when the final norm's gain and bias are zero.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import model as om
from oracle.zo import Weights
from synth.configs import ModelCfg

torch.set_num_threads(4)
rs = np.random.default_rng(0)


def T(a):
    return torch.tensor(np.asarray(a), dtype=torch.float64)


def test_layer_norm_matches_library():
    x = rs.normal(size=(7, 48)) * 3 + 1
    w, b = rs.normal(size=48), rs.normal(size=48)
    ref = F.layer_norm(T(x), (48,), T(w), T(b), 1e-5).numpy()
    assert np.allclose(om.layer_norm(x, w, b, 1e-5), ref, rtol=1e-12, atol=1e-12)


def test_rms_norm_matches_definition_via_library():
    x = rs.normal(size=(5, 32)) * 2
    w = rs.normal(size=32)
    ref = (T(x) * torch.rsqrt(T(x).pow(2).mean(-1, keepdim=True) + 1e-6) * T(w)).numpy()
    ref2 = F.rms_norm(T(x), (32,), T(w), 1e-6).numpy()
    assert np.allclose(om.rms_norm(x, w, 1e-6), ref, rtol=1e-12, atol=1e-13)
    assert np.allclose(om.rms_norm(x, w, 1e-6), ref2, rtol=1e-12, atol=1e-13)


def test_gelu_silu_match_library():
    x = rs.normal(size=1000) * 4
    assert np.allclose(om.gelu(x), F.gelu(T(x)).numpy(), rtol=1e-13, atol=1e-15)
    assert np.allclose(om.silu(x), F.silu(T(x)).numpy(), rtol=1e-13, atol=1e-15)


def test_log_softmax_gather_matches_library():
    z = rs.normal(size=(9, 301)) * 5
    lab = rs.integers(0, 301, size=9)
    ref = F.log_softmax(T(z), -1).numpy()[np.arange(9), lab]
    assert np.allclose(om.log_softmax_gather(z, lab), ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2)])
def test_causal_attention_matches_library(hq, hkv):
    n, hd = 13, 16
    q, k, v = rs.normal(size=(n, hq, hd)), rs.normal(size=(n, hkv, hd)), rs.normal(size=(n, hkv, hd))
    rep = hq // hkv
    kt = T(k).repeat_interleave(rep, dim=1)
    vt = T(v).repeat_interleave(rep, dim=1)
    ref = F.scaled_dot_product_attention(T(q).transpose(0, 1), kt.transpose(0, 1), vt.transpose(0, 1),
                                         is_causal=True).transpose(0, 1).numpy()
    assert np.allclose(om.causal_attention(q, k, v), ref, rtol=1e-12, atol=1e-12)


def test_rope_invariants():
    n, H, hd = 11, 3, 16
    q, k = rs.normal(size=(n, H, hd)), rs.normal(size=(n, H, hd))
    pos = np.arange(n)
    qr = om.rope(q, pos, 1e6)
    assert np.allclose(np.linalg.norm(qr, axis=-1), np.linalg.norm(q, axis=-1), rtol=1e-13)
    # q.k after RoPE depends on the position difference only
    s1 = np.einsum("ihd,jhd->hij", om.rope(q, pos, 1e4), om.rope(k, pos, 1e4))
    s2 = np.einsum("ihd,jhd->hij", om.rope(q, pos + 37, 1e4), om.rope(k, pos + 37, 1e4))
    assert np.allclose(s1, s2, rtol=1e-10, atol=1e-10)
    # position 0 is the identity, and the pairing is rotate-half (i, i + hd/2)
    assert np.array_equal(om.rope(q[:1], np.zeros(1), 1e6), q[:1])
    x = np.zeros((1, 1, hd)); x[0, 0, 0] = 1.0
    y = om.rope(x, np.array([1]), 1e4)
    assert abs(y[0, 0, 0] - np.cos(1.0)) < 1e-15 and abs(y[0, 0, hd // 2] - np.sin(1.0)) < 1e-15


def _opt_hf(cfg, W):
    from transformers import OPTConfig, OPTForCausalLM
    c = OPTConfig(vocab_size=cfg.vocab, hidden_size=cfg.d_model, num_hidden_layers=cfg.n_layers,
                  ffn_dim=cfg.d_ffn, num_attention_heads=cfg.n_heads, max_position_embeddings=cfg.max_pos,
                  do_layer_norm_before=True, word_embed_proj_dim=cfg.d_model, activation_function="gelu",
                  enable_bias=True, dropout=0.0, attention_dropout=0.0, tie_word_embeddings=True,
                  pad_token_id=1, layer_norm_elementwise_affine=True)
    m = OPTForCausalLM(c).to(torch.float64).eval()
    m.config._attn_implementation = "eager"
    G, dec = W.get_global(), m.model.decoder
    with torch.no_grad():
        dec.embed_tokens.weight.copy_(T(G["tok_embed"]))
        dec.embed_positions.weight.zero_()
        dec.embed_positions.weight[2:2 + cfg.max_pos].copy_(T(G["pos_embed"]))   # the library's offset of 2
        dec.final_layer_norm.weight.copy_(T(G["final_norm_w"]))
        dec.final_layer_norm.bias.copy_(T(G["final_norm_b"]))
        for l in range(cfg.n_layers):
            Wl, L = W.get_layer(l), dec.layers[l]
            for mod, w, b in [(L.self_attn.q_proj, "wq", "bq"), (L.self_attn.k_proj, "wk", "bk"),
                              (L.self_attn.v_proj, "wv", "bv"), (L.self_attn.out_proj, "wo", "bo"),
                              (L.fc1, "w_fc1", "b_fc1"), (L.fc2, "w_fc2", "b_fc2"),
                              (L.self_attn_layer_norm, "ln1_w", "ln1_b"), (L.final_layer_norm, "ln2_w", "ln2_b")]:
                mod.weight.copy_(T(Wl[w]))
                mod.bias.copy_(T(Wl[b]))
    return m


def _qwen_hf(cfg, W):
    from transformers import Qwen3Config, Qwen3ForCausalLM
    c = Qwen3Config(vocab_size=cfg.vocab, hidden_size=cfg.d_model, intermediate_size=cfg.d_ffn,
                    num_hidden_layers=cfg.n_layers, num_attention_heads=cfg.n_heads,
                    num_key_value_heads=cfg.n_kv_heads, head_dim=cfg.head_dim, rms_norm_eps=cfg.norm_eps,
                    max_position_embeddings=cfg.max_pos, tie_word_embeddings=False, attention_bias=False,
                    use_sliding_window=False,
                    rope_parameters={"rope_type": "default", "rope_theta": cfg.rope_theta})
    m = Qwen3ForCausalLM(c).to(torch.float64).eval()
    m.config._attn_implementation = "eager"
    G, mm = W.get_global(), m.model
    with torch.no_grad():
        mm.embed_tokens.weight.copy_(T(G["tok_embed"]))
        mm.norm.weight.copy_(T(G["final_norm_w"]))
        m.lm_head.weight.copy_(T(G["lm_head"]))
        for l in range(cfg.n_layers):
            Wl, L = W.get_layer(l), mm.layers[l]
            for mod, w in [(L.self_attn.q_proj, "wq"), (L.self_attn.k_proj, "wk"), (L.self_attn.v_proj, "wv"),
                           (L.self_attn.o_proj, "wo"), (L.self_attn.q_norm, "q_norm_w"),
                           (L.self_attn.k_norm, "k_norm_w"), (L.input_layernorm, "ln1_w"),
                           (L.post_attention_layernorm, "ln2_w"), (L.mlp.gate_proj, "w_gate"),
                           (L.mlp.up_proj, "w_up"), (L.mlp.down_proj, "w_down")]:
                mod.weight.copy_(T(Wl[w]))
    return m


OPT_SMALL = ModelCfg("opt", 2, 64, 4, 4, 16, 128, 97, 64, "f32", 1e-5)
QWEN_SMALL = ModelCfg("qwen3", 2, 64, 4, 2, 16, 96, 101, 128, "f32", 1e-6, 1e6)


@pytest.mark.parametrize("cfg,build", [(OPT_SMALL, _opt_hf), (QWEN_SMALL, _qwen_hf),
                                       (OPT_SMALL.__class__(**{**OPT_SMALL.__dict__, "dtype": "bf16"}), _opt_hf)])
def test_forward_matches_library_architecture(cfg, build):
    W = Weights(cfg, 3, cache_layers=True)
    m = build(cfg, W)
    toks = rs.integers(0, cfg.vocab, size=19)
    with torch.no_grad():
        logits = m(input_ids=torch.tensor(toks)[None]).logits[0]
    ref = torch.log_softmax(logits, -1).numpy()[np.arange(len(toks) - 1), toks[1:]]
    seqs = [dict(tokens=toks, side=lambda l, k: [], positions=np.arange(len(toks) - 1), labels=toks[1:])]
    got = om.forward_logprobs(cfg, W.get_global, W.get_layer, seqs)[0]
    assert np.max(np.abs(got - ref)) < 1e-6


def test_zero_final_norm_gives_uniform():
    cfg = OPT_SMALL
    W = Weights(cfg, 1, cache_layers=True)
    G = W.get_global()
    G["final_norm_w"][:] = 0.0
    G["final_norm_b"][:] = 0.0
    toks = rs.integers(0, cfg.vocab, size=9)
    seqs = [dict(tokens=toks, side=lambda l, k: [], positions=np.arange(8), labels=toks[1:])]
    got = om.forward_logprobs(cfg, W.get_global, W.get_layer, seqs)[0]
    assert np.allclose(got, -np.log(cfg.vocab), rtol=0, atol=1e-14)

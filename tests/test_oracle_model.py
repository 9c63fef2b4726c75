"""Pins for the oracle's whole decode step: an independent library
implementation of the same decoder (transformers' Llama, run in float64),
closed forms that reduce the step to one matrix-vector product, structural
identities (GQA vs repeated-head MHA, tied vs untied head, prefill vs
sequential decode) and cache side effects.  CPU only, tiny shapes."""
import dataclasses

import numpy as np
import pytest
import torch

import synth

TINY = synth.CONFIGS["tiny"]


def shape_of(cfg):
    d = dataclasses.asdict(cfg)
    return {k: d[k] for k in ("n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim", "ffn", "vocab",
                              "rms_eps", "rope_theta", "dtype", "tied")}


def make(orc, cfg, weights, max_seq=None):
    return orc.Model(shape_of(cfg), weights, max_seq or cfg.max_seq)


def widen(orc, a):
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    return orc.f64_array_from_bf16(a)


def hf_logits(orc, cfg, weights, tokens):
    """Last-position logits of transformers' LlamaForCausalLM in float64."""
    from transformers import LlamaConfig, LlamaForCausalLM
    hc = LlamaConfig(vocab_size=cfg.vocab, hidden_size=cfg.hidden, intermediate_size=cfg.ffn,
                     num_hidden_layers=cfg.n_layers, num_attention_heads=cfg.n_heads,
                     num_key_value_heads=cfg.n_kv_heads, head_dim=cfg.head_dim, rms_norm_eps=cfg.rms_eps,
                     rope_theta=cfg.rope_theta, tie_word_embeddings=cfg.tied, attention_bias=False,
                     mlp_bias=False, max_position_embeddings=4096, hidden_act="silu")
    torch.manual_seed(0)
    m = LlamaForCausalLM(hc).double().eval()
    t = lambda a: torch.from_numpy(widen(orc, a))
    sd = {"model.embed_tokens.weight": t(weights["embed"]), "model.norm.weight": t(weights["final_norm"])}
    if not cfg.tied:
        sd["lm_head.weight"] = t(weights["lm_head"])
    names = {"attn_norm": "input_layernorm", "wq": "self_attn.q_proj", "wk": "self_attn.k_proj",
             "wv": "self_attn.v_proj", "wo": "self_attn.o_proj", "ffn_norm": "post_attention_layernorm",
             "w_gate": "mlp.gate_proj", "w_up": "mlp.up_proj", "w_down": "mlp.down_proj"}
    for l, lw in enumerate(weights["layers"]):
        for k, n in names.items():
            sd[f"model.layers.{l}.{n}.weight"] = t(lw[k])
    missing, unexpected = m.load_state_dict(sd, strict=False)
    assert not unexpected
    assert all("rotary" in k or (cfg.tied and k == "lm_head.weight") for k in missing), missing
    with torch.no_grad():
        out = m(input_ids=torch.tensor([list(tokens)]), use_cache=False)
    return out.logits[0, -1].numpy()


@pytest.mark.parametrize("tied", [False, True])
def test_matches_transformers_llama_fp32(orc, tied):
    cfg = TINY.with_(tied=tied)
    w = synth.gen_weights(cfg, seed=11, gains="random")
    toks = synth.gen_tokens(11, 12, cfg.vocab)
    m = make(orc, cfg, w)
    m.prefill(toks[:-1])
    got = m.decode_step(int(toks[-1]), len(toks) - 1)
    ref = hf_logits(orc, cfg, w, toks)
    # The oracle stores K/V as binary32 and the library keeps them in float64;
    # the library also computes RoPE angles in binary32.
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-6)
    assert np.abs(ref).max() > 0.1


def test_matches_transformers_llama_bf16_gqa(orc):
    # bf16 weights and cache, GQA group 4, head_dim 32; the oracle rounds
    # cached K/V to bf16 while the library does not, hence the looser bound.
    cfg = TINY.with_(dtype="bf16", n_heads=8, n_kv_heads=2, head_dim=32, rope_theta=500000.0, tied=True)
    w = synth.gen_weights(cfg, seed=12, gains="random")
    toks = synth.gen_tokens(12, 9, cfg.vocab)
    m = make(orc, cfg, w)
    m.prefill(toks[:-1])
    got = m.decode_step(int(toks[-1]), len(toks) - 1)
    ref = hf_logits(orc, cfg, w, toks)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-2)
    assert np.corrcoef(got, ref)[0, 1] > 0.9999


def test_gqa_equals_mha_with_repeated_kv_heads(orc):
    cfg = TINY.with_(n_layers=1)
    w = synth.gen_weights(cfg, seed=13, gains="random")
    g = cfg.n_heads // cfg.n_kv_heads
    d = cfg.head_dim
    mha_cfg = cfg.with_(n_kv_heads=cfg.n_heads)
    w2 = {k: v for k, v in w.items() if k != "layers"}
    w2["layers"] = []
    for lw in w["layers"]:
        lw2 = dict(lw)
        for key in ("wk", "wv"):
            heads = lw[key].reshape(cfg.n_kv_heads, d, cfg.hidden)
            lw2[key] = np.ascontiguousarray(np.repeat(heads, g, axis=0).reshape(-1, cfg.hidden))
        w2["layers"].append(lw2)
    toks = synth.gen_tokens(13, 6, cfg.vocab)
    a, b = make(orc, cfg, w), make(orc, mha_cfg, w2)
    a.prefill(toks[:-1])
    b.prefill(toks[:-1])
    np.testing.assert_allclose(a.decode_step(int(toks[-1]), 5), b.decode_step(int(toks[-1]), 5), rtol=0,
                               atol=1e-12)


def test_residual_only_model_reduces_to_one_gemv(orc):
    # Wo = 0 and Wd = 0: both residual branches add zero whatever the other
    # weights are, so logits = W_lm . rmsnorm(E[t], g_final).
    cfg = TINY
    w = synth.gen_weights(cfg, seed=14, gains="random")
    for lw in w["layers"]:
        lw["wo"][...] = 0
        lw["w_down"][...] = 0
    m = make(orc, cfg, w)
    m.prefill(synth.gen_tokens(14, 5, cfg.vocab))
    tok = 77
    x = widen(orc, w["embed"][tok])
    g = widen(orc, w["final_norm"])
    h = g * x / np.sqrt(np.mean(x * x) + cfg.rms_eps)
    np.testing.assert_allclose(m.decode_step(tok, 5), widen(orc, w["lm_head"]) @ h, rtol=1e-12, atol=1e-13)


def test_first_position_attention_returns_own_value(orc):
    # One layer, FFN off (Wd = 0), pos = 0: attention over one cached
    # position returns that position's stored V, whatever q and k are:
    # x1 = x0 + Wo . fp32(Wv . rmsnorm(x0)).
    cfg = TINY.with_(n_layers=1)
    w = synth.gen_weights(cfg, seed=15, gains="random")
    lw = w["layers"][0]
    lw["w_down"][...] = 0
    tok = 5
    x0 = widen(orc, w["embed"][tok])
    h = widen(orc, lw["attn_norm"]) * x0 / np.sqrt(np.mean(x0 * x0) + cfg.rms_eps)
    v = (widen(orc, lw["wv"]) @ h).astype(np.float32).astype(np.float64)  # stored as binary32
    o = np.concatenate([v.reshape(cfg.n_kv_heads, -1)[i // 2] for i in range(cfg.n_heads)])
    x1 = x0 + widen(orc, lw["wo"]) @ o
    hf = widen(orc, w["final_norm"]) * x1 / np.sqrt(np.mean(x1 * x1) + cfg.rms_eps)
    m = make(orc, cfg, w)
    np.testing.assert_allclose(m.decode_step(tok, 0), widen(orc, w["lm_head"]) @ hf, rtol=1e-11, atol=1e-12)


def test_tied_equals_untied_with_copied_head(orc):
    cfg = TINY.with_(n_layers=1, tied=True)
    w = synth.gen_weights(cfg, seed=16)
    w2 = dict(w)
    w2["lm_head"] = w["embed"].copy()
    toks = synth.gen_tokens(16, 4, cfg.vocab)
    a, b = make(orc, cfg, w), make(orc, cfg.with_(tied=False), w2)
    a.prefill(toks[:-1])
    b.prefill(toks[:-1])
    np.testing.assert_array_equal(a.decode_step(int(toks[-1]), 3), b.decode_step(int(toks[-1]), 3))


def test_prefill_equals_sequential_decodes_and_touches_only_its_positions(orc):
    cfg = TINY
    w = synth.gen_weights(cfg, seed=17)
    toks = synth.gen_tokens(17, 8, cfg.vocab)
    a, b = make(orc, cfg, w), make(orc, cfg, w)
    a.prefill(toks[:7])
    for i in range(7):
        b.decode_step(int(toks[i]), i, want_logits=False)
    np.testing.assert_array_equal(a.k, b.k)
    np.testing.assert_array_equal(a.v, b.v)
    assert not a.k[:, :, 7:].any() and not a.v[:, :, 7:].any()
    assert a.k[:, :, :7].all(axis=(0, 1, 3)).all()
    la = a.decode_step(int(toks[7]), 7)
    np.testing.assert_array_equal(la, b.decode_step(int(toks[7]), 7))
    assert a.k[:, :, 7].any() and not a.k[:, :, 8:].any()


def test_out_of_range_arguments_are_rejected(orc):
    cfg = TINY.with_(n_layers=1)
    m = make(orc, cfg, synth.gen_weights(cfg, seed=18))
    with pytest.raises(ValueError):
        m.decode_step(cfg.vocab, 0)
    with pytest.raises(ValueError):
        m.decode_step(-1, 0)
    with pytest.raises(ValueError):
        m.decode_step(0, cfg.max_seq)
    with pytest.raises(ValueError):
        m.prefill([1, 2, 3], start_pos=cfg.max_seq - 2)

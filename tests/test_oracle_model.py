"""The oracle decoder against an independent Llama-2 implementation (Hugging Face, float64)."""
import numpy as np
import pytest
import torch

import synth
from oracle import model as mdl
from oracle import ssd
from oracle.numerics import rmsnorm

GQA_SMALL = synth.ModelShape("gqa-small-f32", 2, 128, 4, 2, 32, 96, 100, "f32")
BF16_SMALL = synth.ModelShape("bf16-small", 3, 128, 4, 2, 32, 160, 300, "bf16")


def hf_model(m):
    from transformers import LlamaConfig, LlamaForCausalLM
    s = m.shape
    cfg = LlamaConfig(vocab_size=s.vocab, hidden_size=s.d_model, intermediate_size=s.ffn_dim,
                      num_hidden_layers=m.L, num_attention_heads=s.n_heads, num_key_value_heads=s.n_kv_heads,
                      head_dim=s.head_dim, max_position_embeddings=4096, rms_norm_eps=s.rms_eps,
                      rope_theta=s.rope_theta, tie_word_embeddings=False, attention_bias=False,
                      mlp_bias=False, attn_implementation="eager")
    hf = LlamaForCausalLM(cfg).double().eval()
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    with torch.no_grad():
        hf.model.embed_tokens.weight.copy_(T(m.embed))
        hf.lm_head.weight.copy_(T(m.lm_head))
        hf.model.norm.weight.copy_(T(m.final_norm))
        for l, lw in enumerate(m.layers):
            L = hf.model.layers[l]
            L.self_attn.q_proj.weight.copy_(T(lw.wq)); L.self_attn.k_proj.weight.copy_(T(lw.wk))
            L.self_attn.v_proj.weight.copy_(T(lw.wv)); L.self_attn.o_proj.weight.copy_(T(lw.wo))
            L.mlp.gate_proj.weight.copy_(T(lw.wgate)); L.mlp.up_proj.weight.copy_(T(lw.wup))
            L.mlp.down_proj.weight.copy_(T(lw.wdown))
            L.input_layernorm.weight.copy_(T(lw.attn_norm))
            L.post_attention_layernorm.weight.copy_(T(lw.mlp_norm))
    return hf


@pytest.mark.parametrize("shape", [synth.TINY, GQA_SMALL])
def test_decoder_matches_hf_llama(shape):
    m = mdl.Model.synthetic(shape)
    toks = synth.prompt_tokens(24, shape.vocab)
    kv = mdl.KVCache(shape, 64)
    z = mdl.forward(m, toks, range(24), kv)
    with torch.no_grad():
        ref = hf_model(m)(torch.from_numpy(toks.astype(np.int64))[None]).logits[0].numpy()
    # HF builds its RoPE table in float32; everything else is float64
    assert np.abs(z - ref).max() < 2e-6 * max(1.0, np.abs(ref).max())


def test_decoder_with_rounding_off_matches_hf():
    """The bf16 model with its storage rounding switched off is the same decoder."""
    m = mdl.Model.synthetic(BF16_SMALL)
    m32 = mdl.Model(shape=synth.ModelShape("x", 3, 128, 4, 2, 32, 160, 300, "f32"), embed=m.embed,
                    layers=m.layers, final_norm=m.final_norm, lm_head=m.lm_head)
    toks = synth.prompt_tokens(16, 300)
    z = mdl.forward(m32, toks, range(16), mdl.KVCache(m32.shape, 32))
    with torch.no_grad():
        ref = hf_model(m32)(torch.from_numpy(toks.astype(np.int64))[None]).logits[0].numpy()
    assert np.abs(z - ref).max() < 2e-6
    # and the rounded model stays within bf16 distance of it
    zb = mdl.forward(m, toks, range(16), mdl.KVCache(m.shape, 32))
    assert np.abs(zb - z).max() < 0.05 * np.abs(z).max()
    assert np.abs(zb - z).max() > 0


@pytest.mark.parametrize("shape", [synth.TINY, GQA_SMALL, BF16_SMALL])
def test_incremental_kv_equals_block_forward(shape):
    """Row-at-a-time decoding with the cache gives the block forward's logits."""
    m = mdl.Model.synthetic(shape)
    toks = synth.prompt_tokens(12, shape.vocab)
    z_block = mdl.forward(m, toks, range(12), mdl.KVCache(shape, 16))
    kv = mdl.KVCache(shape, 16)
    z_inc = np.concatenate([mdl.forward(m, toks[i:i + 1], [i], kv) for i in range(12)])
    assert np.abs(z_block - z_inc).max() < 1e-12


def test_skip_plan_semantics():
    """Skipping every sub-layer leaves the embedding; an exit plan equals a truncated model."""
    m = mdl.Model.synthetic(GQA_SMALL)
    toks = synth.prompt_tokens(5, GQA_SMALL.vocab)
    full_skip = synth.mask_exit(2, 0)
    z = mdl.forward(m, toks, range(5), mdl.KVCache(GQA_SMALL, 8), full_skip)
    ref = mdl.final_logits(m, mdl.embed(m, toks))
    assert np.array_equal(z, ref)
    trunc = mdl.Model(shape=synth.ModelShape("t", 1, 128, 4, 2, 32, 96, 100, "f32"), embed=m.embed,
                      layers=m.layers[:1], final_norm=m.final_norm, lm_head=m.lm_head)
    z1 = mdl.forward(m, toks, range(5), mdl.KVCache(GQA_SMALL, 8), synth.mask_exit(2, 1))
    z2 = mdl.forward(trunc, toks, range(5), mdl.KVCache(trunc.shape, 8))
    assert np.array_equal(z1, z2)
    assert mdl.first_skipped_layer(synth.mask_exit(2, 1), 2) == 1
    mlp_only = np.array([0, 0, 0, 1], np.uint8)
    assert mdl.first_skipped_layer(mlp_only, 2) == 1
    assert mdl.first_skipped_layer(None, 2) == 2


def test_attention_single_key_returns_value():
    """With one cached key the attention output is that key's value (softmax of one score is 1)."""
    m = mdl.Model.synthetic(GQA_SMALL)
    s = GQA_SMALL
    lw = m.layers[0]
    kv = mdl.KVCache(s, 4)
    h = mdl.embed(m, [5])
    out = mdl.attention_sublayer(m, 0, h, [0], kv)
    x = rmsnorm(h, lw.attn_norm, s.rms_eps)                # the textbook RMSNorm form
    v = (x @ lw.wv.T).reshape(s.n_kv_heads, s.head_dim)
    G = s.n_heads // s.n_kv_heads
    o = np.repeat(v, G, axis=0).reshape(-1)
    assert np.allclose(out, h + o @ lw.wo.T, atol=1e-14)

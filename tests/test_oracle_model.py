"""Pins of the oracle's forward pass.  The pages print no logits, so the
forward is pinned by (a) a library Llama (transformers) on the same weights
in the all-fp32 configuration, (b) library attention / norm routines,
(c) the property that makes verification work: row i of one pass equals the
distribution a one-token-at-a-time decode produces after the same inputs
[P1 "What one iteration actually does"; P2 "The Idea"], and (d) the shape
facts the first page prints (weight bytes, KV bytes per token)."""
import numpy as np
import pytest
import torch

from oracle import model as OM
from oracle.bf16 import round_bf16
from synth import SHAPES, Shape, make_prompt, make_weights
from tests._golden import load

TINY_GQA = Shape("tiny_gqa", 64, 2, 4, 2, 16, 96, 128, "f32")


def hf_llama(shape, w):
    from transformers import LlamaConfig, LlamaForCausalLM

    cfg = LlamaConfig(vocab_size=shape.vocab, hidden_size=shape.d_model, intermediate_size=shape.d_ff,
                      num_hidden_layers=shape.n_layers, num_attention_heads=shape.n_heads,
                      num_key_value_heads=shape.n_kv_heads, head_dim=shape.head_dim,
                      rms_norm_eps=shape.rms_eps, attention_bias=False, mlp_bias=False,
                      tie_word_embeddings=False, hidden_act="silu", max_position_embeddings=4096)
    cfg.rope_parameters = {"rope_theta": shape.rope_theta, "rope_type": "default"}
    cfg._attn_implementation = "eager"
    m = LlamaForCausalLM(cfg).to(torch.float64).eval()
    H, Hkv, hd, F = shape.n_heads, shape.n_kv_heads, shape.head_dim, shape.d_ff
    f = lambda t: t.detach().to(torch.float64)  # noqa: E731
    with torch.no_grad():
        m.model.embed_tokens.weight.copy_(f(w["embed"]))
        m.lm_head.weight.copy_(f(w["lm_head"]))
        m.model.norm.weight.copy_(f(w["final_norm"]))
        for i, layer in enumerate(m.model.layers):
            qkv = f(w["wqkv"][i])
            layer.self_attn.q_proj.weight.copy_(qkv[: H * hd])
            layer.self_attn.k_proj.weight.copy_(qkv[H * hd:(H + Hkv) * hd])
            layer.self_attn.v_proj.weight.copy_(qkv[(H + Hkv) * hd:])
            layer.self_attn.o_proj.weight.copy_(f(w["wo"][i]))
            gu = f(w["wgu"][i])
            layer.mlp.gate_proj.weight.copy_(gu[:F])
            layer.mlp.up_proj.weight.copy_(gu[F:])
            layer.mlp.down_proj.weight.copy_(f(w["wd"][i]))
            layer.input_layernorm.weight.copy_(f(w["attn_norm"][i]))
            layer.post_attention_layernorm.weight.copy_(f(w["mlp_norm"][i]))
    return m


@pytest.mark.parametrize("shape", [TINY_GQA, SHAPES["tiny"].with_(n_layers=2, vocab=512)])
def test_forward_matches_library_llama(shape):
    w = make_weights(shape, seed=7, norm="random", std=0.08)
    dec = OM.Decoder(shape, w)
    toks = make_prompt(2, 12, shape.vocab, seed=7)
    cache = dec.new_cache(2, 16)
    ours = dec.forward(cache, toks)
    with torch.no_grad():
        ref = hf_llama(shape, w)(torch.from_numpy(toks.astype(np.int64))).logits.numpy()
    # the library runs its norms and softmax in float32
    assert np.abs(ours - ref).max() < 1e-5 * max(1.0, np.abs(ref).max())


def test_verify_rows_equal_sequential_decode():
    """One pass over [t0 .. t4] at positions L..L+4 gives, row by row, the logits
    of feeding the same tokens one at a time."""
    for shape in (TINY_GQA, TINY_GQA.with_(dtype="bf16")):
        w = make_weights(shape, seed=11, norm="random", std=0.08)
        dec = OM.Decoder(shape, w)
        prompt = make_prompt(2, 9, shape.vocab, seed=11)
        block = make_prompt(2, 5, shape.vocab, seed=12)
        c1, c2 = dec.new_cache(2, 32), dec.new_cache(2, 32)
        for c in (c1, c2):
            dec.forward(c, prompt)
            c.length += prompt.shape[1]
        par = dec.forward(c1, block)
        seq = []
        for i in range(block.shape[1]):
            seq.append(dec.forward(c2, block[:, i:i + 1])[:, 0])
            c2.length += 1
        seq = np.stack(seq, 1)
        tol = 1e-10 if shape.dtype == "f32" else 1e-3
        assert np.abs(par - seq).max() < tol
        n = prompt.shape[1] + block.shape[1]
        assert np.abs(c1.k[:, :, :, :n] - c2.k[:, :, :, :n]).max() <= (1e-10 if shape.dtype == "f32" else 1e-2)


def test_rope_properties():
    rng = np.random.default_rng(3)
    x = rng.normal(size=(5, 3, 16))
    assert np.array_equal(OM.rope(x, np.zeros(5), 10000.0), x)
    y = OM.rope(x, np.arange(5) * 7.0, 10000.0)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)
    # scores depend only on the position difference
    q, k = rng.normal(size=(1, 16)), rng.normal(size=(1, 16))
    s1 = (OM.rope(q, np.array(10.0), 500.0) * OM.rope(k, np.array(3.0), 500.0)).sum()
    s2 = (OM.rope(q, np.array(107.0), 500.0) * OM.rope(k, np.array(100.0), 500.0)).sum()
    assert abs(s1 - s2) < 1e-10
    # lowest pair turns by exactly pos radians
    e = np.zeros((1, 16))
    e[0, 0] = 1.0
    r = OM.rope(e, np.array(0.3), 10000.0)
    assert np.allclose([r[0, 0], r[0, 8]], [np.cos(0.3), np.sin(0.3)], atol=1e-15)


def test_attention_matches_sdpa_and_one_key():
    rng = np.random.default_rng(4)
    H, Hkv, n, hd = 8, 2, 13, 16
    q = rng.normal(size=(H, hd))
    K = rng.normal(size=(Hkv, n, hd))
    V = rng.normal(size=(Hkv, n, hd))
    ours = OM.attend(q, K, V)
    G = H // Hkv
    tq = torch.from_numpy(q)[:, None, :]  # [H, 1, hd]
    tk = torch.from_numpy(K).repeat_interleave(G, dim=0)
    tv = torch.from_numpy(V).repeat_interleave(G, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[:, 0].numpy()
    assert np.abs(ours - ref).max() < 1e-12
    one = OM.attend(q, K[:, :1], V[:, :1])
    assert np.allclose(one, np.repeat(V[:, 0], G, axis=0), atol=1e-15)


def test_rms_norm_and_silu_match_torch():
    rng = np.random.default_rng(5)
    h, g = rng.normal(size=(4, 32)) * 3, rng.normal(size=32)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(h), (32,), torch.from_numpy(g), 1e-6).numpy()
    assert np.abs(OM.rms_norm(h, g, 1e-6) - ref).max() < 1e-12
    x = rng.normal(size=100) * 4
    assert np.abs(OM.silu(x) - torch.nn.functional.silu(torch.from_numpy(x)).numpy()).max() < 1e-14


def test_bf16_rounding_matches_library_cast():
    rng = np.random.default_rng(6)
    x = (rng.normal(size=200000) * np.exp(rng.normal(size=200000) * 4)).astype(np.float32)
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -100 * (1 + 2 ** -8), 0.0, -0.0], np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(round_bf16(x), ref)


def test_bf16_contract_points():
    """bf16 mode: cached K/V are bf16 values; logits stay close to the
    unrounded pass on the same weights but are not identical to it."""
    shape = TINY_GQA.with_(dtype="bf16")
    w = make_weights(shape, seed=13, norm="random", std=0.08)
    dec16 = OM.Decoder(shape, w)
    dec32 = OM.Decoder(shape.with_(dtype="f32"), w)
    toks = make_prompt(1, 10, shape.vocab, seed=13)
    c16, c32 = dec16.new_cache(1, 16), dec32.new_cache(1, 16)
    l16, l32 = dec16.forward(c16, toks), dec32.forward(c32, toks)
    assert np.array_equal(round_bf16(c16.k), c16.k) and np.array_equal(round_bf16(c16.v), c16.v)
    d = np.abs(l16 - l32).max()
    assert 0 < d < 0.05


def test_self_spec_prefix_is_early_layers():
    shape = TINY_GQA.with_(n_layers=3)
    w = make_weights(shape, seed=17, norm="random", std=0.08)
    toks = make_prompt(1, 6, shape.vocab, seed=17)
    d1 = OM.Decoder(shape, w, n_layers=1)
    w1 = {k: (v[:1] if k in ("attn_norm", "wqkv", "wo", "mlp_norm", "wgu", "wd") else v) for k, v in w.items()}
    d1b = OM.Decoder(shape.with_(n_layers=1), w1)
    assert np.array_equal(d1.forward(d1.new_cache(1, 8), toks), d1b.forward(d1b.new_cache(1, 8), toks))


def test_shape_facts_p1():
    g = load("p1_shapes.json")
    t, d = SHAPES["qwen3_8b"], SHAPES["qwen3_0p6b"]
    assert round(t.param_count() * 2 / 2 ** 30, 2) == g["target_weight_gib"]
    assert t.kv_bytes_per_token() == g["target_kv_kib_per_token"] * 1024
    assert d.kv_bytes_per_token() == g["draft_kv_kib_per_token"] * 1024
    assert round(100 * d.param_count() / t.param_count()) == g["draft_weight_share_pct"]
    assert round(100 * d.kv_bytes_per_token() / t.kv_bytes_per_token()) == g["draft_kv_share_pct"]

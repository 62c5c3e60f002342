"""Pins of oracle.decoder: Hugging Face transformers' LlamaModel (an
independent pre-norm RMSNorm / rotate-half RoPE / GQA / SwiGLU decoder) fed the
same weights in float64; torch's RMSNorm and SiLU; RoPE's complex form and
relative-position invariance; the transactional KV rules; bf16 handling."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import decoder as dec


def _hf_model(c, w):
    from transformers import LlamaConfig, LlamaModel
    cfg = LlamaConfig(
        vocab_size=c["vocab"], hidden_size=c["hidden"],
        intermediate_size=c["ffn"], num_hidden_layers=c["layers"],
        num_attention_heads=c["q_heads"], num_key_value_heads=c["kv_heads"],
        head_dim=c["head_dim"], rope_theta=float(np.float32(c["rope_theta"])),
        rms_norm_eps=float(np.float32(c["rms_eps"])), attention_bias=False,
        mlp_bias=False, max_position_embeddings=64)
    cfg._attn_implementation = "sdpa"
    m = LlamaModel(cfg).double().eval()
    conv = (lambda a: synth.bf16_to_f32(a)) if c["dtype"] == synth.BF16 \
        else (lambda a: a)
    sd = {}
    for i, lw in enumerate(w["layers"]):
        p = f"layers.{i}."
        sd[p + "input_layernorm.weight"] = lw["attn_norm"]
        sd[p + "post_attention_layernorm.weight"] = lw["ffn_norm"]
        sd[p + "self_attn.q_proj.weight"] = conv(lw["wq"])
        sd[p + "self_attn.k_proj.weight"] = conv(lw["wk"])
        sd[p + "self_attn.v_proj.weight"] = conv(lw["wv"])
        sd[p + "self_attn.o_proj.weight"] = conv(lw["wo"])
        sd[p + "mlp.gate_proj.weight"] = conv(lw["w_gate"])
        sd[p + "mlp.up_proj.weight"] = conv(lw["w_up"])
        sd[p + "mlp.down_proj.weight"] = conv(lw["w_down"])
    sd["norm.weight"] = w["final_norm"]
    sd = {k: torch.from_numpy(np.asarray(v, np.float64)) for k, v in sd.items()}
    missing, unexpected = m.load_state_dict(sd, strict=False)
    assert set(missing) == {"embed_tokens.weight"} and not unexpected
    # transformers evaluates its rotary cos/sin table in float32 on purpose;
    # evaluate the same table (inv_freq = theta^(-2i/d), angles duplicated
    # over both halves) in float64 so the comparison can be tight.
    rot = m.rotary_emb
    dim = c["head_dim"]
    inv = 1.0 / (float(np.float32(c["rope_theta"])) **
                 (torch.arange(0, dim, 2, dtype=torch.float64) / dim))

    def rotary64(x, position_ids):
        freqs = position_ids[:, :, None].double() * inv[None, None, :]
        emb = torch.cat((freqs, freqs), dim=-1)
        return emb.cos().to(x.dtype), emb.sin().to(x.dtype)

    rot.forward = rotary64
    # transformers' RMSNorm also upcasts to float32; use torch's own
    # rms_norm in float64 instead (pinned separately below)
    from transformers.models.llama.modeling_llama import LlamaRMSNorm
    for mod in m.modules():
        if isinstance(mod, LlamaRMSNorm):
            def norm64(x, mod=mod):
                return torch.nn.functional.rms_norm(
                    x, (x.shape[-1],), mod.weight, eps=mod.variance_epsilon)
            mod.forward = norm64
    return m


@pytest.mark.parametrize("c", [
    synth.custom(layers=2, hidden=32, q_heads=4, kv_heads=2, head_dim=8,
                 ffn=48, groups=6, vocab=16, weight_scale=0.2),
    synth.custom(layers=1, hidden=64, q_heads=4, kv_heads=1, head_dim=16,
                 ffn=96, groups=5, vocab=8, dtype=synth.BF16,
                 weight_scale=0.2, rope_theta=500.0, rms_eps=1e-5),
    synth.config("tiny"),
], ids=["gqa2", "mqa-bf16", "config1"])
def test_frame_matches_hf_llama(c):
    """All G positions of a frame, fed one at a time through the KV cache,
    equal LlamaModel's full-sequence causal forward (no cache)."""
    w = synth.make_weights(c)
    m = dec.Model(c, w)
    rng = np.random.default_rng(11)
    G = c["groups"]
    codes = rng.integers(0, c["vocab"], size=G)
    rows = [rng.standard_normal(c["hidden"])]
    rows += [m.embed_row(j - 1, int(codes[j - 1])) for j in range(1, G)]
    kv = m.new_kv()
    ours = np.stack(m.forward_rows(rows, list(range(G)), kv))
    hf = _hf_model(c, w)
    with torch.no_grad():
        ref = hf(inputs_embeds=torch.from_numpy(np.stack(rows))[None]
                 ).last_hidden_state[0].numpy()
    np.testing.assert_allclose(ours, ref, rtol=1e-10, atol=1e-10)


def test_rmsnorm_and_silu_match_torch():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(96)
    g = rng.standard_normal(96)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,),
                                       torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(dec.rmsnorm(x, g, 1e-6), ref, rtol=1e-13)
    ref = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    np.testing.assert_allclose(dec.silu(x), ref, rtol=1e-13)


def test_rope_complex_form_and_relative_position():
    rng = np.random.default_rng(3)
    d, theta = 16, 1e4
    q = rng.standard_normal((3, d))
    k = rng.standard_normal((3, d))
    np.testing.assert_array_equal(dec.rope(q, 0, theta), q)
    # pair (i, i + d/2) is the complex number q_i + 1j q_{i+d/2}, rotated by
    # pos * theta^(-2i/d)
    pos = 7
    zc = q[:, : d // 2] + 1j * q[:, d // 2:]
    ang = pos * theta ** (-np.arange(d // 2) * 2.0 / d)
    rot = zc * np.exp(1j * ang)
    np.testing.assert_allclose(dec.rope(q, pos, theta),
                               np.concatenate([rot.real, rot.imag], -1),
                               rtol=1e-12, atol=1e-12)
    # scores depend only on the position difference
    for m_, n_ in [(5, 2), (9, 6), (3, 0)]:
        a = np.sum(dec.rope(q, m_, theta) * dec.rope(k, n_, theta), -1)
        b = np.sum(dec.rope(q, m_ - n_, theta) * k, -1)
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    # norm preserved
    np.testing.assert_allclose(np.linalg.norm(dec.rope(q, 11, theta), axis=-1),
                               np.linalg.norm(q, axis=-1), rtol=1e-13)


def test_kv_transaction_rules():
    c = synth.custom()
    m = dec.Model(c, synth.make_weights(c))
    rng = np.random.default_rng(4)
    kv = m.new_kv()
    rows = [rng.standard_normal(c["hidden"]) for _ in range(4)]
    m.forward_rows(rows[:3], [0, 1, 2], kv)
    with pytest.raises(ValueError):
        m.forward_row(rows[3], 4, kv)          # must append at length 3
    kv.truncate(2)
    assert np.all(np.isnan(kv.k[:, 2:])) and np.all(np.isnan(kv.v[:, 2:]))
    assert not np.any(np.isnan(kv.k[:, :2]))
    with pytest.raises(ValueError):
        kv.truncate(3)
    out = m.forward_row(rows[3], 2, kv)
    assert np.all(np.isfinite(out))
    # the truncated-and-refilled cache equals a fresh prefill of the prefix
    kv2 = m.new_kv()
    ref = m.forward_rows([rows[0], rows[1], rows[3]], [0, 1, 2], kv2)[2]
    np.testing.assert_array_equal(out, ref)
    np.testing.assert_array_equal(kv.k[:, :3], kv2.k[:, :3])


def test_block_equals_single_steps():
    c = synth.custom(layers=2, q_heads=4, kv_heads=2, hidden=32, head_dim=8,
                     ffn=40, groups=6)
    m = dec.Model(c, synth.make_weights(c))
    rng = np.random.default_rng(5)
    rows = [rng.standard_normal(c["hidden"]) for _ in range(5)]
    kv_a, kv_b = m.new_kv(), m.new_kv()
    a = m.forward_rows(rows, range(5), kv_a)
    b = [m.forward_row(rows[0], 0, kv_b), m.forward_row(rows[1], 1, kv_b)]
    b += m.forward_rows(rows[2:], [2, 3, 4], kv_b)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_one_position_attention_returns_v():
    """With one position, softmax weight is 1: attention output = V."""
    c = synth.custom(layers=1, hidden=16, q_heads=2, kv_heads=2, head_dim=8)
    w = synth.make_weights(c)
    lw = w["layers"][0]
    lw["w_down"][:] = 0                          # isolate the attention half
    m = dec.Model(c, w)
    x = np.random.default_rng(6).standard_normal(16)
    kv = m.new_kv()
    out_pre = m.forward_row(x, 0, kv)
    n = dec.rmsnorm(x, 1.0, m.eps)
    v = lw["wv"].astype(np.float64) @ n
    expect = dec.rmsnorm(x + lw["wo"].astype(np.float64) @ v, 1.0, m.eps)
    np.testing.assert_allclose(out_pre, expect, rtol=1e-12)


def test_bf16_generator_and_conversion_match_torch():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(10000) * 0.02).astype(np.float32)
    bits = synth.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy()
    np.testing.assert_array_equal(bits.view(np.int16), ref)
    back = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float()
    np.testing.assert_array_equal(synth.bf16_to_f32(bits), back.numpy())


def test_heads_and_tables_index_by_depth():
    c = synth.custom(groups=5, vocab=6)
    w = synth.make_weights(c)
    m = dec.Model(c, w)
    h = np.random.default_rng(8).standard_normal(c["hidden"])
    for j in range(1, 5):
        np.testing.assert_array_equal(
            m.logits(j, h), (w["heads"][j - 1].astype(np.float64) @ h
                             ).astype(np.float32))
    with pytest.raises(IndexError):
        m.logits(0, h)
    with pytest.raises(IndexError):
        m.logits(5, h)
    np.testing.assert_array_equal(m.embed_row(3, 2), w["embed"][3, 2])
    assert math.isclose(m.eps, float(np.float32(1e-6)))

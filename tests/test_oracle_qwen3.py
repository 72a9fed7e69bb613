"""Pins of the Qwen3-ASR oracle (CPU only).

* full-prefix recompute == transformers' Qwen3 causal LM (independent library
  implementation: RMSNorm, per-head QK RMSNorm, NeoX RoPE, GQA, SwiGLU, tied
  head) in float64;
* cached step == full prefix; prefill (whole prompt at once, audio spliced) +
  steps == step-by-step from scratch with the audio rows fed as embeddings;
* GQA with each KV head duplicated over its group == plain multi-head
  attention with Hkv = Hq.
"""
import numpy as np
import pytest
import torch

from oracle import qwen3 as OQ

from .oracle_helpers import big_weights, tiny_qwen


def _setup(seed=0, **kw):
    w = tiny_qwen(**kw)
    W = big_weights(w, seed)
    rng = np.random.default_rng(seed + 7)
    ids = rng.integers(0, w.vocab, size=(w.batch, w.prefill_len + w.steps))
    audio = rng.standard_normal((w.batch, w.audio_rows, w.d))
    return w, W, ids, audio


def _hf_qwen(w, W):
    from transformers import Qwen3Config
    from transformers.models.qwen3.modeling_qwen3 import Qwen3ForCausalLM
    cfg = Qwen3Config(vocab_size=w.vocab, hidden_size=w.d, intermediate_size=w.d_ff,
                      num_hidden_layers=w.layers, num_attention_heads=w.heads,
                      num_key_value_heads=w.kv_heads, head_dim=w.head_dim, rms_norm_eps=w.eps,
                      rope_theta=w.rope_base, max_position_embeddings=w.context,
                      tie_word_embeddings=True, attention_bias=False, use_sliding_window=False)
    if getattr(cfg, "rope_parameters", None) is not None:
        cfg.rope_parameters = {"rope_type": "default", "rope_theta": w.rope_base}
    cfg._attn_implementation = "eager"
    m = Qwen3ForCausalLM(cfg).double().eval()
    sd = {"model.embed_tokens.weight": W["embed"], "model.norm.weight": W["norm_f.g"],
          "lm_head.weight": W["embed"]}
    for i in range(w.layers):
        p, h = f"dec.{i}.", f"model.layers.{i}."
        sd[h + "input_layernorm.weight"] = W[p + "norm1.g"]
        sd[h + "post_attention_layernorm.weight"] = W[p + "norm2.g"]
        for a, b in (("q", "q"), ("k", "k"), ("v", "v"), ("o", "o")):
            sd[h + f"self_attn.{b}_proj.weight"] = W[p + f"self.{a}.w"]
        sd[h + "self_attn.q_norm.weight"] = W[p + "q_norm.g"]
        sd[h + "self_attn.k_norm.weight"] = W[p + "k_norm.g"]
        for a in ("gate", "up", "down"):
            sd[h + f"mlp.{a}_proj.weight"] = W[p + f"mlp.{a}.w"]
    missing, unexpected = m.load_state_dict({k: torch.from_numpy(np.asarray(v, np.float64))
                                             for k, v in sd.items()}, strict=False)
    assert not unexpected and not missing, (missing, unexpected)
    inv = m.model.rotary_emb.inv_freq.double().numpy()
    i = np.arange(w.head_dim // 2)
    np.testing.assert_allclose(inv, (w.rope_base ** (-2.0 * i / w.head_dim)).astype(np.float32),
                               rtol=1e-6)
    return m


def test_full_prefix_matches_transformers_qwen3():
    # base 1e4 keeps float32 cos/sin error inside HF small at these positions
    w, W, ids, _ = _setup(1, rope_base=1e4)
    m = _hf_qwen(w, W)
    m.model.rotary_emb.inv_freq = m.model.rotary_emb.inv_freq.double()
    with torch.no_grad():
        ref = m(input_ids=torch.from_numpy(ids[:1]).long()).logits[0].numpy()
    got = OQ.decode_full(OQ.dims_of(w), W, ids[0])
    # HF evaluates cos/sin in float32; allow for that, far below any real error
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-5 * np.abs(ref).max())


@pytest.mark.parametrize("cache_dtype,rc", [("f32", False), ("f16", True)])
def test_cached_step_equals_full_prefix(cache_dtype, rc):
    w, W, ids, _ = _setup(2, cache_dtype=cache_dtype)
    D = OQ.dims_of(w)
    o = OQ.QwenOracle(D, W, round_cache=rc)
    o.reset(w.batch)
    S = 12
    cached = np.stack([o.step(ids[:, p], np.full(w.batch, p)) for p in range(S)], 1)
    assert np.all(np.isfinite(cached))
    for b in range(w.batch):
        full = OQ.decode_full(D, W, ids[b, :S], round_cache=rc)
        np.testing.assert_allclose(cached[b], full, rtol=0, atol=1e-10 * np.abs(full).max())


def test_prefill_with_audio_then_steps_equals_stepwise():
    w, W, ids, audio = _setup(3, cache_dtype="f16")
    D = OQ.dims_of(w)
    T, off, A = w.prefill_len, w.audio_offset, w.audio_rows
    a = OQ.QwenOracle(D, W)
    a.reset(w.batch)
    last = a.prefill(ids[:, :T], audio, off)
    b = OQ.QwenOracle(D, W)
    b.reset(w.batch)
    for t in range(T):
        emb = None
        if off <= t < off + A:
            emb = audio[:, t - off]
        lb = b.step(ids[:, t], np.full(w.batch, t), embeds=emb)
    np.testing.assert_allclose(last, lb, rtol=0, atol=1e-10 * np.abs(lb).max())
    for t in range(T, T + 3):
        la = a.step(ids[:, t], np.full(w.batch, t))
        lb = b.step(ids[:, t], np.full(w.batch, t))
        np.testing.assert_allclose(la, lb, rtol=0, atol=1e-10 * np.abs(lb).max())
    # and both equal the full-prefix recompute with the audio rows spliced
    full = OQ.decode_full(D, W, ids[0, :T + 3], round_cache=True, embeds=audio[0], offset=off)
    np.testing.assert_allclose(la[0], full[-1], rtol=0, atol=1e-10 * np.abs(full).max())


def test_gqa_with_duplicated_kv_equals_mha():
    w, W, ids, _ = _setup(4)
    g = w.heads // w.kv_heads
    wm = tiny_qwen(kv_heads=w.heads)
    Wm = dict(W)
    hd = w.head_dim
    for l in range(w.layers):
        for n in ("k", "v"):
            Wk = W[f"dec.{l}.self.{n}.w"].reshape(w.kv_heads, hd, w.d)
            Wm[f"dec.{l}.self.{n}.w"] = np.repeat(Wk, g, axis=0).reshape(w.heads * hd, w.d)
    a = OQ.decode_full(OQ.dims_of(w), W, ids[0, :9])
    b = OQ.decode_full(OQ.dims_of(wm), Wm, ids[0, :9])
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12 * np.abs(a).max())

"""Pins of the Whisper oracle (CPU only).

* cached step == full-prefix recompute (brute force, tiny dims), with and
  without cache rounding;
* full-prefix recompute == transformers' Whisper decoder (an independent
  library implementation of the same decoder) in float64;
* tied head == E @ h by an independent matmul;
* key bias: invariance in exact arithmetic (the pages claim otherwise), and the
  same vector as a query or value bias does change the output;
* batch independence, NaN-poisoned unwritten cache rows, reorder semantics.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import whisper as OW
from oracle.numerics import round_to_dtype

from .oracle_helpers import big_weights, tiny_whisper

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")


def _setup(seed=0, **kw):
    w = tiny_whisper(**kw)
    W = big_weights(w, seed)
    rng = np.random.default_rng(seed + 100)
    enc = rng.standard_normal((w.n_enc, w.frames, w.d))
    toks = rng.integers(0, w.vocab, size=(w.batch, w.steps))
    return w, W, enc, toks


def _run_cached(w, W, enc, toks, round_cache=True):
    o = OW.WhisperOracle(OW.dims_of(w), W, round_cache=round_cache)
    o.cross_kv(enc)
    o.reset(w.batch, enc_of=np.arange(w.batch) % w.n_enc)
    out = []
    for p in range(toks.shape[1]):
        out.append(o.step(toks[:, p], np.full(w.batch, p)))
    return np.stack(out, 1)   # [B, S, V]


@pytest.mark.parametrize("cache_dtype,round_cache", [("f32", False), ("f16", True), ("bf16", True)])
def test_cached_step_equals_full_prefix(cache_dtype, round_cache):
    w, W, enc, toks = _setup(1, cache_dtype=cache_dtype)
    cached = _run_cached(w, W, enc, toks, round_cache)
    assert np.all(np.isfinite(cached))          # never read a NaN (unwritten) row
    D = OW.dims_of(w)
    for b in range(w.batch):
        full = OW.decode_full(D, W, toks[b], enc[b % w.n_enc], round_cache=round_cache)
        np.testing.assert_allclose(cached[b], full, rtol=0, atol=1e-10 * np.abs(full).max())


def test_context_edge_full_length():
    w, W, enc, toks = _setup(2, steps=12, context=12)
    cached = _run_cached(w, W, enc, toks, False)
    full = OW.decode_full(OW.dims_of(w), W, toks[0], enc[0])
    np.testing.assert_allclose(cached[0], full, rtol=0, atol=1e-10 * np.abs(full).max())


def _hf_decoder(w, W):
    from transformers import WhisperConfig
    from transformers.models.whisper.modeling_whisper import WhisperDecoder
    cfg = WhisperConfig(vocab_size=w.vocab, d_model=w.d, decoder_attention_heads=w.heads,
                        decoder_layers=w.layers, decoder_ffn_dim=w.d_ff,
                        encoder_attention_heads=w.heads, encoder_layers=1, encoder_ffn_dim=w.d_ff,
                        max_target_positions=w.context, max_source_positions=w.frames,
                        activation_function="gelu", dropout=0.0, attention_dropout=0.0,
                        activation_dropout=0.0, pad_token_id=0)
    cfg._attn_implementation = "eager"
    dec = WhisperDecoder(cfg).double().eval()
    sd = {"embed_tokens.weight": W["embed"], "embed_positions.weight": W["pos"],
          "layer_norm.weight": W["ln_f.g"], "layer_norm.bias": W["ln_f.b"]}
    for i in range(w.layers):
        p, h = f"dec.{i}.", f"layers.{i}."
        for mine, theirs in (("self", "self_attn"), ("cross", "encoder_attn")):
            for proj, hp in (("q", "q_proj"), ("k", "k_proj"), ("v", "v_proj"), ("o", "out_proj")):
                sd[h + f"{theirs}.{hp}.weight"] = W[p + f"{mine}.{proj}.w"]
                if proj != "k":
                    sd[h + f"{theirs}.{hp}.bias"] = W[p + f"{mine}.{proj}.b"]
        for ln, hl in (("ln1", "self_attn_layer_norm"), ("ln2", "encoder_attn_layer_norm"),
                       ("ln3", "final_layer_norm")):
            sd[h + f"{hl}.weight"] = W[p + ln + ".g"]
            sd[h + f"{hl}.bias"] = W[p + ln + ".b"]
        for fc in ("fc1", "fc2"):
            sd[h + f"{fc}.weight"] = W[p + fc + ".w"]
            sd[h + f"{fc}.bias"] = W[p + fc + ".b"]
    missing, unexpected = dec.load_state_dict({k: torch.from_numpy(np.asarray(v, np.float64))
                                               for k, v in sd.items()}, strict=False)
    assert not unexpected, unexpected
    # the only parameters left unset must be the (absent) key biases: HF has none either
    assert not [m for m in missing if "k_proj" not in m], missing
    return dec


def test_full_prefix_matches_transformers_whisper_decoder():
    w, W, enc, toks = _setup(3)
    dec = _hf_decoder(w, W)
    with torch.no_grad():
        h = dec(input_ids=torch.from_numpy(toks[:1]).long(),
                encoder_hidden_states=torch.from_numpy(enc[:1])).last_hidden_state[0].numpy()
    ref = h @ W["embed"].T
    got = OW.decode_full(OW.dims_of(w), W, toks[0], enc[0])
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-10 * np.abs(ref).max())


def test_tied_head_equals_embed_times_hidden():
    w, W, enc, toks = _setup(4)
    o = OW.WhisperOracle(OW.dims_of(w), W)
    o.cross_kv(enc)
    o.reset(w.batch, enc_of=np.arange(w.batch) % w.n_enc)
    logits, h = o.step(toks[:, 0], np.zeros(w.batch, int), return_hidden=True)
    ref = torch.matmul(torch.from_numpy(h), torch.from_numpy(W["embed"]).T).numpy()
    np.testing.assert_allclose(logits, ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_key_bias_is_softmax_invariant_but_query_and_value_bias_are_not():
    """The pages assert that a key bias would matter because a softmax does not
    ignore it.  In exact arithmetic it cannot: q.(k_j + b) = q.k_j + q.b shifts
    every score of one query by the same amount.  This test records the truth:
    adding a key bias leaves the logits unchanged to rounding, while the same
    vector as a query or value bias, or the fused cross bias placed on the K half
    instead of the V half, changes them by orders of magnitude more.  The
    asymmetry matters for where the bias goes, not for its absence on keys."""
    w, W, enc, toks = _setup(5)
    D = OW.dims_of(w)
    rng = np.random.default_rng(55)
    bias = {f"dec.{l}.{s}": 3.0 * rng.standard_normal(w.d) for l in range(w.layers)
            for s in ("self", "cross")}
    base = OW.decode_full(D, W, toks[0], enc[0])
    kb = OW.decode_full(D, W, toks[0], enc[0], key_bias=bias)
    scale = np.abs(base).max()
    assert np.abs(kb - base).max() <= 1e-12 * scale * 10
    W2 = dict(W)
    for l in range(w.layers):
        W2[f"dec.{l}.self.q.b"] = W[f"dec.{l}.self.q.b"] + bias[f"dec.{l}.self"]
    assert np.abs(OW.decode_full(D, W2, toks[0], enc[0]) - base).max() > 1e-3 * scale
    W3 = dict(W)
    for l in range(w.layers):
        W3[f"dec.{l}.self.v.b"] = W[f"dec.{l}.self.v.b"] + bias[f"dec.{l}.self"]
    assert np.abs(OW.decode_full(D, W3, toks[0], enc[0]) - base).max() > 1e-3 * scale
    # fused cross bias [b_v | 0] instead of [0 | b_v]: bias on keys, none on values
    W4 = dict(W)
    kbias = {}
    for l in range(w.layers):
        kbias[f"dec.{l}.cross"] = W[f"dec.{l}.cross.v.b"]
        W4[f"dec.{l}.cross.v.b"] = np.zeros(w.d)
    assert np.abs(OW.decode_full(D, W4, toks[0], enc[0], key_bias=kbias) - base).max() > 1e-3 * scale
    # the oracle refuses a key-bias tensor outright
    with pytest.raises(ValueError):
        OW.WhisperOracle(D, dict(W, **{"dec.0.self.k.b": np.zeros(w.d)}))


def test_key_bias_absent_from_page_bindings_and_workload_names():
    facts = json.load(open(GOLDEN))["bindings_layer0_attention"]
    assert any(n.endswith("q_proj.bias") for n in facts["present"])
    assert any(n.endswith("v_proj.bias") for n in facts["present"])
    assert all(n.endswith("k_proj.bias") for n in facts["absent"])
    import workloads as WL
    for wl in WL.WORKLOADS:
        names = [n for n, _, _ in WL.weight_specs(wl)]
        assert not [n for n in names if n.endswith(".k.b")]
        if wl.arch == "whisper":
            assert "dec.0.self.q.b" in names and "dec.0.self.v.b" in names
            assert "dec.0.cross.v.b" in names


def test_batch_rows_are_independent():
    w, W, enc, toks = _setup(6)
    allb = _run_cached(w, W, enc, toks)
    for b in range(w.batch):
        o = OW.WhisperOracle(OW.dims_of(w), W)
        o.cross_kv(enc[b % w.n_enc][None])
        o.reset(1)
        alone = np.stack([o.step(toks[b:b + 1, p], [p])[0] for p in range(w.steps)], 0)
        np.testing.assert_allclose(allb[b], alone, rtol=0, atol=1e-12 * np.abs(alone).max())


def test_ragged_window_rows_equal_their_set_alone():
    """Sets of different lengths in one window: every row equals a full-prefix
    recompute (brute force) over its own set's frames only."""
    w, W, enc, toks = _setup(11)
    lens = [w.frames, 3, 1]
    o = OW.WhisperOracle(OW.dims_of(w), W)
    o.cross_kv([enc[e, :lens[e]] for e in range(w.n_enc)])
    o.reset(w.batch, enc_of=np.arange(w.batch) % w.n_enc)
    got = np.stack([o.step(toks[:, p], np.full(w.batch, p)) for p in range(w.steps)], 1)
    for b in range(w.batch):
        e = b % w.n_enc
        ref = OW.decode_full(OW.dims_of(w), W, toks[b], enc[e, :lens[e]], round_cache=True)
        np.testing.assert_allclose(got[b], ref, rtol=0, atol=1e-9 * np.abs(ref).max())
    # and a set cut to fewer frames really changes its rows
    full = _run_cached(w, W, enc, toks)
    assert np.abs(full[1] - got[1]).max() > 1e-3 and np.abs(full[2] - got[2]).max() > 1e-3


def test_cross_kv_once_equals_recompute_and_rounds_to_cache_dtype():
    w, W, enc, toks = _setup(7, cache_dtype="f16")
    o = OW.WhisperOracle(OW.dims_of(w), W)
    o.cross_kv(enc)
    for l in range(w.layers):
        k = enc @ W[f"dec.{l}.cross.k.w"].T
        np.testing.assert_array_equal(o.Kc[l], round_to_dtype(k, "f16"))
        assert np.all(o.Kc[l].astype(np.float16).astype(np.float64) == o.Kc[l])


def test_reorder_semantics():
    w, W, enc, toks = _setup(8, n_enc=1, batch=4)
    o = OW.WhisperOracle(OW.dims_of(w), W)
    o.cross_kv(enc)
    o.reset(4)
    for p in range(3):
        o.step(toks[:, p], np.full(4, p))
    K0 = [k.copy() for k in o.Ks]
    o.reorder([0, 1, 2, 3])                              # identity: untouched
    for a, b in zip(K0, o.Ks):
        np.testing.assert_array_equal(a, b)
    perm = np.array([2, 0, 3, 1])
    o.reorder(perm)
    for a, b in zip(K0, o.Ks):
        np.testing.assert_array_equal(a[perm], b)
    o.reorder(np.argsort(perm))                          # inverse restores
    for a, b in zip(K0, o.Ks):
        np.testing.assert_array_equal(a, b)
    Kc0 = [k.copy() for k in o.Kc]
    o.reorder([1, 1, 0, 0])
    for a, b in zip(Kc0, o.Kc):                          # broadcast cross cache untouched
        np.testing.assert_array_equal(a, b)

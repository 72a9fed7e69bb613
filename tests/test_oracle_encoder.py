"""Pins of the audio-encoder oracle (CPU only).

* the convolution equals torch's conv1d (an independent library routine) in float64, at
  both strides and odd and even lengths;
* the whole encoder equals transformers' Whisper encoder (an independent implementation of
  the same model) in float64, with the same weights and position table;
* 3000 mel frames give 1500 positions on real tensors, as (Frames - 1) / 2 + 1 states;
* a key bias is rejected, as in the decoder.
"""
import numpy as np
import pytest
import torch

from oracle import encoder as OE


def _weights(d=16, mels=6, heads=2, layers=2, d_ff=32, positions=10, seed=0):
    rng = np.random.default_rng(seed)
    s = lambda *shape: rng.standard_normal(shape) * (0.9 / np.sqrt(shape[-1] if len(shape) > 1 else 1))
    W = {"enc.conv1.w": rng.standard_normal((d, mels, 3)) * 0.4, "enc.conv1.b": 0.3 * rng.standard_normal(d),
         "enc.conv2.w": rng.standard_normal((d, d, 3)) * 0.2, "enc.conv2.b": 0.3 * rng.standard_normal(d),
         "enc.pos": rng.standard_normal((positions, d)),
         "enc.ln_post.g": 1 + 0.2 * rng.standard_normal(d), "enc.ln_post.b": 0.3 * rng.standard_normal(d)}
    for i in range(layers):
        p = f"enc.{i}."
        for ln in ("ln1", "ln2"):
            W[p + ln + ".g"] = 1 + 0.2 * rng.standard_normal(d)
            W[p + ln + ".b"] = 0.3 * rng.standard_normal(d)
        for proj in ("q", "k", "v", "o"):
            W[p + f"attn.{proj}.w"] = s(d, d) * 3
            if proj != "k":
                W[p + f"attn.{proj}.b"] = 0.3 * rng.standard_normal(d)
        W[p + "fc1.w"] = s(d_ff, d) * 3
        W[p + "fc1.b"] = 0.3 * rng.standard_normal(d_ff)
        W[p + "fc2.w"] = s(d, d_ff) * 3
        W[p + "fc2.b"] = 0.3 * rng.standard_normal(d)
    return W


@pytest.mark.parametrize("L,stride", [(7, 1), (7, 2), (10, 1), (10, 2), (3000, 2)])
def test_conv1d_equals_torch_conv1d(L, stride):
    rng = np.random.default_rng(L + stride)
    x = rng.standard_normal((L, 5))
    w = rng.standard_normal((4, 5, 3))
    b = rng.standard_normal(4)
    got = OE.conv1d(x, w, b, stride, 1)
    ref = torch.nn.functional.conv1d(torch.from_numpy(x.T[None]), torch.from_numpy(w), torch.from_numpy(b),
                                     stride=stride, padding=1)[0].numpy().T
    assert got.shape == ref.shape == ((L - 1) // stride + 1, 4)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_encoder_equals_transformers_whisper_encoder():
    from transformers import WhisperConfig
    from transformers.models.whisper.modeling_whisper import WhisperEncoder
    d, mels, heads, layers, d_ff, P = 16, 6, 2, 2, 32, 10
    W = _weights(d, mels, heads, layers, d_ff, P, seed=3)
    cfg = WhisperConfig(d_model=d, num_mel_bins=mels, encoder_attention_heads=heads, encoder_layers=layers,
                        encoder_ffn_dim=d_ff, decoder_attention_heads=heads, decoder_layers=1,
                        decoder_ffn_dim=d_ff, max_source_positions=P, activation_function="gelu",
                        dropout=0.0, attention_dropout=0.0, activation_dropout=0.0)
    cfg._attn_implementation = "eager"
    enc = WhisperEncoder(cfg).double().eval()
    sd = {"conv1.weight": W["enc.conv1.w"], "conv1.bias": W["enc.conv1.b"],
          "conv2.weight": W["enc.conv2.w"], "conv2.bias": W["enc.conv2.b"],
          "embed_positions.weight": W["enc.pos"],
          "layer_norm.weight": W["enc.ln_post.g"], "layer_norm.bias": W["enc.ln_post.b"]}
    for i in range(layers):
        p, h = f"enc.{i}.", f"layers.{i}."
        for proj, hp in (("q", "q_proj"), ("k", "k_proj"), ("v", "v_proj"), ("o", "out_proj")):
            sd[h + f"self_attn.{hp}.weight"] = W[p + f"attn.{proj}.w"]
            if proj != "k":
                sd[h + f"self_attn.{hp}.bias"] = W[p + f"attn.{proj}.b"]
        for ln, hl in (("ln1", "self_attn_layer_norm"), ("ln2", "final_layer_norm")):
            sd[h + f"{hl}.weight"] = W[p + ln + ".g"]
            sd[h + f"{hl}.bias"] = W[p + ln + ".b"]
        for fc in ("fc1", "fc2"):
            sd[h + f"{fc}.weight"] = W[p + fc + ".w"]
            sd[h + f"{fc}.bias"] = W[p + fc + ".b"]
    missing, unexpected = enc.load_state_dict({k: torch.from_numpy(np.asarray(v, np.float64))
                                               for k, v in sd.items()}, strict=False)
    assert not unexpected, unexpected
    assert not [m for m in missing if "k_proj" not in m], missing
    mel = np.random.default_rng(4).standard_normal((2 * P, mels))   # the frames HF expects: 2 x positions
    with torch.no_grad():
        ref = enc(torch.from_numpy(mel.T[None].copy())).last_hidden_state[0].numpy()
    got = OE.encode(W, mel, heads, layers)
    assert got.shape == ref.shape == (P, d)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-10 * np.abs(ref).max())
    # a small change of one term moves the result far above that tolerance (one channel: a
    # shift of every channel alike would vanish in the final LayerNorm)
    W2 = dict(W)
    W2["enc.1.fc2.b"] = W["enc.1.fc2.b"] + 1e-3 * (np.arange(d) == 0)
    assert np.abs(OE.encode(W2, mel, heads, layers) - got).max() > 1e-6


def test_3000_mel_frames_give_1500_states():
    W = _weights(d=8, mels=4, heads=2, layers=1, d_ff=16, positions=1500, seed=5)
    mel = np.random.default_rng(6).standard_normal((3000, 4))
    out = OE.encode(W, mel, heads=2, layers=1)
    assert out.shape == (1500, 8) and np.all(np.isfinite(out))


def test_encoder_key_bias_rejected():
    W = _weights()
    W["enc.0.attn.k.b"] = np.zeros(16)
    with pytest.raises(ValueError):
        OE.encode(W, np.zeros((20, 6)), heads=2, layers=2)

"""Pins of the oracle's numerics against library routines, closed forms and
brute force.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import numerics as N

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")


def _edge_values(rng, n=20000):
    mags = np.exp(rng.uniform(np.log(1e-9), np.log(7e4), n))
    return np.concatenate([mags * rng.choice([-1, 1], n),
                           [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 1e5, 6e-8, 3e-8]])


def test_round_f16_matches_numpy_half():
    rng = np.random.default_rng(0)
    x = _edge_values(rng)
    # exact ties between two f16 neighbours (round half to even)
    h = rng.standard_normal(5000).astype(np.float16).astype(np.float64)
    ulp = np.spacing(np.abs(h).astype(np.float16)).astype(np.float64)
    x = np.concatenate([x, h + ulp / 2, h - ulp / 2])
    ref = x.astype(np.float16).astype(np.float64)     # numpy's direct double->half
    got = N.round_to_dtype(x, "f16")
    np.testing.assert_array_equal(got, ref)


def test_round_bf16_matches_torch_bfloat16():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [0.0, 1.0, -1.0, 1e-39, 3e38, 3.4e38, 1e-45]]).astype(np.float32)
    # exact ties: a bf16 value plus half its spacing, representable in fp32
    b = torch.from_numpy(rng.standard_normal(5000).astype(np.float32)).to(torch.bfloat16)
    bb = b.to(torch.float32).numpy().view(np.uint32)
    ties = np.concatenate([(bb + 0x8000).view(np.float32), (bb + 0x18000).view(np.float32)])
    x = np.concatenate([x, ties]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = N.round_to_dtype(x.astype(np.float64), "bf16")
    np.testing.assert_array_equal(got, ref)


def test_round_f32_identity_on_f32_values():
    x = np.random.default_rng(2).standard_normal(1000).astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(N.round_to_dtype(x, "f32"), x)


def test_layer_norm_matches_torch():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((7, 96)) * 3 + 1.5
    g = 1 + 0.1 * rng.standard_normal(96)
    b = 0.1 * rng.standard_normal(96)
    ref = F.layer_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), torch.from_numpy(b), 1e-5)
    np.testing.assert_allclose(N.layer_norm(x, g, b, 1e-5), ref.numpy(), rtol=0, atol=1e-12)


def test_rms_norm_matches_torch():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 128)) * 2 + 0.3
    g = 1 + 0.1 * rng.standard_normal(128)
    ref = F.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(g), 1e-6)
    np.testing.assert_allclose(N.rms_norm(x, g, 1e-6), ref.numpy(), rtol=0, atol=1e-12)


def test_gelu_erf_matches_torch_and_math_erf():
    x = np.linspace(-8, 8, 2001)
    ref = F.gelu(torch.from_numpy(x), approximate="none").numpy()
    np.testing.assert_allclose(N.gelu_erf(x), ref, rtol=0, atol=1e-14)
    ref2 = np.array([v * (1 + math.erf(v / math.sqrt(2))) / 2 for v in x[::50]])
    np.testing.assert_allclose(N.gelu_erf(x[::50]), ref2, rtol=0, atol=1e-14)
    # not the tanh form: they differ by ~1e-3 near |x| ~ 2
    tanh = F.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    assert np.max(np.abs(tanh - N.gelu_erf(x))) > 1e-4


def test_silu_matches_torch():
    x = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(N.silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=0, atol=1e-14)


def test_softmax_rows_sum_to_one_and_mask_zero():
    rng = np.random.default_rng(5)
    S = 37
    s = rng.standard_normal((4, S, S)) * 6
    mask = np.where(np.arange(S)[None, :] <= np.arange(S)[:, None], 0.0, -np.inf)
    a = N.softmax(s + mask, -1)
    np.testing.assert_allclose(a.sum(-1), 1.0, rtol=0, atol=1e-12)
    assert np.all(a[:, np.triu_indices(S, 1)[0], np.triu_indices(S, 1)[1]] == 0.0)
    ref = torch.softmax(torch.from_numpy(s + mask), -1).numpy()
    np.testing.assert_allclose(a, ref, rtol=0, atol=1e-14)
    np.testing.assert_allclose(N.log_softmax(s, -1), torch.log_softmax(torch.from_numpy(s), -1).numpy(),
                               rtol=0, atol=1e-12)
    # shift invariance that the key-bias argument rests on
    np.testing.assert_allclose(N.softmax(s + 3.7, -1), N.softmax(s, -1), rtol=0, atol=1e-14)


def _hf_rope(z, pos, base):
    """NeoX RoPE as transformers' Qwen3 implementation applies it."""
    from transformers import Qwen3Config
    from transformers.models.qwen3.modeling_qwen3 import Qwen3RotaryEmbedding, apply_rotary_pos_emb
    hd = z.shape[-1]
    cfg = Qwen3Config(hidden_size=hd * 2, num_attention_heads=2, num_key_value_heads=1, head_dim=hd,
                      max_position_embeddings=4096, rope_theta=base)
    if getattr(cfg, "rope_parameters", None) is not None:
        cfg.rope_parameters = {"rope_type": "default", "rope_theta": base}
    rot = Qwen3RotaryEmbedding(cfg)
    t = torch.from_numpy(z)[None, :, None, :].double()        # [1, n, 1, hd] -> heads axis
    t = t.transpose(1, 2)                                     # [1, 1, n, hd]
    p = torch.from_numpy(np.asarray(pos))[None, :]
    cos, sin = rot(t.float(), p)
    qe, _ = apply_rotary_pos_emb(t, t, cos.double(), sin.double())
    return qe[0, 0].numpy(), rot.inv_freq.double().numpy()


def test_rope_matches_transformers_and_invariants():
    rng = np.random.default_rng(6)
    hd, base = 128, 1e6
    z = rng.standard_normal((9, hd))
    pos = np.array([0, 1, 2, 7, 100, 511, 900, 1023, 3000])
    got = N.rope_neox(z, pos, base)
    ref, inv = _hf_rope(z, pos, base)
    # transformers builds inv_freq in float32 and cos/sin in float32: compare loosely,
    # then pin the frequencies exactly against its inv_freq (rounded to f32)
    np.testing.assert_allclose(got, ref, rtol=0, atol=2e-3 * np.abs(z).max())
    i = np.arange(hd // 2)
    np.testing.assert_allclose((base ** (-2.0 * i / hd)).astype(np.float32), inv.astype(np.float32),
                               rtol=1e-6)
    # invariants: norm preserved, position 0 is the identity, scores depend on m - n
    np.testing.assert_allclose(np.linalg.norm(got, axis=-1), np.linalg.norm(z, axis=-1), rtol=1e-13)
    np.testing.assert_allclose(N.rope_neox(z, np.zeros(9), base), z, rtol=0, atol=0)
    q, k = rng.standard_normal(hd), rng.standard_normal(hd)
    d1 = N.rope_neox(q, 40, base) @ N.rope_neox(k, 13, base)
    d2 = N.rope_neox(q, 927, base) @ N.rope_neox(k, 900, base)
    assert abs(d1 - d2) < 1e-10


def test_conv_output_length_closed_form_and_brute_force():
    facts = json.load(open(GOLDEN))["conv_stem"]
    assert N.conv_out_len(facts["mel_frames"], facts["kernel"], facts["stride"], facts["pad"]) == \
        facts["encoder_positions"]
    for f in range(1, 4001):
        # brute force: count window starts o*stride whose k taps fit the padded signal
        n = sum(1 for o in range(f + 2) if o * 2 + 3 <= f + 2)
        assert N.conv_out_len(f) == n == (f - 1) // 2 + 1
    for f in (1, 2, 3, 4, 5, 1499, 1500, 2999, 3000, 3001):
        out = F.conv1d(torch.zeros(1, 1, f), torch.zeros(1, 1, 3), stride=2, padding=1)
        assert out.shape[-1] == N.conv_out_len(f)


def test_argmax_lowest_index_on_ties_and_margin():
    l = np.array([[0.5, 2.0, 2.0, -1.0], [3.0, 3.0, 3.0, 3.0], [-1, -2, -0.5, -0.5]])
    np.testing.assert_array_equal(N.argmax_lowest(l), [1, 0, 2])
    np.testing.assert_allclose(N.top2_margin(l), [0.0, 0.0, 0.0])
    np.testing.assert_allclose(N.top2_margin(np.array([[1.0, 3.5, 2.0]])), [1.5])

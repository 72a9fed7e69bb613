"""The seeded input generators: deterministic, subset draws equal full draws,
values exactly representable in the storage dtype, recipe statistics (CPU)."""
import numpy as np

import workloads as WL


def test_weights_deterministic_and_subset_equal():
    w = WL.reduced(WL.by_name("whisper_base_f16_beam5"), layers=2, vocab=3000)
    a = WL.make_weights(w)
    b = WL.make_weights(w, names=["dec.1.fc1.w", "embed"])
    np.testing.assert_array_equal(a["dec.1.fc1.w"], b["dec.1.fc1.w"])
    np.testing.assert_array_equal(a["embed"], b["embed"])
    c = WL.make_weights(w)
    for k in a:
        np.testing.assert_array_equal(a[k], c[k])


def test_storage_dtype_exact_and_recipe():
    for name, np_check in (("whisper_base_f16_beam5", np.float16), ("whisper_large_bf16_b64", None)):
        w = WL.reduced(WL.by_name(name), layers=1, vocab=5000, d=256, d_ff=512, heads=4)
        W = WL.make_weights(w)
        if np_check is not None:
            assert np.all(W["embed"].astype(np_check).astype(np.float32) == W["embed"])
        else:
            bits = W["embed"].view(np.uint32)
            assert np.all((bits & 0xFFFF) == 0)
        assert abs(W["embed"].std() - 0.02) < 1e-3
        assert abs(W["dec.0.ln1.g"].mean() - 1.0) < 0.01
        assert abs(W["dec.0.ln1.b"].mean()) < 0.01


def test_encoder_states_and_prompts():
    w = WL.reduced(WL.by_name("whisper_small_f16_b16"), frames=300)
    e = WL.make_encoder_states(w)
    assert e.shape == (16, 300, 768)
    np.testing.assert_array_equal(WL.make_encoder_states(w, streams=[3, 7]), e[[3, 7]])
    assert abs(e.std() - 1.0) < 0.01
    p = WL.make_prompt(w)
    assert p.shape == (16, 4) and np.all(p == p[0])


def test_qwen_prefill_inputs():
    w = WL.reduced(WL.by_name("qwen3asr_bf16_b8"), d=64)
    ids, audio = WL.make_qwen_prefill(w)
    assert ids.shape == (8, 900) and audio.shape == (8, 750, 64)
    assert ids.min() >= 0 and ids.max() < w.vocab
    ids2, audio2 = WL.make_qwen_prefill(w, streams=[5])
    np.testing.assert_array_equal(ids2[0], ids[5])
    np.testing.assert_array_equal(audio2[0], audio[5])

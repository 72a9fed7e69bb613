"""Helpers for the oracle pins: tiny-dimension weight sets with large scales, so
that a dropped term or a transposed operand moves the outputs well above
rounding (CPU only; imports the oracle and the workload shapes only)."""
import numpy as np

import workloads as WL


def tiny_whisper(**kw):
    base = dict(d=16, heads=2, kv_heads=2, head_dim=8, layers=2, d_ff=32, vocab=23,
                context=12, batch=3, w_dtype="f32", cache_dtype="f32", steps=12, frames=7,
                n_enc=3)
    base.update(kw)
    return WL.reduced(WL.by_name("whisper_tiny_f32_b1"), **base)


def tiny_qwen(**kw):
    base = dict(d=32, heads=4, kv_heads=2, head_dim=8, layers=2, d_ff=48, vocab=29,
                context=16, batch=3, w_dtype="f32", cache_dtype="f32", steps=8,
                prefill_len=10, audio_offset=2, audio_rows=4)
    base.update(kw)
    return WL.reduced(WL.by_name("qwen3asr_bf16_b8"), **base)


def big_weights(w, seed=0, scale=0.3):
    """Weights with the canonical names/shapes of ``w`` and O(1) effect sizes."""
    rng = np.random.default_rng(seed)
    out = {}
    for name, shape, kind in WL.weight_specs(w):
        if kind == "gain":
            out[name] = 1.0 + 0.2 * rng.standard_normal(shape)
        elif kind == "mat":
            fan_in = shape[-1]
            out[name] = rng.standard_normal(shape) * (scale * 3 / np.sqrt(fan_in))
        else:
            out[name] = 0.3 * rng.standard_normal(shape)
    return out

"""Elementwise and row-wise maths of the decoder, in float64 (oracle; test-only).

Every function here follows a definition stated on the source pages:
  * LayerNorm with a population variance and eps inside the square root, eps
    1e-5 (Whisper tiny model page (Nest), lib.linnet: the LayerNorm block uses
    torch's default epsilon);
  * RMSNorm  g * x / sqrt(mean(x^2) + eps), eps 1e-6 (transcribe.cpp
    qwen3_asr/decoder.h, header comment);
  * GELU in its error-function form (Nest model page, README "Numerics";
    mlx-bun whisper.ts, the compiled ``gelu`` graph);
  * softmax over a row (mlx-bun whisper.ts ``#attention``, precise softmax);
  * NeoX rotate-half RoPE (decoder.h header comment);
  * rounding to the cache dtype, f16 or bf16, round to nearest even
    (wavo decoder.rs module comment: the caches are f16).
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf as _erf

F64 = np.float64

# (significant bits p, frexp exponent of the smallest normal, largest finite)
_FORMATS = {
    "f16": (11, -13, 65504.0),
    "bf16": (8, -125, 3.3895313892515355e38),
}


def round_to_dtype(x, dtype: str) -> np.ndarray:
    """Round float64 values to the nearest value of ``dtype`` (ties to even),
    returned as float64.  "f32"/"f64"-style identity for "f32".

    Written as the definition: keep p significant bits, with the quantum fixed
    at the subnormal spacing below the smallest normal, and overflow to inf."""
    x = np.asarray(x, dtype=F64)
    if dtype == "f32":
        # the fp32 caches of the fp32 mode store float32 values
        return x.astype(np.float32).astype(F64)
    p, emin, vmax = _FORMATS[dtype]
    _, e = np.frexp(x)
    q = np.maximum(e, emin) - p          # exponent of the quantum
    r = np.ldexp(np.rint(np.ldexp(x, -q)), q)
    r = np.where(np.abs(r) > vmax, np.copysign(np.inf, x), r)
    r = np.where(np.isfinite(x), r, x)
    return r


def layer_norm(x, g, b, eps: float):
    x = np.asarray(x, F64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * g + b


def rms_norm(x, g, eps: float):
    x = np.asarray(x, F64)
    ms = (x * x).mean(axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def gelu_erf(x):
    x = np.asarray(x, F64)
    return x * (1.0 + _erf(x / np.sqrt(2.0))) / 2.0


def silu(x):
    x = np.asarray(x, F64)
    return x / (1.0 + np.exp(-x))


def softmax(s, axis: int = -1):
    """exp(s - max s) / sum exp(s - max s).  Entries equal to -inf get weight 0."""
    s = np.asarray(s, F64)
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=axis, keepdims=True)


def log_softmax(s, axis: int = -1):
    s = np.asarray(s, F64)
    m = np.max(s, axis=axis, keepdims=True)
    z = s - m
    return z - np.log(np.exp(z).sum(axis=axis, keepdims=True))


def rope_neox(z, pos, base: float):
    """Rotate-half RoPE on head vectors ``z`` [..., hd] at integer position(s)
    ``pos`` (broadcast against the leading axes): for i < hd/2,
    theta_i = pos * base^(-2i/hd) and the pair (z_i, z_{i+hd/2}) turns by
    theta_i."""
    z = np.asarray(z, F64)
    hd = z.shape[-1]
    half = hd // 2
    i = np.arange(half, dtype=F64)
    inv = base ** (-2.0 * i / hd)
    theta = np.asarray(pos, F64)[..., None] * inv
    c, s = np.cos(theta), np.sin(theta)
    a, b = z[..., :half], z[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def argmax_lowest(logits) -> np.ndarray:
    """Index of the row maximum, lowest index on ties, decided on the float32
    values the device produces (logits are float32 on both sides)."""
    l32 = np.asarray(logits).astype(np.float32)
    return np.argmax(l32, axis=-1).astype(np.int32)


def top2_margin(logits) -> np.ndarray:
    """Gap between the largest and second-largest logit of each row."""
    l = np.asarray(logits, F64)
    part = np.partition(l, -2, axis=-1)
    return part[..., -1] - part[..., -2]


def conv_out_len(frames: int, kernel: int = 3, stride: int = 2, pad: int = 1) -> int:
    """Output length of a 1-D convolution (Nest model page, README "The
    convolutional stem" and lib.linnet ``conv1d``): (L + 2*pad - k)//stride + 1."""
    return (frames + 2 * pad - kernel) // stride + 1

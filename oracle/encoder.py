"""Whisper-style audio encoder, float64 (oracle; test-only: only the test suite imports it).

What it computes, with the passage each part follows:

* The stem: a 1-D convolution of kernel 3, stride 1, one frame of padding over the mel
  channels, plus bias, then GELU (erf form); a second one of kernel 3, stride 2, one frame of
  padding, plus bias, then GELU.  ``Frames`` mel frames become ``(Frames - 1) // 2 + 1``
  positions (Nest whisper-tiny model page, "The convolutional stem" and lib.linnet
  ``encoded``; mlx-bun whisper.ts ``encode``).  A convolution is written here as its
  definition: output position o sums, over taps k and input channels c, the padded input at
  ``o * stride + k`` times the kernel ``w[out, c, k]``.
* The stored position table is added to the stem's output (the Nest page: the checkpoint
  keeps the positions as an ordinary tensor; mlx-bun adds its sinusoids at the same place).
* Each layer is pre-LN: ``x += attn(LN1(x))`` over all positions (no mask; no key bias; q
  and k each scaled by hd^-1/4, as in the decoder), then ``x += W2 GELU(W1 LN2(x) + b1) + b2``
  (mlx-bun ``encode``: ``attn_ln``, ``#attention``, ``#mlp``).
* A final LayerNorm (mlx-bun ``encoder.ln_post``; lib.linnet ``encoder_norm``), eps 1e-5.

Canonical tensor names (i = layer): ``enc.conv1.w`` [d, mels, 3], ``enc.conv1.b`` [d],
``enc.conv2.w`` [d, d, 3], ``enc.conv2.b``, ``enc.pos`` [positions, d], ``enc.{i}.ln1.g/.b``,
``enc.{i}.attn.q.w/.b``, ``enc.{i}.attn.k.w``, ``enc.{i}.attn.v.w/.b``, ``enc.{i}.attn.o.w/.b``,
``enc.{i}.ln2.g/.b``, ``enc.{i}.fc1.w/.b``, ``enc.{i}.fc2.w/.b``, ``enc.ln_post.g/.b``.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from .numerics import conv_out_len, gelu_erf, layer_norm, softmax

F64 = np.float64


def conv1d(x, w, b, stride: int, pad: int):
    """x [L, Cin] (positions first), w [Cout, Cin, K], b [Cout] -> [Lout, Cout]."""
    x = np.asarray(x, F64)
    w = np.asarray(w, F64)
    L, cin = x.shape
    cout, cin_w, K = w.shape
    assert cin == cin_w
    xp = np.concatenate([np.zeros((pad, cin)), x, np.zeros((pad, cin))], 0)
    lout = conv_out_len(L, K, stride, pad)
    out = np.empty((lout, cout))
    for o in range(lout):
        win = xp[o * stride:o * stride + K]            # [K, Cin]
        out[o] = np.tensordot(w, win.T, axes=([1, 2], [0, 1])) + b
    return out


def attention(y, W, p, heads: int):
    """Multi-head self-attention of y [P, d] over all positions."""
    P, d = y.shape
    hd = d // heads
    c = hd ** -0.25
    q = (y @ W[p + "q.w"].T + W[p + "q.b"]) * c
    k = (y @ W[p + "k.w"].T) * c
    v = y @ W[p + "v.w"].T + W[p + "v.b"]
    qh = q.reshape(P, heads, hd).transpose(1, 0, 2)
    kh = k.reshape(P, heads, hd).transpose(1, 0, 2)
    vh = v.reshape(P, heads, hd).transpose(1, 0, 2)
    o = (softmax(qh @ kh.transpose(0, 2, 1), -1) @ vh).transpose(1, 0, 2).reshape(P, d)
    return o @ W[p + "o.w"].T + W[p + "o.b"]


def encode(weights: Dict[str, np.ndarray], mel, heads: int, layers: int, eps: float = 1e-5):
    """mel [Frames, Mels] -> encoder states [(Frames - 1) // 2 + 1, d]."""
    W = {k: np.asarray(v, F64) for k, v in weights.items()}
    if any(k.endswith(".k.b") for k in W):
        raise ValueError("the key projections carry no bias")
    x = gelu_erf(conv1d(mel, W["enc.conv1.w"], W["enc.conv1.b"], 1, 1))
    x = gelu_erf(conv1d(x, W["enc.conv2.w"], W["enc.conv2.b"], 2, 1))
    x = x + W["enc.pos"][:x.shape[0]]
    for i in range(layers):
        p = f"enc.{i}."
        x = x + attention(layer_norm(x, W[p + "ln1.g"], W[p + "ln1.b"], eps), W, p + "attn.", heads)
        y = layer_norm(x, W[p + "ln2.g"], W[p + "ln2.b"], eps)
        x = x + gelu_erf(y @ W[p + "fc1.w"].T + W[p + "fc1.b"]) @ W[p + "fc2.w"].T + W[p + "fc2.b"]
    return layer_norm(x, W["enc.ln_post.g"], W["enc.ln_post.b"], eps)

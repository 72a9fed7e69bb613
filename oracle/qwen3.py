"""Qwen3-ASR-style causal LM step and prefill, float64 (oracle; test-only).

Follows transcribe.cpp qwen3_asr/decoder.h (header comment and the
``StepBuildBatched`` / ``PrefillBuild`` descriptors):
  * pre-norm RMSNorm, eps 1e-6, g * x / sqrt(mean(x^2) + eps);
  * grouped-query attention: Hq query heads over Hkv key/value heads, query
    head h reads kv head h // (Hq/Hkv) (contiguous groups);
  * per-head RMSNorm of q and k over head_dim, after the projection and
    before RoPE, one gain vector of length head_dim shared by the heads;
  * NeoX rotate-half RoPE at base 1e6 (the multimodal section split reduces to
    plain RoPE when every position has one coordinate, as the header says);
  * SwiGLU MLP down(silu(gate(x)) * up(x)); no biases anywhere;
  * tied head: logits = E @ RMSNorm_f(x);
  * the K/V of the current position is written before attending, and the step
    reads rows 0..p (rows beyond n_past are masked to -inf in the header's step
    graph; here they are simply not read);
  * audio injection: prompt rows [offset, offset + A) take the audio
    embeddings instead of the token embeddings (the header's concat /
    keep-mask blend; both give the same block input).
Attention scale 1/sqrt(head_dim) (the pages are silent; standard reading).
The cache dtype rounding applies to K and V when written.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .numerics import F64, rms_norm, rope_neox, round_to_dtype, silu, softmax


class QwenDims:
    def __init__(self, d, heads, kv_heads, head_dim, layers, d_ff, vocab, context,
                 eps=1e-6, rope_base=1e6, cache_dtype="f16"):
        assert heads % kv_heads == 0
        self.d, self.hq, self.hkv, self.hd = d, heads, kv_heads, head_dim
        self.layers, self.d_ff, self.vocab, self.context = layers, d_ff, vocab, context
        self.eps, self.base, self.cache_dtype = eps, rope_base, cache_dtype
        self.group = heads // kv_heads


def dims_of(w) -> QwenDims:
    return QwenDims(w.d, w.heads, w.kv_heads, w.head_dim, w.layers, w.d_ff, w.vocab,
                    w.context, w.eps, w.rope_base, w.cache_dtype)


class QwenOracle:
    def __init__(self, dims: QwenDims, weights: Dict[str, np.ndarray], round_cache=True):
        self.D = dims
        self.W = {k: np.asarray(v, F64) for k, v in weights.items()}
        self.rc = (lambda a: round_to_dtype(a, dims.cache_dtype)) if round_cache else (lambda a: a)
        self.K = self.V = None

    def reset(self, B: int):
        D = self.D
        shape = (B, D.context, D.hkv, D.hd)
        self.K = [np.full(shape, np.nan) for _ in range(D.layers)]
        self.V = [np.full(shape, np.nan) for _ in range(D.layers)]

    def _qkv(self, l, x, pos):
        """x [n, d], pos [n] -> q [n, Hq, hd] (normed, rotated), k, v [n, Hkv, hd]."""
        D, W = self.D, self.W
        p = f"dec.{l}."
        y = rms_norm(x, W[p + "norm1.g"], D.eps)
        q = (y @ W[p + "self.q.w"].T).reshape(-1, D.hq, D.hd)
        k = (y @ W[p + "self.k.w"].T).reshape(-1, D.hkv, D.hd)
        v = (y @ W[p + "self.v.w"].T).reshape(-1, D.hkv, D.hd)
        q = rope_neox(rms_norm(q, W[p + "q_norm.g"], D.eps), np.asarray(pos)[:, None], D.base)
        k = rope_neox(rms_norm(k, W[p + "k_norm.g"], D.eps), np.asarray(pos)[:, None], D.base)
        return q, k, v

    def _mlp(self, l, x):
        D, W = self.D, self.W
        p = f"dec.{l}."
        y = rms_norm(x, W[p + "norm2.g"], D.eps)
        return (silu(y @ W[p + "mlp.gate.w"].T) * (y @ W[p + "mlp.up.w"].T)) @ W[p + "mlp.down.w"].T

    def _head(self, x):
        return rms_norm(x, self.W["norm_f.g"], self.D.eps) @ self.W["embed"].T

    def _gqa(self, q, K, V, mask=None):
        """q [nq, Hq, hd], K/V [nk, Hkv, hd] -> [nq, Hq*hd]."""
        D = self.D
        kv_of = np.arange(D.hq) // D.group
        Kx, Vx = K[:, kv_of, :], V[:, kv_of, :]                # [nk, Hq, hd]
        s = np.einsum("qhc,khc->hqk", q, Kx) / np.sqrt(D.hd)
        if mask is not None:
            s = s + mask
        a = softmax(s, -1)
        return np.einsum("hqk,khc->qhc", a, Vx).reshape(q.shape[0], D.hq * D.hd)

    def step(self, tokens, positions, embeds: Optional[np.ndarray] = None):
        """One token per row: tokens, positions [B]; ``embeds`` [B, d] (optional)
        replaces the token embedding.  Returns logits [B, V]."""
        D, W = self.D, self.W
        tokens = np.asarray(tokens, np.int64)
        positions = np.asarray(positions, np.int64)
        B = tokens.shape[0]
        x = W["embed"][tokens] if embeds is None else np.asarray(embeds, F64).copy()
        for l in range(D.layers):
            q, k, v = self._qkv(l, x, positions)
            o = np.empty((B, D.hq * D.hd))
            for b in range(B):
                p = positions[b]
                self.K[l][b, p] = self.rc(k[b])
                self.V[l][b, p] = self.rc(v[b])
                o[b] = self._gqa(q[b:b + 1], self.K[l][b, :p + 1], self.V[l][b, :p + 1])[0]
            x = x + o @ W[f"dec.{l}.self.o.w"].T
            x = x + self._mlp(l, x)
        return self._head(x)

    def prefill(self, ids, audio=None, offset: int = 0):
        """ids [B, T]; audio [B, A, d] spliced at rows offset..offset+A-1.  Fills
        cache rows 0..T-1 with causal attention over the whole prompt at once and
        returns the logits of the last row [B, V]."""
        D, W = self.D, self.W
        ids = np.asarray(ids, np.int64)
        B, T = ids.shape
        causal = np.where(np.arange(T)[None, :] <= np.arange(T)[:, None], 0.0, -np.inf)
        out = np.empty((B, D.vocab))
        pos = np.arange(T)
        for b in range(B):
            x = W["embed"][ids[b]]
            if audio is not None:
                A = audio.shape[1]
                x[offset:offset + A] = np.asarray(audio[b], F64)
            for l in range(D.layers):
                q, k, v = self._qkv(l, x, pos)
                k, v = self.rc(k), self.rc(v)
                self.K[l][b, :T] = k
                self.V[l][b, :T] = v
                x = x + self._gqa(q, k, v, causal) @ W[f"dec.{l}.self.o.w"].T
                x = x + self._mlp(l, x)
            out[b] = self._head(x[-1:])[0]
        return out


def decode_full(dims: QwenDims, weights, ids, round_cache=False, embeds=None, offset=0):
    """Full-prefix recompute for one stream: ids [S] -> logits [S, V] at every
    position (causal).  ``embeds`` [A, d] replaces rows offset..offset+A-1."""
    o = QwenOracle(dims, weights, round_cache=round_cache)
    D, W = o.D, o.W
    ids = np.asarray(ids, np.int64)
    S = ids.shape[0]
    x = W["embed"][ids]
    if embeds is not None:
        x[offset:offset + embeds.shape[0]] = np.asarray(embeds, F64)
    causal = np.where(np.arange(S)[None, :] <= np.arange(S)[:, None], 0.0, -np.inf)
    pos = np.arange(S)
    for l in range(D.layers):
        q, k, v = o._qkv(l, x, pos)
        k, v = o.rc(k), o.rc(v)
        x = x + o._gqa(q, k, v, causal) @ W[f"dec.{l}.self.o.w"].T
        x = x + o._mlp(l, x)
    return o._head(x)

"""Whisper-style decoder step, float64 (oracle; test-only).

What it computes, with the passage each part follows:

* Weights: ``W`` is [out, in] and a projection is ``W @ y + b`` (mlx-bun
  whisper.ts, ``#linear``: addmm with the transposed weight).  The key
  projections carry no bias; query, value and output projections do (wavo
  decoder.rs, ``Layer::cross_kv`` doc and ``Decoder::load``, whose fused cross
  bias is zero over the K half; Nest model page, README "The key projection
  has no bias").
* Cross K/V are computed once per window from the encoder states and kept
  (wavo ``record_cross``; Nest lib.linnet ``DecoderLayer.listen``; mlx-bun
  ``decode``, which fills ``crossK/crossV`` on first use and reuses them).
* One step at position p with token t (wavo ``record_step``; Nest lib.linnet
  ``Model.step`` and ``DecoderLayer.step``):
    x = E[t] + P[p]
    per layer: y = LN1(x); q = Wq y + bq; k = Wk y; v = Wv y + bv;
      k, v are written to cache row p BEFORE attending (wavo passes
      ``pos + 1`` rows to ``attend`` after the ``pack``; Nest ``step`` writes
      with ``write_at`` then masks ``slot <= pos``);
      heads split the feature axis into [H, hd] (Nest ``heads``);
      score_j = (q_h * c) . (K_j,h * c), c = hd^(-1/4) (mlx-bun
      ``#attention`` scales q and k each by that factor); the cache keeps the
      unscaled K (mlx-bun ``WhisperLayerCache`` doc);
      o_h = softmax(score) @ V_h over rows 0..p;  x += Wo o + bo;
      y = LN2(x); q = Wcq y + bcq; attend over ALL encoder frames, no mask;
      x += Wco o + bco;  y = LN3(x); x += W2 GELU(W1 y + b1) + b2
    logits = E @ LNf(x) (tied head, no bias: wavo ``Decoder::embed`` doc;
    Nest ``Model.decode``).
* Caches are rounded to the cache dtype when written (wavo module comment:
  f16 caches; the fp32 mode stores float32).
* Beam reorder takes self-cache rows along the batch axis and leaves a cross
  cache broadcast from one encoder set alone (mlx-bun ``WhisperKvCache``
  ``rearrange``).

The full-prefix ``decode_full`` (Nest ``Model.decode``, which recomputes the
whole prefix with a causal mask) is the brute-force pin of the cached step.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from .numerics import F64, gelu_erf, layer_norm, round_to_dtype, softmax


class WhisperDims:
    def __init__(self, d, heads, layers, d_ff, vocab, context, eps=1e-5,
                 cache_dtype="f32"):
        assert d % heads == 0
        self.d, self.heads, self.layers, self.d_ff = d, heads, layers, d_ff
        self.vocab, self.context, self.eps = vocab, context, eps
        self.hd = d // heads
        self.cache_dtype = cache_dtype


def dims_of(w) -> WhisperDims:
    """Dims from any object with the workload's attribute names."""
    return WhisperDims(w.d, w.heads, w.layers, w.d_ff, w.vocab, w.context, w.eps,
                       w.cache_dtype)


class WhisperOracle:
    """Cached decoder over B rows; row b reads encoder set ``enc_of[b]``."""

    def __init__(self, dims: WhisperDims, weights: Dict[str, np.ndarray],
                 round_cache: bool = True):
        self.D = dims
        self.W = {k: np.asarray(v, F64) for k, v in weights.items()}
        if any(k.endswith(".k.b") for k in self.W):
            raise ValueError("the key projections carry no bias")
        self.rc = (lambda a: round_to_dtype(a, dims.cache_dtype)) if round_cache else (lambda a: a)
        self.Kc = self.Vc = None
        self.Ks = self.Vs = None
        self.enc_of = None

    # -- cross K/V, once per window ---------------------------------------------------
    def cross_kv(self, enc):
        """enc [n_enc, F, d] -> per layer Kc, Vc [n_enc, F, d] (cache dtype).

        ``enc`` may also be a sequence of per-set arrays [F_e, d] of different lengths
        (a window whose sets come from audio of different durations): set e's rows then
        attend over its own F_e frames, exactly as a window of that set alone (Nest model
        page: ``listen`` accepts states shorter than the full 1500 frames)."""
        if isinstance(enc, np.ndarray) and enc.ndim == 3:
            sets = None
            enc = np.asarray(enc, F64)
        else:
            sets = [np.asarray(e, F64) for e in enc]
        self.Kc, self.Vc = [], []
        for l in range(self.D.layers):
            p = f"dec.{l}.cross."
            wk, wv, bv = self.W[p + "k.w"].T, self.W[p + "v.w"].T, self.W[p + "v.b"]
            if sets is None:
                self.Kc.append(self.rc(enc @ wk))
                self.Vc.append(self.rc(enc @ wv + bv))
            else:
                self.Kc.append([self.rc(e @ wk) for e in sets])
                self.Vc.append([self.rc(e @ wv + bv) for e in sets])

    def reset(self, B: int, enc_of: Optional[Sequence[int]] = None):
        """Empty self caches for B rows.  Unwritten rows hold NaN, so any read of a
        row beyond the current position poisons the result."""
        D = self.D
        self.Ks = [np.full((B, D.context, D.d), np.nan) for _ in range(D.layers)]
        self.Vs = [np.full((B, D.context, D.d), np.nan) for _ in range(D.layers)]
        self.enc_of = np.zeros(B, np.int64) if enc_of is None else np.asarray(enc_of, np.int64)

    # -- attention ---------------------------------------------------------------------
    def _attend(self, q, K, V):
        """q [hd*H], K/V [n, d]: per head softmax((q c)(K c)^T) V, c = hd^-1/4."""
        D = self.D
        c = D.hd ** -0.25
        qh = (q * c).reshape(D.heads, D.hd)
        Kh = (K * c).reshape(-1, D.heads, D.hd)
        Vh = V.reshape(-1, D.heads, D.hd)
        s = np.einsum("hc,jhc->hj", qh, Kh)
        a = softmax(s, axis=-1)
        return np.einsum("hj,jhc->hc", a, Vh).reshape(D.d)

    # -- one step ----------------------------------------------------------------------
    def step(self, tokens, positions, return_hidden: bool = False):
        """tokens, positions [B] -> logits [B, V] (float64)."""
        D, W = self.D, self.W
        tokens = np.asarray(tokens, np.int64)
        positions = np.asarray(positions, np.int64)
        B = tokens.shape[0]
        x = W["embed"][tokens] + W["pos"][positions]
        for l in range(D.layers):
            p = f"dec.{l}."
            y = layer_norm(x, W[p + "ln1.g"], W[p + "ln1.b"], D.eps)
            q = y @ W[p + "self.q.w"].T + W[p + "self.q.b"]
            k = y @ W[p + "self.k.w"].T
            v = y @ W[p + "self.v.w"].T + W[p + "self.v.b"]
            o = np.empty((B, D.d))
            for b in range(B):
                pos = positions[b]
                self.Ks[l][b, pos] = self.rc(k[b])
                self.Vs[l][b, pos] = self.rc(v[b])
                o[b] = self._attend(q[b], self.Ks[l][b, :pos + 1], self.Vs[l][b, :pos + 1])
            x = x + o @ W[p + "self.o.w"].T + W[p + "self.o.b"]
            y = layer_norm(x, W[p + "ln2.g"], W[p + "ln2.b"], D.eps)
            q = y @ W[p + "cross.q.w"].T + W[p + "cross.q.b"]
            for b in range(B):
                e = self.enc_of[b]
                o[b] = self._attend(q[b], self.Kc[l][e], self.Vc[l][e])
            x = x + o @ W[p + "cross.o.w"].T + W[p + "cross.o.b"]
            y = layer_norm(x, W[p + "ln3.g"], W[p + "ln3.b"], D.eps)
            h = gelu_erf(y @ W[p + "fc1.w"].T + W[p + "fc1.b"])
            x = x + h @ W[p + "fc2.w"].T + W[p + "fc2.b"]
        hf = layer_norm(x, W["ln_f.g"], W["ln_f.b"], D.eps)
        logits = hf @ W["embed"].T
        if return_hidden:
            return logits, hf
        return logits

    def reorder(self, beam_idx, n_rows: Optional[int] = None):
        """New row b takes the self-cache rows of old row beam_idx[b]; a cross
        cache shared by all rows (one encoder set) is left alone."""
        idx = np.asarray(beam_idx, np.int64)
        if np.array_equal(idx, np.arange(idx.size)):
            return
        for l in range(self.D.layers):
            self.Ks[l] = self.Ks[l][idx].copy()
            self.Vs[l] = self.Vs[l][idx].copy()
        self.enc_of = self.enc_of[idx]


def decode_full(dims: WhisperDims, weights: Dict[str, np.ndarray], tokens, enc,
                round_cache: bool = False,
                key_bias: Optional[Dict[str, np.ndarray]] = None) -> np.ndarray:
    """Full-prefix recompute: tokens [S], enc [F, d] -> logits [S, V] at every
    position, causal self-attention over the whole prefix (Nest lib.linnet
    ``Model.decode`` / ``DecoderLayer.forward``).  With ``round_cache`` the keys
    and values are rounded to the cache dtype before attending, which is the
    same model as the cached step with rounded caches.

    ``key_bias`` (a what-if, not part of the model) adds a bias to the keys:
    {"dec.{l}.self": b} and/or {"dec.{l}.cross": b}.  It exists so that a test
    can show that such a bias leaves the output unchanged in exact arithmetic:
    it shifts every score of a query by the same amount q.b."""
    kb = key_bias or {}
    D = dims
    W = {k: np.asarray(v, F64) for k, v in weights.items()}
    rc = (lambda a: round_to_dtype(a, D.cache_dtype)) if round_cache else (lambda a: a)
    tokens = np.asarray(tokens, np.int64)
    enc = np.asarray(enc, F64)
    S = tokens.shape[0]
    H, hd = D.heads, D.hd
    c = hd ** -0.25
    causal = np.where(np.arange(S)[None, :] <= np.arange(S)[:, None], 0.0, -np.inf)

    def mha(q, k, v, mask):
        qh = (q * c).reshape(q.shape[0], H, hd).transpose(1, 0, 2)
        kh = (k * c).reshape(k.shape[0], H, hd).transpose(1, 0, 2)
        vh = v.reshape(v.shape[0], H, hd).transpose(1, 0, 2)
        s = qh @ kh.transpose(0, 2, 1)
        if mask is not None:
            s = s + mask
        return (softmax(s, -1) @ vh).transpose(1, 0, 2).reshape(q.shape[0], H * hd)

    x = W["embed"][tokens] + W["pos"][np.arange(S)]
    for l in range(D.layers):
        p = f"dec.{l}."
        y = layer_norm(x, W[p + "ln1.g"], W[p + "ln1.b"], D.eps)
        q = y @ W[p + "self.q.w"].T + W[p + "self.q.b"]
        k = rc(y @ W[p + "self.k.w"].T + kb.get(p + "self", 0.0))
        v = rc(y @ W[p + "self.v.w"].T + W[p + "self.v.b"])
        x = x + mha(q, k, v, causal) @ W[p + "self.o.w"].T + W[p + "self.o.b"]
        y = layer_norm(x, W[p + "ln2.g"], W[p + "ln2.b"], D.eps)
        q = y @ W[p + "cross.q.w"].T + W[p + "cross.q.b"]
        kc = rc(enc @ W[p + "cross.k.w"].T + kb.get(p + "cross", 0.0))
        vc = rc(enc @ W[p + "cross.v.w"].T + W[p + "cross.v.b"])
        x = x + mha(q, kc, vc, None) @ W[p + "cross.o.w"].T + W[p + "cross.o.b"]
        y = layer_norm(x, W[p + "ln3.g"], W[p + "ln3.b"], D.eps)
        x = x + gelu_erf(y @ W[p + "fc1.w"].T + W[p + "fc1.b"]) @ W[p + "fc2.w"].T + W[p + "fc2.b"]
    return layer_norm(x, W["ln_f.g"], W["ln_f.b"], D.eps) @ W["embed"].T

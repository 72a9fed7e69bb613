"""Synthetic workloads for the KV-cached decoder step: shapes and seeded inputs.

This package is the only code shared by the CPU oracle's tests and the GPU
path's tests and benchmark.  It holds *no* arithmetic of the decoder itself:
it names the five workload shapes, draws seeded random weights, encoder
states, prompts and audio rows, and rounds each draw once to its storage
dtype (the numbers a checkpoint in that dtype would hold).  Both sides then
consume exactly these values.

Input recipe (all draws are float32, then rounded to the storage dtype):
  * every weight matrix (token embedding, learned positions, projections)
    ~ N(0, 0.02); every bias ~ N(0, 0.02);
  * norm gains ~ 1 + N(0, 0.02), norm biases ~ N(0, 0.02);
  * encoder states ~ N(0, 1), shape [n_enc, frames, d] (frames = 1500, the
    encoder length of a 30 s window), one set per independent stream, or one
    set broadcast over the beams of a beam search;
  * Whisper prompts: 4 fixed ids (start-of-transcript, language, task,
    no-timestamps in Whisper's conventional vocabulary; any in-range ids
    serve equally with random weights);
  * Qwen3-ASR prefill: 900 positions per stream, rows 10..759 are N(0, 1)
    audio embeddings, the other 150 are uniform token ids.

Seeds: every workload has one integer seed.  ``SeedSequence(seed)`` spawns
four children (weights, encoder states or audio, token ids, spare); each
tensor then takes the child of the weight stream at its position in the
canonical name order, and large tensors are drawn in fixed-size row chunks,
each from its own grandchild, so the values do not depend on thread count.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Tuple

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "by_name", "weight_specs", "make_weights",
    "make_encoder_states", "make_prompt", "make_qwen_prefill", "round_to",
    "reduced",
]

WHISPER_PROMPT = (50258, 50259, 50359, 50363)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    arch: str                 # "whisper" or "qwen3"
    d: int
    heads: int                # query heads
    kv_heads: int             # key/value heads (== heads for Whisper)
    head_dim: int
    layers: int
    d_ff: int
    vocab: int
    context: int              # self-cache rows per stream
    batch: int                # rows per decode step (streams or beams)
    w_dtype: str              # "f32" | "f16" | "bf16"
    cache_dtype: str
    steps: int                # decode positions stepped (prompt included)
    seed: int
    frames: int = 1500        # encoder frames (Whisper only)
    n_enc: int = 1            # distinct encoder-state sets
    mode: str = "greedy"      # "greedy" | "beam"
    eps: float = 1e-5
    rope_base: float = 0.0
    prefill_len: int = 0      # Qwen3: prompt rows prefilled before decoding
    audio_offset: int = 0     # Qwen3: first audio row of the prompt
    audio_rows: int = 0       # Qwen3: number of audio rows

    @property
    def first_pos(self) -> int:
        return self.prefill_len

    def describe(self) -> str:
        return (f"{self.name}: {self.arch} d={self.d} heads={self.heads}/{self.kv_heads} "
                f"hd={self.head_dim} L={self.layers} ff={self.d_ff} V={self.vocab} "
                f"ctx={self.context} B={self.batch} w={self.w_dtype} cache={self.cache_dtype}")


WORKLOADS: Tuple[Workload, ...] = (
    Workload("whisper_tiny_f32_b1", "whisper", d=384, heads=6, kv_heads=6, head_dim=64,
             layers=4, d_ff=1536, vocab=51865, context=448, batch=1, w_dtype="f32",
             cache_dtype="f32", steps=32, seed=1),
    Workload("whisper_base_f16_beam5", "whisper", d=512, heads=8, kv_heads=8, head_dim=64,
             layers=6, d_ff=2048, vocab=51865, context=448, batch=5, w_dtype="f16",
             cache_dtype="f16", steps=128, seed=2, n_enc=1, mode="beam"),
    Workload("whisper_small_f16_b16", "whisper", d=768, heads=12, kv_heads=12, head_dim=64,
             layers=12, d_ff=3072, vocab=51865, context=448, batch=16, w_dtype="f16",
             cache_dtype="f16", steps=224, seed=3, n_enc=16),
    Workload("whisper_large_bf16_b64", "whisper", d=1280, heads=20, kv_heads=20, head_dim=64,
             layers=32, d_ff=5120, vocab=51866, context=448, batch=64, w_dtype="bf16",
             cache_dtype="bf16", steps=448, seed=4, n_enc=64),
    Workload("qwen3asr_bf16_b8", "qwen3", d=2048, heads=16, kv_heads=8, head_dim=128,
             layers=28, d_ff=6144, vocab=151936, context=1024, batch=8, w_dtype="bf16",
             cache_dtype="f16", steps=124, seed=5, frames=0, n_enc=0, eps=1e-6,
             rope_base=1e6, prefill_len=900, audio_offset=10, audio_rows=750),
)


def by_name(name: str) -> Workload:
    for w in WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


def reduced(w: Workload, **changes) -> Workload:
    """A smaller variant of a workload (same arch and dtypes) for fast tests."""
    return dataclasses.replace(w, **changes)


# ----------------------------------------------------------------------------------------
# Canonical tensor list.  kind: "mat" N(0,.02), "bias" N(0,.02), "gain" 1+N(0,.02),
# "nbias" N(0,.02).  The order fixes each tensor's seed.
# ----------------------------------------------------------------------------------------

def weight_specs(w: Workload) -> List[Tuple[str, Tuple[int, ...], str]]:
    d, ff = w.d, w.d_ff
    s: List[Tuple[str, Tuple[int, ...], str]] = []
    if w.arch == "whisper":
        s += [("embed", (w.vocab, d), "mat"), ("pos", (w.context, d), "mat"),
              ("ln_f.g", (d,), "gain"), ("ln_f.b", (d,), "nbias")]
        for i in range(w.layers):
            p = f"dec.{i}."
            s += [(p + "ln1.g", (d,), "gain"), (p + "ln1.b", (d,), "nbias"),
                  (p + "self.q.w", (d, d), "mat"), (p + "self.q.b", (d,), "bias"),
                  (p + "self.k.w", (d, d), "mat"),
                  (p + "self.v.w", (d, d), "mat"), (p + "self.v.b", (d,), "bias"),
                  (p + "self.o.w", (d, d), "mat"), (p + "self.o.b", (d,), "bias"),
                  (p + "ln2.g", (d,), "gain"), (p + "ln2.b", (d,), "nbias"),
                  (p + "cross.q.w", (d, d), "mat"), (p + "cross.q.b", (d,), "bias"),
                  (p + "cross.k.w", (d, d), "mat"),
                  (p + "cross.v.w", (d, d), "mat"), (p + "cross.v.b", (d,), "bias"),
                  (p + "cross.o.w", (d, d), "mat"), (p + "cross.o.b", (d,), "bias"),
                  (p + "ln3.g", (d,), "gain"), (p + "ln3.b", (d,), "nbias"),
                  (p + "fc1.w", (ff, d), "mat"), (p + "fc1.b", (ff,), "bias"),
                  (p + "fc2.w", (d, ff), "mat"), (p + "fc2.b", (d,), "bias")]
    elif w.arch == "qwen3":
        hq, hk, hd = w.heads, w.kv_heads, w.head_dim
        s += [("embed", (w.vocab, d), "mat"), ("norm_f.g", (d,), "gain")]
        for i in range(w.layers):
            p = f"dec.{i}."
            s += [(p + "norm1.g", (d,), "gain"),
                  (p + "self.q.w", (hq * hd, d), "mat"),
                  (p + "self.k.w", (hk * hd, d), "mat"),
                  (p + "self.v.w", (hk * hd, d), "mat"),
                  (p + "self.o.w", (d, hq * hd), "mat"),
                  (p + "q_norm.g", (hd,), "gain"), (p + "k_norm.g", (hd,), "gain"),
                  (p + "norm2.g", (d,), "gain"),
                  (p + "mlp.gate.w", (ff, d), "mat"), (p + "mlp.up.w", (ff, d), "mat"),
                  (p + "mlp.down.w", (d, ff), "mat")]
    else:
        raise ValueError(w.arch)
    return s


# ----------------------------------------------------------------------------------------
# Rounding a float32 draw to its storage dtype (round to nearest even), returned as
# float32 holding exactly representable values.
# ----------------------------------------------------------------------------------------

def round_to(a: np.ndarray, dtype: str) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f32":
        return a
    if dtype == "f16":
        return a.astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(a)
        return t.to(torch.bfloat16).to(torch.float32).numpy()
    raise ValueError(dtype)


_CHUNK = 1 << 22  # elements per independent draw


def _draw(seq: np.random.SeedSequence, shape, scale: float, offset: float,
          dtype: str) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nchunks = max(1, (n + _CHUNK - 1) // _CHUNK)
    kids = seq.spawn(nchunks)
    for c in range(nchunks):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        g = np.random.Generator(np.random.PCG64(kids[c]))
        g.standard_normal(out=out[lo:hi], dtype=np.float32)
    if scale != 1.0:
        out *= np.float32(scale)
    if offset != 0.0:
        out += np.float32(offset)
    return round_to(out, dtype).reshape(shape)


def _streams(w: Workload):
    return np.random.SeedSequence(w.seed).spawn(4)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_weights(w: Workload, names: Optional[List[str]] = None) -> Dict[str, np.ndarray]:
    """All weights of ``w`` as float32 arrays holding storage-dtype values.

    ``names`` restricts the draw to a subset (values are identical to the full
    draw, since each tensor has its own seed)."""
    specs = weight_specs(w)
    kids = _streams(w)[0].spawn(len(specs))
    jobs = []
    for (name, shape, kind), seq in zip(specs, kids):
        if names is not None and name not in names:
            continue
        scale, off = {"mat": (0.02, 0.0), "bias": (0.02, 0.0), "gain": (0.02, 1.0),
                      "nbias": (0.02, 0.0)}[kind]
        jobs.append((name, seq, shape, scale, off))
    with ThreadPoolExecutor(_threads()) as ex:
        arrs = list(ex.map(lambda j: _draw(j[1], j[2], j[3], j[4], w.w_dtype), jobs))
    return {j[0]: a for j, a in zip(jobs, arrs)}


def make_encoder_states(w: Workload, streams: Optional[List[int]] = None) -> np.ndarray:
    """Encoder states [n_enc, frames, d] ~ N(0,1) in the weight dtype.  ``streams``
    selects a subset of the encoder sets (same values as in the full draw)."""
    assert w.arch == "whisper"
    kids = _streams(w)[1].spawn(w.n_enc)
    sel = list(range(w.n_enc)) if streams is None else list(streams)
    with ThreadPoolExecutor(_threads()) as ex:
        arrs = list(ex.map(lambda e: _draw(kids[e], (w.frames, w.d), 1.0, 0.0, w.w_dtype), sel))
    return np.stack(arrs, 0)


def make_prompt(w: Workload) -> np.ndarray:
    """Whisper prompt ids [batch, 4] (the same 4 ids in every row); reduced test
    vocabularies take the ids modulo their size."""
    return np.tile(np.array(WHISPER_PROMPT, dtype=np.int32) % w.vocab, (w.batch, 1)).astype(np.int32)


def make_qwen_prefill(w: Workload, streams: Optional[List[int]] = None):
    """Qwen3-ASR prefill inputs: ids [B, T] int32 (uniform on [0, V)) and audio
    rows [B, A, d] ~ N(0,1) in the weight dtype, to be spliced at rows
    audio_offset .. audio_offset + A - 1 (the ids there are placeholders)."""
    assert w.arch == "qwen3"
    T, A = w.prefill_len, w.audio_rows
    sel = list(range(w.batch)) if streams is None else list(streams)
    id_kids = _streams(w)[2].spawn(w.batch)
    au_kids = _streams(w)[1].spawn(w.batch)
    ids = np.stack([np.random.Generator(np.random.PCG64(id_kids[b])).integers(
        0, w.vocab, size=T, dtype=np.int64).astype(np.int32) for b in sel], 0)
    audio = np.stack([_draw(au_kids[b], (A, w.d), 1.0, 0.0, w.w_dtype) for b in sel], 0)
    return ids, audio


def random_ids(w: Workload, n: int, salt: int = 0) -> np.ndarray:
    """Seeded uniform token ids [batch, n] for teacher-forced runs."""
    kid = _streams(w)[3].spawn(salt + 1)[salt]
    g = np.random.Generator(np.random.PCG64(kid))
    return g.integers(0, w.vocab, size=(w.batch, n), dtype=np.int64).astype(np.int32)

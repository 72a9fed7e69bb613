"""Beam-selection rule that drives the beam reorder (oracle; test-only).

The pages give only the reorder itself (mlx-bun whisper.ts,
``WhisperKvCache.rearrange``: keep rows ``indices`` along the batch axis,
identity returns early).  The rule that produces the indices is the plain
reading of a width-W beam search with no length penalty and no end token:

  * scores S_b start at 0 and every beam is fed the same prompt;
  * at the first generated position all beams are identical, so only beam 0
    is expanded;
  * afterwards candidate (b, v) scores S_b + log_softmax(logits_b)_v (float64);
  * the W best candidates are kept, best first; ties go to the lower flat
    index b*V + v;
  * the kept candidates' source rows are the beam indices, their v the next
    tokens.
"""
from __future__ import annotations

import numpy as np

from .numerics import log_softmax


def select(scores, logits, first: bool):
    """scores [W] float64, logits [W, V] -> (beam_idx [W] int32,
    tokens [W] int32, new_scores [W] float64, gaps [W] float64).

    ``gaps[i]`` is the score gap between kept candidate i and the next
    candidate in the ranking (the i+1-th kept one, or the best rejected one for
    the last): a decision is robust when its gap is large."""
    logits = np.asarray(logits, np.float64)
    W, V = logits.shape
    cand = np.asarray(scores, np.float64)[:, None] + log_softmax(logits, -1)
    if first:
        cand = cand[:1]
    flat = cand.reshape(-1)
    # order: score descending, then flat index ascending
    order = np.lexsort((np.arange(flat.size), -flat))
    keep = order[:W]
    nxt = order[1:W + 1]
    gaps = flat[keep] - flat[nxt]
    beam_idx = (keep // V).astype(np.int32)
    tokens = (keep % V).astype(np.int32)
    return beam_idx, tokens, flat[keep].copy(), gaps

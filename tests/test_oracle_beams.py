"""Pins of the beam-selection rule (CPU only): brute-force ranking with Python's
tuple sort, width 1 == greedy, tie order, first-step expansion of beam 0 only."""
import numpy as np

from oracle import beams
from oracle.numerics import argmax_lowest, log_softmax


def _brute(scores, logits, first, W):
    cands = []
    for b in range(1 if first else logits.shape[0]):
        ls = log_softmax(logits[b])
        for v in range(logits.shape[1]):
            cands.append((-(scores[b] + ls[v]), b * logits.shape[1] + v, b, v))
    cands.sort()
    top = cands[:W]
    return [c[2] for c in top], [c[3] for c in top], [-c[0] for c in top]


def test_select_matches_brute_force_ranking():
    rng = np.random.default_rng(0)
    for trial in range(40):
        W, V = 5, 13
        logits = np.round(rng.standard_normal((W, V)) * 2, 1)   # coarse: forces ties
        scores = np.round(rng.standard_normal(W), 1) if trial % 2 else np.zeros(W)
        first = trial % 5 == 0
        bi, tk, sc, gaps = beams.select(scores, logits, first)
        rb, rt, rs = _brute(scores, logits, first, W)
        assert list(bi) == rb and list(tk) == rt
        np.testing.assert_allclose(sc, rs, rtol=0, atol=1e-12)
        assert np.all(gaps >= -1e-15)


def test_width_one_is_greedy():
    rng = np.random.default_rng(1)
    for _ in range(20):
        logits = rng.standard_normal((1, 50))
        bi, tk, _, _ = beams.select(np.zeros(1), logits, first=False)
        assert bi[0] == 0 and tk[0] == argmax_lowest(logits)[0]


def test_first_step_expands_beam_zero_only_and_distinct_tokens():
    logits = np.tile(np.linspace(0, 1, 20), (5, 1))
    bi, tk, _, _ = beams.select(np.zeros(5), logits, first=True)
    assert list(bi) == [0] * 5
    assert len(set(tk.tolist())) == 5
    assert list(tk) == [19, 18, 17, 16, 15]

"""GPU parity of the Whisper decoder step against the oracle (teacher-forced:
both sides are fed the same tokens and beam indices, so one legitimate flip at
a low-margin step does not invalidate the steps after it)."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as WL
from oracle import beams as OB
from oracle import whisper as OW
from oracle.numerics import argmax_lowest

from .gpu_helpers import GpuRun, compare_logits, need_gpu, say, to_dev, torch_dtype

pytestmark = pytest.mark.gpu


def _greedy_parity(w, steps=None, frames=None, B=None, W=None):
    """Oracle-driven greedy decode (the oracle's argmax is the next token of both
    sides); compares every step's logits of every row."""
    need_gpu()
    say(f"[whisper greedy] {w.describe()} steps={steps or w.steps}")
    W = WL.make_weights(w) if W is None else W
    enc = WL.make_encoder_states(w)
    F = w.frames if frames is None else frames
    O = OW.WhisperOracle(OW.dims_of(w), W)
    O.cross_kv(enc[:, :F])
    B = w.batch if B is None else B
    O.reset(B, enc_of=np.arange(B) // (w.batch // w.n_enc))
    G = GpuRun(w, W)
    G.cross(enc, F)
    toks = WL.make_prompt(w)[:B, 0]
    prompt = WL.make_prompt(w)[:B]
    worst, checked = 0.0, 0
    for p in range(steps or w.steps):
        if p < prompt.shape[1]:
            toks = prompt[:, p]
        ref = O.step(toks, np.full(B, p))
        lg, am = G.step(toks, p, B=B)
        e, n = compare_logits(w, lg, ref, f"pos {p}", gpu_argmax=am)
        worst, checked = max(worst, e), checked + n
        toks = argmax_lowest(ref)
    assert G.check() == 0
    G.close()
    say(f"  worst err {worst:.3e}, argmax rows checked {checked}")
    return worst


def test_tiny_f32_b1_greedy_full():
    _greedy_parity(WL.by_name("whisper_tiny_f32_b1"))


def test_tiny_f32_ragged_frames_and_short_split():
    w = WL.reduced(WL.by_name("whisper_tiny_f32_b1"), layers=2)
    _greedy_parity(w, steps=6, frames=1000)
    _greedy_parity(w, steps=4, frames=37)


def test_f16_batch_rows_below_max():
    w = WL.reduced(WL.by_name("whisper_small_f16_b16"), layers=2, batch=6, n_enc=6, vocab=9001)
    _greedy_parity(w, steps=5, B=6)
    _greedy_parity(w, steps=5, B=3)


def test_bf16_small_dims_frames_1499():
    w = WL.reduced(WL.by_name("whisper_large_bf16_b64"), layers=2, batch=4, n_enc=4, d=256,
                   heads=4, kv_heads=4, d_ff=1024, vocab=5003)
    _greedy_parity(w, steps=8, frames=1499)


@pytest.mark.parametrize("B", [4, 24])
def test_layernorm_rows_with_large_mean(B):
    """Rows whose mean is large against their spread: layer 0's self-attention output bias
    carries +20 on every channel (exactly 20 after bf16 rounding for all but a few
    channels), so every LayerNorm after it sees rows of mean about 20 and spread about
    0.05, where a one-pass E[x^2] - mean^2 in fp32 would lose the variance.  At 24 rows the
    norms also fold split-K partial slabs."""
    w = WL.reduced(WL.by_name("whisper_large_bf16_b64"), layers=2, batch=B, n_enc=B, d=256, heads=4,
                   kv_heads=4, d_ff=512, vocab=3001, frames=64)
    W = WL.make_weights(w)
    W["dec.0.self.o.b"] = torch.from_numpy(W["dec.0.self.o.b"] + 20.0).to(torch.bfloat16).float().numpy()
    _greedy_parity(w, steps=5, W=W)


def _sampled_parity(w, steps, streams, frames=None):
    """All rows step on the GPU, teacher-forced with seeded ids after the prompt;
    the oracle recomputes the sampled rows' full prefix once (identical to the
    cached step, pinned on the CPU) and every position of them is compared.  At
    every step the argmax the library returns is checked for every row against
    its own logits, and for the sampled rows against the oracle's."""
    need_gpu()
    say(f"[whisper sampled] {w.describe()} steps={steps} rows={streams}")
    W = WL.make_weights(w)
    enc = WL.make_encoder_states(w)
    F = w.frames if frames is None else frames
    ids = WL.random_ids(w, steps)
    ids[:, :4] = WL.make_prompt(w)
    G = GpuRun(w, W)
    G.cross(enc, F)
    got = {b: [] for b in streams}
    amx = {b: [] for b in streams}
    for p in range(steps):
        lg, am = G.step(ids[:, p], p, rows=list(streams), check_all=True)
        for i, b in enumerate(streams):
            got[b].append(lg[i])
            amx[b].append(am[b])
    assert G.check() == 0
    G.close()
    del G
    torch.cuda.empty_cache()
    D = OW.dims_of(w)
    worst = 0.0
    for b in streams:
        say(f"  oracle full prefix, row {b}")
        e = b // (w.batch // w.n_enc)
        ref = OW.decode_full(D, W, ids[b], enc[e, :F], round_cache=True)
        err, _ = compare_logits(w, np.stack(got[b]), ref, f"row {b}", gpu_argmax=np.array(amx[b]))
        worst = max(worst, err)
    say(f"  worst err {worst:.3e}")


def test_small_f16_b16_sampled_rows():
    _sampled_parity(WL.by_name("whisper_small_f16_b16"), steps=40, streams=(0, 7, 15))


def test_large_bf16_b64_reduced_layers():
    w = WL.reduced(WL.by_name("whisper_large_bf16_b64"), layers=3)
    _sampled_parity(w, steps=24, streams=(0, 63))


@pytest.mark.slow
def test_large_bf16_b64_full_window_sampled_rows():
    """The large-v3 workload at its full size: 32 layers, 64 rows with their own encoder
    sets, all 448 positions (teacher-forced ids); rows 0, 9, ..., 63 (one in every 16-row
    tile of the projections and the head) against the oracle's full-prefix recompute at
    every position, and every row's returned argmax against its logits."""
    _sampled_parity(WL.by_name("whisper_large_bf16_b64"), steps=448, streams=(0, 9, 18, 27, 36, 45, 54, 63))


@pytest.mark.slow
def test_small_f16_b16_full_window_sampled_rows():
    _sampled_parity(WL.by_name("whisper_small_f16_b16"), steps=224, streams=(0, 15))


@pytest.mark.parametrize("batch", [24, 40])
def test_split_k_projections_above_16_rows(batch):
    """Rows 17..64 take the split-K projections (K groups write partials that the next
    norm or the finish kernel adds): 24 rows use 32-row tiles, 40 rows a partly filled
    64-row tile; K = 768 and 2048 give uneven K groups."""
    w = WL.reduced(WL.by_name("whisper_large_bf16_b64"), layers=2, batch=batch, n_enc=batch, d=768, heads=12,
                   kv_heads=12, d_ff=2048, vocab=9001, frames=300)
    _sampled_parity(w, steps=6, streams=(0, batch - 1))


def test_wide_model_32_k_groups_into_the_norm():
    """d = 2560 (not a multiple of 1024) and d_ff = 8192 at 24 rows: fc2 splits K into 32
    groups, and the final norm folds 32 partial slabs over 4 passes per thread, loading them
    in two halves."""
    w = WL.reduced(WL.by_name("whisper_large_bf16_b64"), layers=1, batch=24, n_enc=24, d=2560, heads=40,
                   kv_heads=40, d_ff=8192, vocab=5001, frames=100)
    _sampled_parity(w, steps=5, streams=(0, 23))


def test_ragged_window_sets_of_different_lengths():
    """wd_cross_kv_ragged: encoder sets of 1500, 777, 1 and 1024 frames in one window, the
    padding rows filled with large values that must never be read; every row's logits
    against the oracle's window of its own set, over greedy steps."""
    need_gpu()
    w = WL.reduced(WL.by_name("whisper_large_bf16_b64"), layers=2, batch=4, n_enc=4, d=256,
                   heads=4, kv_heads=4, d_ff=1024, vocab=5003)
    say(f"[whisper ragged] {w.describe()}")
    W = WL.make_weights(w)
    enc = WL.make_encoder_states(w)
    lens = [1500, 777, 1, 1024]
    padded = enc.copy()
    for e, n in enumerate(lens):
        padded[e, n:] = 50.0
    O = OW.WhisperOracle(OW.dims_of(w), W)
    O.cross_kv([enc[e, :lens[e]] for e in range(w.n_enc)])
    O.reset(w.batch, enc_of=np.arange(w.batch))
    G = GpuRun(w, W)
    G.dec.cross_kv_ragged(to_dev(np.ascontiguousarray(padded), torch_dtype(w.w_dtype)), lens)
    prompt = WL.make_prompt(w)
    toks = prompt[:, 0]
    worst = 0.0
    for p in range(8):
        toks = prompt[:, p] if p < prompt.shape[1] else toks
        ref = O.step(toks, np.full(w.batch, p))
        lg, am = G.step(toks, p)
        e, _ = compare_logits(w, lg, ref, f"pos {p}", gpu_argmax=am)
        worst = max(worst, e)
        toks = argmax_lowest(ref)
    assert G.check() == 0
    # a later uniform window returns every set to the full length
    G.cross(enc)
    O.cross_kv(enc)
    ref = O.step(toks, np.full(w.batch, 8))
    lg, am = G.step(toks, 8)
    compare_logits(w, lg, ref, "uniform window after a ragged one", gpu_argmax=am)
    G.close()
    say(f"  worst err {worst:.3e}")


def test_rows_at_different_positions():
    """Rows of one step at different positions: row b starts 3b steps late (repeating its
    position-0 token until then), so the rows' cache lengths differ in every step."""
    need_gpu()
    w = WL.reduced(WL.by_name("whisper_small_f16_b16"), layers=2, batch=4, n_enc=4, d=256, heads=4,
                   kv_heads=4, d_ff=512, vocab=3001, frames=300)
    say(f"[whisper positions] {w.describe()}")
    W = WL.make_weights(w)
    enc = WL.make_encoder_states(w)
    O = OW.WhisperOracle(OW.dims_of(w), W)
    O.cross_kv(enc)
    O.reset(w.batch, enc_of=np.arange(w.batch))
    G = GpuRun(w, W)
    G.cross(enc)
    ids = WL.random_ids(w, 24)
    delays = 3 * np.arange(w.batch)
    worst = 0.0
    for st in range(24):
        pos = np.maximum(0, st - delays).astype(np.int32)
        toks = ids[np.arange(w.batch), pos]
        ref = O.step(toks, pos)
        lg, am = G.step(toks, pos)
        e, _ = compare_logits(w, lg, ref, f"step {st} positions {pos}", gpu_argmax=am)
        worst = max(worst, e)
    assert G.check() == 0
    G.close()
    say(f"  worst err {worst:.3e}")


def _merge_candidates(scores, vals, ids, lse, V, first):
    """Width-W beam step from per-row device candidates: scores S_b + (logit - lse_b) of the
    W x W candidates, the W best kept, ties to the lower flat index b * V + v."""
    W = vals.shape[0]
    rows = 1 if first else W
    cand = np.asarray(scores, np.float64)[:rows, None] + (vals[:rows].astype(np.float64) -
                                                          lse[:rows, None].astype(np.float64))
    flat = (np.arange(rows)[:, None] * V + ids[:rows]).reshape(-1)
    c = cand.reshape(-1)
    keep = np.lexsort((flat, -c))[:W]
    return (flat[keep] // V).astype(np.int32), (flat[keep] % V).astype(np.int32), c[keep]


def _topk_definition(lg, W):
    """Per row: ids of the W largest values, equal values lower id first, NaN as -inf; and
    log(sum exp) over the non-NaN values, in float64."""
    x = np.where(np.isnan(lg), -np.inf, lg.astype(np.float64))
    ids = np.stack([np.lexsort((np.arange(x.shape[1]), -x[b]))[:W] for b in range(x.shape[0])])
    m = x.max(1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(x - m).sum(1))
    return ids, lse


def test_topk_candidates_ties_and_nan():
    """wd_topk against its definition on seeded logits over the full 51865-id vocabulary,
    with exact ties (lowest id first), a row of equal values and NaNs (never picked, left out
    of the log-sum-exp)."""
    need_gpu()
    w = WL.reduced(WL.by_name("whisper_small_f16_b16"), layers=1, d=256, heads=4, kv_heads=4, d_ff=512)
    G = GpuRun(w, WL.make_weights(w))
    rng = np.random.default_rng(123)
    lg = (rng.standard_normal((w.batch, w.vocab)) * 3).astype(np.float32)
    lg[0, [5, 17, 40000]] = 20.0
    lg[1, :] = 1.0
    lg[2, [3, 99]] = np.nan
    lg[2, 4] = 30.0
    lg[3, [50, 100, 200, w.vocab - 1]] = np.float32(7.5)
    dev = torch.from_numpy(lg).cuda()
    for W in (1, 5, 8):
        vals, ids, lse = G.dec.topk(dev, W)
        ids_r, lse_r = _topk_definition(lg, W)
        np.testing.assert_array_equal(ids.cpu().numpy(), ids_r, err_msg=f"W={W}")
        ref_vals = np.take_along_axis(np.where(np.isnan(lg), -np.inf, lg), ids_r, 1)
        np.testing.assert_array_equal(vals.cpu().numpy(), ref_vals, err_msg=f"W={W}")
        np.testing.assert_allclose(lse.cpu().numpy(), lse_r, rtol=0, atol=1e-4, err_msg=f"W={W}")
    for bad in (0, 9):
        with pytest.raises(G.K.WdError):
            G.dec.topk(dev, bad)
    assert G.check() == 0
    G.close()


def test_base_f16_beam5_full():
    """Width-5 beam search over one broadcast encoder set, 128 positions: the
    oracle's beam indices drive both sides' cache reorder; the beam choices made
    from the GPU logits must equal the oracle's wherever the ranking gaps exceed
    the margin."""
    need_gpu()
    w = WL.by_name("whisper_base_f16_beam5")
    say(f"[whisper beam] {w.describe()}")
    W = WL.make_weights(w)
    enc = WL.make_encoder_states(w)
    O = OW.WhisperOracle(OW.dims_of(w), W)
    O.cross_kv(enc)
    O.reset(w.batch)
    G = GpuRun(w, W)
    G.cross(enc)
    prompt = WL.make_prompt(w)
    scores = np.zeros(w.batch)
    toks = prompt[:, 0]
    beam_idx = None
    decided, merged, worst = 0, 0, 0.0
    for p in range(w.steps):
        if p < prompt.shape[1]:
            toks = prompt[:, p]
        elif beam_idx is not None:
            O.reorder(beam_idx)
            G.dec.reorder(beam_idx, p)
        ref = O.step(toks, np.full(w.batch, p))
        lg, am = G.step(toks, p)
        e, _ = compare_logits(w, lg, ref, f"pos {p}", gpu_argmax=am)
        worst = max(worst, e)
        if p >= prompt.shape[1] - 1:
            first = p == prompt.shape[1] - 1
            bi, tk, sc, gaps = OB.select(scores, ref, first)
            gbi, gtk, _, ggaps = OB.select(scores, lg.astype(np.float64), first)
            if np.all(gaps > 1e-2):
                np.testing.assert_array_equal(gbi, bi, err_msg=f"beam indices at pos {p}")
                np.testing.assert_array_equal(gtk, tk, err_msg=f"beam tokens at pos {p}")
                decided += 1
            # the same choice from the device candidates (wd_topk: W per row + lse), merged here
            vals, ids, lse = G.dec.topk(G.logits[:w.batch], w.batch)
            tbi, ttk, _ = _merge_candidates(scores, vals.cpu().numpy(), ids.cpu().numpy(), lse.cpu().numpy(),
                                            w.vocab, first)
            if np.all(ggaps > 1e-4):
                np.testing.assert_array_equal(tbi, gbi, err_msg=f"device-candidate beams at pos {p}")
                np.testing.assert_array_equal(ttk, gtk, err_msg=f"device-candidate tokens at pos {p}")
                merged += 1
            beam_idx, toks, scores = bi, tk, sc
    assert G.check() == 0
    G.close()
    say(f"  worst err {worst:.3e}; beam decisions compared {decided}, from device candidates {merged}")
    assert decided > 0 and merged > 0


def test_beam_step_on_device_matches_host_merge():
    """wd_beam_step (candidates, W x W merge and cache rearrangement, all on the device, the
    next tokens written straight into the token buffer) against the same step taken from the
    device candidates with the merge in float64 on the host and wd_reorder: over 64 positions of
    a width-5 search the two decoders write bit-identical logits, and the beam indices, tokens
    and float64 scores agree exactly (the same operations in the same order).  The host merge
    is the rule that test_base_f16_beam5_full checks against the oracle."""
    need_gpu()
    w = WL.reduced(WL.by_name("whisper_base_f16_beam5"), layers=2)
    say(f"[beam step on device] {w.describe()}")
    W = WL.make_weights(w)
    enc = WL.make_encoder_states(w)
    A, H = GpuRun(w, W), GpuRun(w, W)
    A.cross(enc)
    H.cross(enc)
    nb, steps = w.batch, 64
    prompt = WL.make_prompt(w)
    scores_dev = torch.zeros(nb, dtype=torch.float64, device="cuda")
    bi_dev = torch.zeros(nb, dtype=torch.int32, device="cuda")
    scores, toks = np.zeros(nb), prompt[:, 0]
    merged = 0
    for p in range(steps):
        if p < prompt.shape[1]:
            toks = prompt[:, p]
            A.tok.copy_(torch.as_tensor(np.asarray(toks, np.int32)))
        A.pos.fill_(p)
        A.dec.step(A.tok, A.pos, A.logits, A.amax)
        lg_h, _ = H.step(toks, p)
        np.testing.assert_array_equal(A.logits.cpu().numpy(), lg_h, err_msg=f"logits at pos {p}")
        if p >= prompt.shape[1] - 1:
            first = p == prompt.shape[1] - 1
            n_rows = p + 1 if p + 1 < steps else 0
            A.dec.beam_step(A.logits, nb, first, scores_dev, bi_dev, A.tok, n_rows)
            vals, ids, lse = H.dec.topk(H.logits, nb)
            hbi, htk, hsc = _merge_candidates(scores, vals.cpu().numpy(), ids.cpu().numpy(), lse.cpu().numpy(),
                                              w.vocab, first)
            np.testing.assert_array_equal(bi_dev.cpu().numpy(), hbi, err_msg=f"beam indices at pos {p}")
            np.testing.assert_array_equal(A.tok.cpu().numpy(), htk, err_msg=f"tokens at pos {p}")
            np.testing.assert_array_equal(scores_dev.cpu().numpy(), hsc, err_msg=f"scores at pos {p}")
            if n_rows:
                H.dec.reorder(hbi, n_rows)
            toks, scores = htk, hsc
            merged += 1
    K = A.K
    for bad in (dict(W=nb + 1), dict(first=2), dict(n_rows=w.context + 1)):
        args = {**dict(W=nb, first=0, n_rows=1), **bad}
        st = K.lib().wd_beam_step(A.dec.ctx, ctypes.c_void_p(A.logits.data_ptr()), args["W"], args["first"],
                                  ctypes.c_void_p(scores_dev.data_ptr()), ctypes.c_void_p(bi_dev.data_ptr()),
                                  ctypes.c_void_p(A.tok.data_ptr()), args["n_rows"])
        assert st == 1, (bad, st)
    assert A.check() == 0 and H.check() == 0
    A.close()
    H.close()
    say(f"  device beam steps compared {merged}")


def test_reorder_identity_and_inverse_restore_cache():
    need_gpu()
    w = WL.reduced(WL.by_name("whisper_base_f16_beam5"), layers=2, vocab=4001)
    W = WL.make_weights(w)
    enc = WL.make_encoder_states(w)
    ids = WL.random_ids(w, 8)
    A, B = GpuRun(w, W), GpuRun(w, W)
    A.cross(enc)
    B.cross(enc)
    for p in range(6):
        A.step(ids[:, p], p)
        B.step(ids[:, p], p)
    perm = [3, 0, 4, 1, 2]
    inv = list(np.argsort(perm))
    B.dec.reorder([0, 1, 2, 3, 4], 6)    # identity: returns at once
    B.dec.reorder(perm, 6)
    B.dec.reorder(inv, 6)
    la, _ = A.step(ids[:, 6], 6)
    lb, _ = B.step(ids[:, 6], 6)
    np.testing.assert_array_equal(la, lb)
    # a real permutation: row b of the reordered run equals row perm[b] of the plain run's
    # continuation from the same state (same token fed)
    C = GpuRun(w, W)
    C.cross(enc)
    for p in range(7):
        C.step(ids[:, p], p)
    B.dec.reorder(perm, 7)
    t = np.full(w.batch, 17, np.int32)
    lb, _ = B.step(t, 7)
    lc, _ = C.step(t, 7)
    np.testing.assert_array_equal(lb, lc[perm])
    for g in (A, B, C):
        g.close()


def test_argmax_exact_ties_lowest_index():
    need_gpu()
    w = WL.reduced(WL.by_name("whisper_tiny_f32_b1"), layers=1, vocab=3000)
    W = WL.make_weights(w)
    E = W["embed"].copy()
    E[:] = E[5]
    E[1234] = 2 * E[5]
    E[2345] = 2 * E[5]
    W["embed"] = E
    enc = WL.make_encoder_states(w)
    G = GpuRun(w, W)
    G.cross(enc)
    O = OW.WhisperOracle(OW.dims_of(w), W)
    O.cross_kv(enc)
    O.reset(1)
    for p in range(3):
        ref = O.step([5], [p])
        lg, am = G.step([5], p)
        want = argmax_lowest(ref)[0]
        assert want in (0, 1234)
        assert am[0] == want, (am[0], want)
    G.close()


def _tied_embedding(W, base, top):
    """Every embedding row equal to row `base`, and the rows in `top` equal to twice it:
    all logits E.h of a row tie exactly on two values (equal rows give bit-identical dot
    products), so the argmax is min(top) when E[base].h > 0 and 0 otherwise."""
    E = W["embed"].copy()
    E[:] = E[base]
    for t in top:
        E[t] = 2 * E[base]
    W["embed"] = E
    return W


def _tie_winner(ref, top):
    """The lowest-index argmax the tied logits must give (from the oracle's values), or -1
    where the two tied values are too close to decide."""
    hi, lo = ref[:, top[0]], ref[:, 0]
    return np.where(hi - lo > 1e-2, min(top), np.where(lo - hi > 1e-2, 0, -1))


def test_argmax_exact_ties_mfma_head_b64():
    """Exact ties through the 16-bit tied head at 64 rows (the LDS-shared MFMA kernel, rows in
    all four 16-row tiles, per-block argmax keys merged in a second kernel) over the full
    51866-id vocabulary: ties inside one output block (1234, 1235), across blocks (2345) and
    across every block at once (all other ids)."""
    need_gpu()
    w = WL.reduced(WL.by_name("whisper_large_bf16_b64"), layers=1, d=256, heads=4, kv_heads=4, d_ff=512,
                   frames=64)
    top = [1234, 1235, 2345]
    W = _tied_embedding(WL.make_weights(w), 5, top)
    enc = WL.make_encoder_states(w)
    O = OW.WhisperOracle(OW.dims_of(w), W)
    O.cross_kv(enc)
    O.reset(w.batch, enc_of=np.arange(w.batch))
    G = GpuRun(w, W)
    G.cross(enc)
    ids = WL.random_ids(w, 3)
    decided = 0
    for p in range(3):
        ref = O.step(ids[:, p], np.full(w.batch, p))
        lg, am = G.step(ids[:, p], p, check_all=True)
        for t in top[1:]:
            np.testing.assert_array_equal(lg[:, t], lg[:, top[0]], err_msg=f"tied logits, pos {p}")
        np.testing.assert_array_equal(lg[:, 1], lg[:, 0], err_msg=f"tied logits, pos {p}")
        want = _tie_winner(ref, top)
        sel = want >= 0
        np.testing.assert_array_equal(am[sel], want[sel], err_msg=f"tie winner, pos {p}")
        decided += int(sel.sum())
    assert G.check() == 0
    G.close()
    say(f"  tie winners checked {decided}")
    assert decided > 0


def test_step_graph_cache_many_output_buffers():
    """A step is captured once per output-buffer set and replayed; more distinct buffers
    than the cache holds evict the least recently used graphs (after the stream has passed
    them).  Re-stepping one position with the same tokens rewrites the same cache row, so
    every call must give the same logits and ids, whichever graph serves it."""
    need_gpu()
    w = WL.reduced(WL.by_name("whisper_small_f16_b16"), layers=2, batch=4, n_enc=4, d=256, heads=4, kv_heads=4,
                   d_ff=512, vocab=3001, frames=100)
    W = WL.make_weights(w)
    enc = WL.make_encoder_states(w)
    G = GpuRun(w, W)
    G.cross(enc)
    ids = WL.random_ids(w, 2)
    G.step(ids[:, 0], 0)
    ref_lg, ref_am = G.step(ids[:, 1], 1)
    outs = [(torch.empty(w.batch, w.vocab, dtype=torch.float32, device="cuda"),
             torch.empty(w.batch, dtype=torch.int32, device="cuda")) for _ in range(12)]
    tok = torch.from_numpy(ids[:, 1].copy()).cuda()
    pos = torch.ones(w.batch, dtype=torch.int32, device="cuda")
    order = list(range(12)) + [0, 11, 3, 7] + list(range(12))
    for i in order:
        G.dec.step(tok, pos, outs[i][0], outs[i][1])
    torch.cuda.synchronize()
    for i in set(order):
        np.testing.assert_array_equal(outs[i][0].cpu().numpy(), ref_lg, err_msg=f"buffer set {i}")
        np.testing.assert_array_equal(outs[i][1].cpu().numpy(), ref_am, err_msg=f"buffer set {i}")
    assert G.check() == 0
    G.close()


@pytest.mark.parametrize("name", ["whisper_large_bf16_b64", "whisper_small_f16_b16", "qwen3asr_bf16_b8"])
def test_graph_replay_equals_eager_launches(name):
    """wd_set_option(WD_OPT_GRAPHS): the captured-and-replayed step and the eagerly launched one
    run the same kernels in the same order, so logits and ids must be bit-identical; two
    contexts with the same weights and inputs step side by side, one with graphs, one
    without, at full batch and width (reduced depth and vocabulary)."""
    need_gpu()
    w0 = WL.by_name(name)
    kw = dict(layers=2, vocab=20011)
    if w0.arch == "whisper":
        kw["frames"] = 300
    w = WL.reduced(w0, **kw)
    W = WL.make_weights(w)
    A, E = GpuRun(w, W), GpuRun(w, W)
    E.dec.set_graphs(False)
    assert G_opt(E) == 0 and G_opt(A) == 1
    if w.arch == "whisper":
        enc = WL.make_encoder_states(w)
        A.cross(enc)
        E.cross(enc)
    ids = WL.random_ids(w, 6)
    for p in range(6):
        la, aa = A.step(ids[:, p], p)
        le, ae = E.step(ids[:, p], p)
        np.testing.assert_array_equal(la, le, err_msg=f"logits, position {p}")
        np.testing.assert_array_equal(aa, ae, err_msg=f"argmax, position {p}")
    assert A.check() == 0 and E.check() == 0
    with pytest.raises(A.K.WdError):
        A.K.wd_set_option(A.dec.ctx, A.K.WD_OPT_GRAPHS, 2)
    A.close()
    E.close()


def G_opt(G):
    return G.K.wd_get_option(G.dec.ctx, G.K.WD_OPT_GRAPHS)


def test_out_of_range_inputs_set_device_flag():
    need_gpu()
    w = WL.reduced(WL.by_name("whisper_tiny_f32_b1"), layers=1, vocab=2000, context=16, batch=2,
                   n_enc=2)
    W = WL.make_weights(w)
    enc = WL.make_encoder_states(w)
    G = GpuRun(w, W)
    G.cross(enc)
    G.step([1, 2], 0)
    assert G.check() == 0
    G.step([1, 2], [1, 16])            # position == context: flagged, cache write skipped
    assert G.check() == 3
    assert "position" in G.dec.last_error()
    G.step([1, 2000], 1)               # token == vocab
    assert G.check() == 3
    G.step([1, -1], 1)
    assert G.check() == 3
    G.step([3, 4], 2)                  # the flag clears after a check
    assert G.check() == 0
    G.close()


def test_step_before_cross_kv_is_a_state_error():
    need_gpu()
    import kv_cached_autoregressive_amd as K
    w = WL.reduced(WL.by_name("whisper_tiny_f32_b1"), layers=1, vocab=500)
    dec = K.Decoder(w, WL.make_weights(w))
    t = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(K.WdError) as e:
        dec.step(t, t)
    assert e.value.status == 2
    with pytest.raises(K.WdError):
        dec.reorder([0], 1)            # no spare cache for a single row
    dec.close()

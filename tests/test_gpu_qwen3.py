"""GPU parity of the Qwen3-ASR decoder step and prompt prefill (audio rows
spliced into the prompt) against the oracle."""
import numpy as np
import pytest
import torch

import workloads as WL
from oracle import qwen3 as OQ

from .gpu_helpers import GpuRun, check_device_argmax, compare_logits, need_gpu, say, to_dev, torch_dtype

pytestmark = pytest.mark.gpu


def _qwen_parity(w, T, steps, streams):
    """Prefill T rows (audio at rows audio_offset.. of the workload, clipped to T)
    on all rows, then `steps` teacher-forced decode steps; the sampled rows are
    compared at the prefill's last position and at every decode step.  The argmax
    the prefill and every step return is checked for every row against the logits
    they wrote, and for the sampled rows against the oracle's."""
    need_gpu()
    say(f"[qwen3] {w.describe()} T={T} steps={steps} rows={streams}")
    W = WL.make_weights(w)
    ids, audio = WL.make_qwen_prefill(w)
    off = w.audio_offset
    A = max(0, min(w.audio_rows, T - off))
    ids = ids[:, :T]
    audio = audio[:, :A]
    dec_ids = WL.random_ids(w, steps)
    G = GpuRun(w, W)
    tok = torch.from_numpy(np.ascontiguousarray(ids)).to(device="cuda", dtype=torch.int32)
    emb = to_dev(audio, torch_dtype(w.w_dtype)) if A > 0 else None
    logits = torch.empty(w.batch, w.vocab, dtype=torch.float32, device="cuda")
    _, pam = G.dec.prefill(tok, emb, off, logits)
    check_device_argmax(logits, pam, "prefill")
    pam = pam.cpu().numpy()
    got = {b: [logits[b].cpu().numpy()] for b in streams}
    amx = {b: [pam[b]] for b in streams}
    for s in range(steps):
        lg, am = G.step(dec_ids[:, s], T + s, rows=list(streams), check_all=True)
        for i, b in enumerate(streams):
            got[b].append(lg[i])
            amx[b].append(am[b])
    assert G.check() == 0
    G.close()
    del G
    torch.cuda.empty_cache()
    D = OQ.dims_of(w)
    worst = 0.0
    for b in streams:
        say(f"  oracle full prefix, row {b}")
        seq = np.concatenate([ids[b], dec_ids[b]])
        ref = OQ.decode_full(D, W, seq, round_cache=True, embeds=audio[b] if A else None, offset=off)
        e, _ = compare_logits(w, np.stack(got[b]), ref[T - 1:], f"row {b}", gpu_argmax=np.array(amx[b]))
        worst = max(worst, e)
    say(f"  worst err {worst:.3e}")


@pytest.mark.slow
def test_qwen3_full_prefill_and_decode_sampled_rows():
    """The Qwen3-ASR workload at its full size: 28 layers, 8 rows, a 900-token prefill with
    750 audio rows at offset 10, then 124 decode steps to the context end; rows 0 and 7
    against the oracle's full-prefix recompute."""
    _qwen_parity(WL.by_name("qwen3asr_bf16_b8"), T=900, steps=124, streams=(0, 7))


def test_qwen3_reduced_layers_full_width():
    w = WL.reduced(WL.by_name("qwen3asr_bf16_b8"), layers=3)
    _qwen_parity(w, T=40, steps=6, streams=(0, 7))


def test_qwen3_small_dims_context_end():
    w = WL.reduced(WL.by_name("qwen3asr_bf16_b8"), layers=2, d=256, heads=4, kv_heads=2,
                   d_ff=512, vocab=7001, context=48, batch=3, audio_offset=3, audio_rows=9)
    _qwen_parity(w, T=20, steps=28, streams=(0, 1, 2))   # last step at position 47 = context - 1


def test_qwen3_split_k_above_16_rows():
    """20 rows: the q|k|v and gate|up projections finish their split-K partials in the
    finish kernel (store, SwiGLU), the o and down projections fold theirs into the next
    norm, including across the prefill's head-less positions."""
    w = WL.reduced(WL.by_name("qwen3asr_bf16_b8"), layers=2, d=512, heads=4, kv_heads=2, d_ff=1536,
                   vocab=7001, context=64, batch=20, audio_offset=2, audio_rows=6)
    _qwen_parity(w, T=16, steps=6, streams=(0, 19))


def test_qwen3_prefill_two_chunks_hd64_bf16_cache_gqa4():
    """Head dim 64, a bf16 cache and 4 query heads per kv head (the prefill attention's
    other instantiation), over two prefill chunks of 512 and 88 positions."""
    w = WL.reduced(WL.by_name("qwen3asr_bf16_b8"), layers=2, d=256, heads=8, kv_heads=2, head_dim=64,
                   cache_dtype="bf16", d_ff=512, vocab=7001, context=640, batch=2, audio_offset=5,
                   audio_rows=300)
    _qwen_parity(w, T=600, steps=4, streams=(0, 1))


@pytest.mark.parametrize("batch", [6, 64])
def test_qwen3_gqa8_decode_attention(batch):
    """8 query heads per kv head: the decode attention serves all 8 from one block (8 queries
    per block), split over rows in 8-wave blocks at 6 rows (48 slabs) and unsplit in 4-wave
    blocks at 64 rows (512 slabs, 2 rows per pass per lane)."""
    w = WL.reduced(WL.by_name("qwen3asr_bf16_b8"), layers=1, d=256, heads=64, kv_heads=8, head_dim=64,
                   d_ff=512, vocab=7001, context=40, batch=batch, audio_offset=2, audio_rows=6)
    _qwen_parity(w, T=12, steps=4, streams=(0, batch - 1))


def test_qwen3_prefill_mha_odd_rows():
    """One query head per kv head (no GQA) and 3 streams of 70 positions: the prefill
    attention's query tiles mix positions across a partial last block."""
    w = WL.reduced(WL.by_name("qwen3asr_bf16_b8"), layers=2, d=256, heads=4, kv_heads=4, d_ff=512, vocab=7001,
                   context=96, batch=3, audio_offset=4, audio_rows=30)
    _qwen_parity(w, T=70, steps=3, streams=(0, 2))


def test_qwen3_argmax_exact_ties_full_vocab():
    """Exact ties through the 16-bit tied head over the full 151936-id vocabulary at 8 rows:
    every embedding row equals row 7 except ids 100000, 100001 and 151935 (twice row 7), so
    each row's logits take two values; the argmax is 100000 where those win and 0 otherwise
    (lowest index on ties, across every output block of the head)."""
    need_gpu()
    w = WL.reduced(WL.by_name("qwen3asr_bf16_b8"), layers=1, d=256, heads=4, kv_heads=2, d_ff=512, context=16)
    top = [100000, 100001, 151935]
    W = WL.make_weights(w)
    E = W["embed"].copy()
    E[:] = E[7]
    for t in top:
        E[t] = 2 * E[7]
    W["embed"] = E
    O = OQ.QwenOracle(OQ.dims_of(w), W, round_cache=True)
    O.reset(w.batch)
    G = GpuRun(w, W)
    ids = WL.random_ids(w, 4)
    decided = 0
    for p in range(4):
        ref = O.step(ids[:, p], [p] * w.batch)
        lg, am = G.step(ids[:, p], p, check_all=True)
        for t in top[1:]:
            np.testing.assert_array_equal(lg[:, t], lg[:, top[0]], err_msg=f"tied logits, pos {p}")
        hi, lo = ref[:, top[0]], ref[:, 0]
        want = np.where(hi - lo > 1e-2, top[0], np.where(lo - hi > 1e-2, 0, -1))
        sel = want >= 0
        np.testing.assert_array_equal(am[sel], want[sel], err_msg=f"tie winner, pos {p}")
        decided += int(sel.sum())
    assert G.check() == 0
    G.close()
    say(f"  tie winners checked {decided}")
    assert decided > 0

"""Element-wise parity of the caches the GPU writes: the cross K/V from the
once-per-window projection (MFMA GEMM for f16/bf16, VALU for fp32) and the self
K/V rows appended by each step, against the oracle's rounded caches.

A cache element is a rounding of a float sum; the device rounds its fp32 sum,
the oracle its fp64 sum, so the two may land on different sides of a rounding
boundary when the sum is within fp32 error of it.  The bar: every element equal,
except a small fraction that differ by at most one unit in the last place of
the cache dtype (fp32 caches: within a few fp32 ulps of the row scale)."""
import numpy as np
import pytest
import torch

import workloads as WL
from oracle import whisper as OW

from .gpu_helpers import GpuRun, need_gpu, say

pytestmark = pytest.mark.gpu


def _ulp(r, dtype):
    a = np.abs(r)
    a = np.where(a == 0, 1e-30, a)
    e = np.floor(np.log2(a))
    if dtype == "bf16":
        return 2.0 ** (np.maximum(e, -126) - 7)
    if dtype == "f16":
        return 2.0 ** (np.maximum(e, -14) - 10)
    return 2.0 ** (e - 23)


def _cmp(g, r, dtype, what, max_frac):
    g = np.asarray(g, np.float64)
    diff = np.abs(g - r)
    if dtype == "f32":
        scale = np.abs(r).max()
        bad = diff > 1e-5 * scale
        assert not bad.any(), f"{what}: {bad.sum()} elements off by > 1e-5 of the block scale"
        return 0.0
    mism = diff > 0
    frac = mism.mean()
    # one ulp of the cache dtype, plus the fp32 accumulation error of the sum (absolute,
    # a few fp32 ulps of the block scale) which dominates for values near zero
    allow = _ulp(r, dtype) * 1.0001 + 4e-6 * np.abs(r).max()
    over = diff > allow
    if over.any():
        i = np.argmax(diff - allow)
        raise AssertionError(f"{what}: {over.sum()} differences above one ulp; worst gpu {g.flat[i]:.6e} "
                             f"oracle {r.flat[i]:.6e} diff {diff.flat[i]:.3e} allowed {allow.flat[i]:.3e}")
    assert frac <= max_frac, f"{what}: {frac:.2e} of elements differ (by one ulp)"
    return frac


@pytest.mark.parametrize("w_dtype,cache_dtype,batch,frames",
                         [("bf16", "bf16", 3, 333), ("f16", "f16", 3, 333), ("f32", "f32", 3, 333),
                          ("bf16", "f16", 3, 333), ("f32", "bf16", 3, 333),
                          ("bf16", "bf16", 24, 333), ("f16", "f16", 40, 333),
                          ("bf16", "bf16", 64, 1500), ("f16", "f16", 48, 1500)])
def test_cross_and_self_caches_match_oracle(w_dtype, cache_dtype, batch, frames):
    """Above 16 rows the q|k|v projection is split over K groups and the self-attention
    kernel appends the k, v row from the partials: the rows must round the same way.
    The 1500-frame cases give the cross K/V GEMM its 256-row, LDS-staged blocks (at
    least 512 of them; 72000 rows leave a partial last block)."""
    need_gpu()
    w = WL.reduced(WL.by_name("whisper_large_bf16_b64"), layers=2, batch=batch, n_enc=batch, d=384, heads=6,
                   kv_heads=6, d_ff=768, vocab=3001, w_dtype=w_dtype, cache_dtype=cache_dtype,
                   frames=frames)
    say(f"[caches] {w.describe()}")
    W = WL.make_weights(w)
    enc = WL.make_encoder_states(w)
    O = OW.WhisperOracle(OW.dims_of(w), W)
    O.cross_kv(enc)
    O.reset(w.batch, enc_of=range(w.batch))
    G = GpuRun(w, W)
    G.cross(enc)
    worst = 0.0
    for l in range(w.layers):
        for which, ref in ((2, O.Kc[l]), (3, O.Vc[l])):
            g = G.dec.cache(which, l).float().cpu().numpy()[:, :, :w.frames]
            r = ref.reshape(w.n_enc, w.frames, w.heads, w.head_dim).transpose(0, 2, 1, 3)
            worst = max(worst, _cmp(g, r, cache_dtype, f"cross {'KV'[which - 2]} layer {l}", 2e-3))
    ids = WL.random_ids(w, 5)
    for p in range(5):
        O.step(ids[:, p], np.full(w.batch, p))
        G.step(ids[:, p], p)
        # layer 0 sees identical inputs up to fp32 rounding: rows must match
        for which, arr in ((0, O.Ks[0]), (1, O.Vs[0])):
            g = G.dec.cache(which, 0).float().cpu().numpy()[:, :, :p + 1]
            r = arr[:, :p + 1].reshape(w.batch, p + 1, w.heads, w.head_dim).transpose(0, 2, 1, 3)
            worst = max(worst, _cmp(g, r, cache_dtype, f"self {'KV'[which]} pos {p}", 2e-2))
    G.close()
    say(f"  largest one-ulp fraction {worst:.2e}")


@pytest.mark.parametrize("name", ["whisper_large_bf16_b64", "whisper_small_f16_b16"])
def test_cross_kv_full_size_sampled_rows(name):
    """The cross K/V projection at the full benchmark shapes (large-v3: 96000 x 1280 x 2560,
    256 x 256 blocks; whisper-small: 24000 x 768 x 1536, 256 x 128 blocks), one layer, in
    the launch configuration of the benchmark: sampled rows of both caches, every column,
    against the oracle's projection of the same rows (each cache row depends only on its
    own encoder row).  The rows cover the first and last sets, the first and last frames and
    256-row panel edges."""
    need_gpu()
    base = WL.by_name(name)
    w = WL.reduced(base, layers=1)
    say(f"[cross K/V full size] {w.describe()}")
    W = WL.make_weights(w)
    enc = WL.make_encoder_states(w)
    G = GpuRun(w, W)
    G.cross(enc)
    rng = np.random.default_rng(5)
    sets = sorted({0, 1, w.n_enc // 2, w.n_enc - 2, w.n_enc - 1})
    frames = sorted({0, 1, 255, 256, 511, 777, 1023, 1024, w.frames - 2, w.frames - 1,
                     *rng.integers(0, w.frames, 12).tolist()})
    O = OW.WhisperOracle(OW.dims_of(w), W)
    O.cross_kv([enc[e][frames] for e in sets])
    worst = 0.0
    fi = torch.tensor(frames, device="cuda")
    for which, ref in ((2, O.Kc[0]), (3, O.Vc[0])):
        c = G.dec.cache(which, 0)
        for k, e in enumerate(sets):
            g = c[e].index_select(1, fi).float().cpu().numpy()          # [H, n_frames, hd]
            g = g.transpose(1, 0, 2).reshape(len(frames), w.d)
            worst = max(worst, _cmp(g, ref[k], w.cache_dtype, f"cross {'KV'[which - 2]} set {e}", 2e-3))
    assert G.check() == 0
    G.close()
    say(f"  {len(sets)} sets x {len(frames)} frames x {2 * w.d} columns; largest one-ulp fraction {worst:.2e}")

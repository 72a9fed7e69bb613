"""GPU parity of the audio encoder (wd_load_encoder / wd_encode) against the oracle's
encoder: the convolution stem over 3000 mel frames, 1500 states, two pre-LN layers."""
import numpy as np
import pytest
import torch

import workloads as WL
from oracle import encoder as OE

from .gpu_helpers import GpuRun, need_gpu, say, torch_dtype

pytestmark = pytest.mark.gpu


def _enc_weights(d, mels, layers, d_ff, P, dtype, seed=7):
    """Seeded N(0, 0.02) matrices, N(0, 1) positions, 1 + N(0, 0.02) gains, N(0, 0.02) biases,
    rounded to the weight dtype (both sides use the rounded values)."""
    rng = np.random.default_rng(seed)
    W = {"enc.conv1.w": rng.normal(0, 0.02, (d, mels, 3)), "enc.conv1.b": rng.normal(0, 0.02, d),
         "enc.conv2.w": rng.normal(0, 0.02, (d, d, 3)), "enc.conv2.b": rng.normal(0, 0.02, d),
         "enc.pos": rng.normal(0, 1, (P, d)),
         "enc.ln_post.g": 1 + rng.normal(0, 0.02, d), "enc.ln_post.b": rng.normal(0, 0.02, d)}
    for i in range(layers):
        p = f"enc.{i}."
        for ln in ("ln1", "ln2"):
            W[p + ln + ".g"] = 1 + rng.normal(0, 0.02, d)
            W[p + ln + ".b"] = rng.normal(0, 0.02, d)
        for proj in ("q", "k", "v", "o"):
            W[p + f"attn.{proj}.w"] = rng.normal(0, 0.02, (d, d))
            if proj != "k":
                W[p + f"attn.{proj}.b"] = rng.normal(0, 0.02, d)
        W[p + "fc1.w"] = rng.normal(0, 0.02, (d_ff, d))
        W[p + "fc1.b"] = rng.normal(0, 0.02, d_ff)
        W[p + "fc2.w"] = rng.normal(0, 0.02, (d, d_ff))
        W[p + "fc2.b"] = rng.normal(0, 0.02, d)
    td = torch_dtype(dtype)
    return {k: torch.from_numpy(v).to(td).double().numpy() for k, v in W.items()}


@pytest.mark.parametrize("w_dtype", ["bf16", "f16"])
def test_encoder_3000_frames_two_sets(w_dtype):
    need_gpu()
    base = WL.by_name("whisper_large_bf16_b64" if w_dtype == "bf16" else "whisper_small_f16_b16")
    w = WL.reduced(base, layers=1, batch=2, n_enc=2, d=256, heads=4, kv_heads=4, d_ff=512, vocab=3001)
    mels, frames, layers, d_ff, n_sets = 80, 3000, 2, 1024, 2
    P = (frames - 1) // 2 + 1
    say(f"[encoder] d={w.d} heads={w.heads} mels={mels} frames={frames} layers={layers} sets={n_sets} {w_dtype}")
    W = _enc_weights(w.d, mels, layers, d_ff, P, w_dtype)
    td = torch_dtype(w_dtype)
    mel = torch.from_numpy(np.random.default_rng(8).standard_normal((n_sets, frames, mels))).to(td)
    G = GpuRun(w, WL.make_weights(w))
    G.dec.load_encoder(W, mels, frames, layers, d_ff, max_sets=n_sets)
    out = G.dec.encode(mel.cuda()).float().cpu().numpy()
    torch.cuda.synchronize()
    assert out.shape == (n_sets, P, w.d)
    worst, rms, scale = 0.0, 0.0, 0.0
    for e in range(n_sets):
        ref = OE.encode(W, mel[e].double().numpy(), w.heads, layers)
        err = np.abs(out[e] - ref)
        worst = max(worst, float(err.max()))
        scale = max(scale, float(np.abs(ref).max()))
        rms = max(rms, float(np.sqrt((err ** 2).mean()) / np.sqrt((ref ** 2).mean())))
    say(f"  max abs err {worst:.3e} (max |ref| {scale:.2f}), relative rms err {rms:.3e}")
    # the output is rounded to the weight dtype (relative 2^-8 for bf16, 2^-11 for f16) and the
    # attention reads K and V rounded to it: errors of a few units of that rounding
    unit = 2.0 ** -8 if w_dtype == "bf16" else 2.0 ** -11
    assert rms < 4 * unit, rms
    assert worst < 8 * unit * scale, worst
    assert G.check() == 0
    G.close()


def test_listen_equals_encode_then_cross_kv():
    """wd_listen is wd_encode of every set followed by wd_cross_kv of its states: the step
    after it gives the same logits, bit for bit, as the step after the two separate calls
    (each of those is checked against the oracle on its own).  Before an encoder is loaded
    it is refused."""
    need_gpu()
    K = pytest.importorskip("kv_cached_autoregressive_amd")
    base = WL.by_name("whisper_large_bf16_b64")
    w = WL.reduced(base, layers=2, batch=4, n_enc=2, d=256, heads=4, kv_heads=4, d_ff=512, vocab=3001)
    mels, frames, layers, d_ff = 80, 3000, 1, 1024
    P = (frames - 1) // 2 + 1
    say(f"[listen] d={w.d} mels={mels} frames={frames} layers={layers} sets={w.n_enc} batch={w.batch}")
    W = _enc_weights(w.d, mels, layers, d_ff, P, w.w_dtype, seed=11)
    td = torch_dtype(w.w_dtype)
    mel = torch.from_numpy(np.random.default_rng(12).standard_normal((w.n_enc, frames, mels))).to(td).cuda()
    G = GpuRun(w, WL.make_weights(w))
    with pytest.raises(K.WdError):
        G.dec.listen(mel)
    G.dec.load_encoder(W, mels, frames, layers, d_ff, max_sets=w.n_enc)
    toks = np.arange(w.batch) * 7 + 3
    G.dec.listen(mel)
    torch.cuda.synchronize()
    lg1, am1 = G.step(toks, 0)
    states = G.dec.encode(mel)
    G.dec.cross_kv(states, P)
    torch.cuda.synchronize()
    lg2, am2 = G.step(toks, 0)
    assert np.all(np.isfinite(lg1))
    assert np.array_equal(lg1, lg2) and np.array_equal(am1, am2)
    assert G.check() == 0
    G.close()


def test_encoder_large_v3_dims_one_layer():
    """The encoder at the large-v3 widths the decoder benchmark runs behind (d = 1280, 20
    heads, 128 mels, d_ff = 5120), one layer, 3000 frames, one set: every output compared
    with the oracle's."""
    need_gpu()
    base = WL.by_name("whisper_large_bf16_b64")
    w = WL.reduced(base, layers=1, batch=1, n_enc=1, vocab=3001)
    assert (w.d, w.heads) == (1280, 20)
    mels, frames, layers, d_ff = 128, 3000, 1, 5120
    P = (frames - 1) // 2 + 1
    say(f"[encoder large-v3 dims] d={w.d} heads={w.heads} mels={mels} frames={frames} layers={layers}")
    W = _enc_weights(w.d, mels, layers, d_ff, P, w.w_dtype, seed=21)
    td = torch_dtype(w.w_dtype)
    mel = torch.from_numpy(np.random.default_rng(22).standard_normal((1, frames, mels))).to(td)
    G = GpuRun(w, WL.make_weights(w))
    G.dec.load_encoder(W, mels, frames, layers, d_ff, max_sets=1)
    out = G.dec.encode(mel.cuda()).float().cpu().numpy()
    torch.cuda.synchronize()
    ref = OE.encode(W, mel[0].double().numpy(), w.heads, layers)
    err = np.abs(out[0] - ref)
    scale = float(np.abs(ref).max())
    rms = float(np.sqrt((err ** 2).mean()) / np.sqrt((ref ** 2).mean()))
    say(f"  max abs err {float(err.max()):.3e} (max |ref| {scale:.2f}), relative rms err {rms:.3e}")
    unit = 2.0 ** -8   # bf16 output and K/V rounding, as in the two-set test
    assert rms < 4 * unit, rms
    assert float(err.max()) < 8 * unit * scale, float(err.max())
    assert G.check() == 0
    G.close()

"""wd_topk_noalloc (the allocation-free beam-candidate entry point, scratch in a static device
array) against wd_topk (the context entry point, scratch in the caller's workspace): the same
kernels on the same logits must give bit-identical candidates and log-sum-exp, on two calls in
a row (the second smaller) and on a strided logits buffer."""
import numpy as np
import pytest
import torch

import workloads as WL

from .gpu_helpers import need_gpu, say

pytestmark = pytest.mark.gpu


def _logits(rng, B, V, ld=None):
    ld = V if ld is None else ld
    x = (rng.standard_normal((B, ld)) * 3).astype(np.float32)
    x[0, [5, 17, V - 1]] = 20.0          # exact ties: lowest id first
    if B > 2:
        x[1, :V] = 1.0                   # a row of equal values
        x[2, [3, 99]] = np.nan           # NaN: never picked, left out of the log-sum-exp
    return torch.from_numpy(x).cuda()


def _noalloc(K, lg, B, V, ld, W):
    vals = torch.full((B, W), -7.0, dtype=torch.float32, device="cuda")
    ids = torch.full((B, W), -7, dtype=torch.int32, device="cuda")
    lse = torch.full((B,), -7.0, dtype=torch.float32, device="cuda")
    K.wd_topk_noalloc(lg.data_ptr(), B, V, ld, W, vals.data_ptr(), ids.data_ptr(), lse.data_ptr(),
                      torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return vals.cpu().numpy(), ids.cpu().numpy(), lse.cpu().numpy()


def _with_context(dec, lg, W):
    v, i, l = dec.topk(lg, W)
    torch.cuda.synchronize()
    return v.cpu().numpy(), i.cpu().numpy(), l.cpu().numpy()


def _same(a, b, what):
    for x, y, n in zip(a, b, ("values", "ids", "lse")):
        np.testing.assert_array_equal(x, y, err_msg=f"{what}: {n}")


def test_topk_noalloc_matches_context_entry_point():
    need_gpu()
    import kv_cached_autoregressive_amd as K
    rng = np.random.default_rng(7)
    big = WL.reduced(WL.by_name("whisper_large_bf16_b64"), layers=1, d=256, heads=4, kv_heads=4, d_ff=512, frames=32)
    small = WL.reduced(WL.by_name("whisper_tiny_f32_b1"), layers=1, vocab=3001, batch=5, n_enc=5)
    say("[no-alloc] loading two contexts")
    d_big = K.Decoder(big, WL.make_weights(big))
    d_small = K.Decoder(small, WL.make_weights(small))
    # first call: 64 rows over 51866 ids, W = 8
    lg = _logits(rng, 64, big.vocab)
    say("[no-alloc] call 1: 64 x 51866, W 8")
    _same(_noalloc(K, lg, 64, big.vocab, big.vocab, 8), _with_context(d_big, lg, 8), "64 x 51866, W 8")
    # second call, smaller: 5 rows over 3001 ids, W = 5 (the scratch keeps the first call's lists)
    lg = _logits(rng, 5, small.vocab)
    say("[no-alloc] call 2: 5 x 3001, W 5")
    _same(_noalloc(K, lg, 5, small.vocab, small.vocab, 5), _with_context(d_small, lg, 5), "5 x 3001, W 5")
    # rows of 3001 logits in a buffer of 4000 columns
    wide = _logits(rng, 3, small.vocab, ld=4000)
    say("[no-alloc] call 3: 3 x 3001 in rows of 4000, W 4")
    got = _noalloc(K, wide, 3, small.vocab, 4000, 4)
    ref = _with_context(d_small, wide[:, :small.vocab].contiguous(), 4)
    _same(got, (ref[0][:3], ref[1][:3], ref[2][:3]), "3 x 3001 in rows of 4000, W 4")
    # sizes beyond the static scratch are refused before any launch
    with pytest.raises(K.WdError) as e:
        K.wd_topk_noalloc(lg.data_ptr(), 65, small.vocab, small.vocab, 5, 1, 1, 1)
    assert e.value.status == 1 and "scratch" in str(e.value)
    with pytest.raises(K.WdError):
        K.wd_topk_noalloc(lg.data_ptr(), 5, small.vocab, small.vocab - 1, 5, 1, 1, 1)
    d_big.close()
    d_small.close()


"""Helpers of the GPU parity tests: drive the HIP path through the C ABI binding
and compare against the oracle on the same seeded inputs.

Tolerances (the decoder's stated parity bar):
  * fp32 mode: per row max|gpu - oracle| / max|oracle| <= 1e-4;
  * f16 / bf16 modes: max|gpu - oracle| <= 2e-2 absolute per logit;
  * argmax ids (and beam choices) identical wherever the oracle's top-2 logit
    margin (score gap) exceeds 1e-2.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from oracle.numerics import argmax_lowest, top2_margin

REL_F32 = 1e-4
ABS_16 = 2e-2
MARGIN = 1e-2


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cached_autoregressive_amd as K
    K.lib()  # raises when the library is missing: no fallback


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_dtype(name):
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[name]


def to_dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device="cuda", dtype=dtype)


def compare_logits(w, gpu, ref, where=""):
    """gpu (float32) and ref (float64) logits [..., V]; asserts the parity bar and
    returns (max error, argmax rows checked)."""
    gpu = np.asarray(gpu, np.float64).reshape(-1, ref.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    assert np.all(np.isfinite(gpu)), f"non-finite GPU logits {where}"
    if w.w_dtype == "f32" and w.cache_dtype == "f32":
        err = np.abs(gpu - ref).max(-1) / np.abs(ref).max(-1)
        bad = np.nonzero(err > REL_F32)[0]
        assert bad.size == 0, f"{where}: row rel err {err.max():.3e} > {REL_F32} at rows {bad[:8]}"
        emax = float(err.max())
    else:
        err = np.abs(gpu - ref).max(-1)
        bad = np.nonzero(err > ABS_16)[0]
        assert bad.size == 0, f"{where}: abs err {err.max():.3e} > {ABS_16} at rows {bad[:8]}"
        emax = float(err.max())
    m = top2_margin(ref)
    sel = m > MARGIN
    ga, oa = argmax_lowest(gpu), argmax_lowest(ref)
    mism = np.nonzero(sel & (ga != oa))[0]
    assert mism.size == 0, f"{where}: argmax differs at rows {mism[:8]} (margins {m[mism[:8]]})"
    return emax, int(sel.sum())


class GpuRun:
    """A loaded decoder plus device buffers for teacher-forced stepping."""

    def __init__(self, w, weights):
        import kv_cached_autoregressive_amd as K
        self.K = K
        self.w = w
        self.dec = K.Decoder(w, weights)
        B = w.batch
        self.tok = torch.zeros(B, dtype=torch.int32, device="cuda")
        self.pos = torch.zeros(B, dtype=torch.int32, device="cuda")
        self.logits = torch.empty(B, w.vocab, dtype=torch.float32, device="cuda")
        self.amax = torch.empty(B, dtype=torch.int32, device="cuda")

    def cross(self, enc, frames=None):
        """enc [n_enc, >= frames, d]; the library takes [n_enc, frames, d] contiguous."""
        F = enc.shape[1] if frames is None else frames
        e = to_dev(np.ascontiguousarray(enc[:, :F]), torch_dtype(self.w.w_dtype))
        self.dec.cross_kv(e, F)
        torch.cuda.synchronize()

    def step(self, tokens, pos, rows=None, B=None):
        """Feeds tokens [B] at position(s) pos; returns (logits of `rows`, argmax)."""
        B = self.w.batch if B is None else B
        self.tok[:B].copy_(torch.as_tensor(np.asarray(tokens, np.int32)))
        p = np.broadcast_to(np.asarray(pos, np.int32), (B,))
        self.pos[:B].copy_(torch.as_tensor(np.ascontiguousarray(p)))
        self.dec.step(self.tok[:B], self.pos[:B], self.logits[:B], self.amax[:B])
        lg = self.logits[:B] if rows is None else self.logits[rows]
        return lg.cpu().numpy(), self.amax[:B].cpu().numpy()

    def check(self):
        return self.dec.check()

    def close(self):
        self.dec.close()

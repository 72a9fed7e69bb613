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


def compare_logits(w, gpu, ref, where="", gpu_argmax=None):
    """gpu (float32) and ref (float64) logits [..., V]; asserts the parity bar and
    returns (max error, argmax rows checked).  gpu_argmax: the ids the library
    returned for these rows, which must equal the lowest-index argmax of its own
    logits everywhere and the oracle's wherever the oracle's top-2 margin exceeds
    the bar."""
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
    if gpu_argmax is not None:
        da = np.asarray(gpu_argmax, np.int32).reshape(-1)
        bad = np.nonzero(da != ga)[0]
        assert bad.size == 0, f"{where}: device argmax {da[bad[:8]]} != argmax of its logits {ga[bad[:8]]}"
        mism = np.nonzero(sel & (da != oa))[0]
        assert mism.size == 0, f"{where}: device argmax differs from the oracle's at rows {mism[:8]}"
    return emax, int(sel.sum())


def check_device_argmax(logits, amax, where=""):
    """Every row: the id the library returned equals the lowest-index argmax of the
    logits it wrote (device tensors [B, V] fp32 and [B] int32)."""
    lg = logits.cpu().numpy()
    want = argmax_lowest(lg)
    got = amax.cpu().numpy()
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{where}: device argmax {got[bad[:8]]} != argmax of its logits {want[bad[:8]]} at rows {bad[:8]}"


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

    def step(self, tokens, pos, rows=None, B=None, check_all=False):
        """Feeds tokens [B] at position(s) pos; returns (logits of `rows`, argmax of all B
        rows).  check_all: also assert, for every row, that the returned argmax is the
        lowest-index argmax of the logits the step wrote."""
        B = self.w.batch if B is None else B
        self.tok[:B].copy_(torch.as_tensor(np.asarray(tokens, np.int32)))
        p = np.broadcast_to(np.asarray(pos, np.int32), (B,))
        self.pos[:B].copy_(torch.as_tensor(np.ascontiguousarray(p)))
        self.dec.step(self.tok[:B], self.pos[:B], self.logits[:B], self.amax[:B])
        if check_all:
            check_device_argmax(self.logits[:B], self.amax[:B], f"position(s) {np.unique(p)}")
        lg = self.logits[:B] if rows is None else self.logits[rows]
        return lg.cpu().numpy(), self.amax[:B].cpu().numpy()

    def check(self):
        return self.dec.check()

    def close(self):
        self.dec.close()

"""The machine-floor probe (wd_probe) that bench.py --floors reports: every kind runs through the
C ABI and returns a plausible per-launch time on the device."""
import pytest
import torch

import kv_cached_autoregressive_amd as K
from .gpu_helpers import need_gpu, say

pytestmark = pytest.mark.gpu


def test_probe_empty_launch_and_stream():
    need_gpu()
    say("[wd_probe] kind 0 (200 launches), kind 1 (2 x 64 MiB, 5 launches)")
    launch = K.wd_probe(0, iters=200)
    assert 0.1 < launch < 100.0, launch
    n = 64 << 20
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.ones(n, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4096, dtype=torch.float32, device="cuda")
    us = K.wd_probe(1, a.data_ptr(), b.data_ptr(), n, 5, sink.data_ptr())
    rate = 2 * n / us / 1e3   # bytes per us / 1000 = GB/s
    assert 500.0 < rate < 9000.0, rate
    # hand-offs between dependent launches (same and other XCD), fence reductions in a kernel
    for kind in (2, 3):
        t = K.wd_probe(kind, a.data_ptr(), b.data_ptr(), 327680, 100)
        assert 0.1 < t < 200.0, (kind, t)
    ctr = torch.zeros(2, dtype=torch.int32, device="cuda")
    for kind in (4, 5):
        t = K.wd_probe(kind, a.data_ptr(), ctr.data_ptr(), 4096, 20)
        assert 0.1 < t < 2000.0, (kind, t)
    torch.cuda.synchronize()
    assert int(ctr[0].item()) == 0   # the last block re-arms the counter
    # the reduction's sum of block indices 0..1023
    assert float(ctr.view(torch.float32)[1].item()) == 1023 * 1024 / 2
    with pytest.raises(K.WdError):
        K.wd_probe(1, a.data_ptr() + 8, b.data_ptr(), n - 16, 1, sink.data_ptr())

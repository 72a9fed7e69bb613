"""The machine-floor probe (wd_probe) that bench.py --floors reports: both kinds run through the
C ABI and return plausible per-launch times on the device."""
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
    torch.cuda.synchronize()
    with pytest.raises(K.WdError):
        K.wd_probe(1, a.data_ptr() + 8, b.data_ptr(), n - 16, 1, sink.data_ptr())

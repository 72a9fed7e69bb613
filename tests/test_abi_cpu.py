"""C ABI checks that need no GPU: the library loads, exports every function that
include/wd.h declares, sizes workspaces, and rejects bad arguments on the host
before any device work (fake device addresses are never dereferenced on these
paths)."""
import ctypes
import os

import numpy as np
import pytest

import kv_cached_autoregressive_amd as K
import workloads as WL

pytestmark = pytest.mark.skipif(not os.path.exists(K.lib_path()), reason="libwd.so not built")

FAKE_WS = 1 << 40          # aligned, never touched: every case below fails before launching
FAKE_DATA = 1 << 41


def test_exports_every_declared_symbol():
    L = ctypes.CDLL(K.lib_path())
    names = K.declared_functions()
    assert {"wd_load", "wd_cross_kv", "wd_step", "wd_reorder", "wd_prefill", "wd_check",
            "wd_free", "wd_workspace_bytes", "wd_last_error"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert K.wd_abi_version() == 5


def test_workspace_bytes_plan():
    for w in WL.WORKLOADS:
        n = K.wd_workspace_bytes(K.config_from(w))
        assert n > 0 and n % 256 == 0
    w = WL.by_name("whisper_large_bf16_b64")
    n = K.wd_workspace_bytes(K.config_from(w))
    cross = w.layers * 2 * w.n_enc * w.frames * w.d * 2
    self_c = w.layers * 2 * w.batch * w.context * w.d * 2
    assert cross + self_c < n < cross + self_c + 3 * 2**30
    # beams reserve a second self cache
    wb = WL.by_name("whisper_base_f16_beam5")
    one = WL.reduced(wb, n_enc=5)
    # (and one encoder-state operand copy per window, rows rounded up to 256)
    r128 = lambda n: (n + 255) // 256 * 256
    assert K.wd_workspace_bytes(K.config_from(wb)) - K.wd_workspace_bytes(K.config_from(one)) == \
        wb.layers * 2 * wb.batch * wb.context * wb.d * 2 - wb.layers * 2 * 4 * wb.frames * wb.d * 2 \
        - (r128(5 * wb.frames) - r128(wb.frames)) * wb.d * 2


@pytest.mark.parametrize("field,value", [("d_model", 0), ("d_model", 100), ("head_dim", 32),
                                         ("n_kv_heads", 5), ("max_batch", 65), ("max_batch", 0),
                                         ("w_dtype", 7), ("n_enc", 3), ("context", 0),
                                         ("norm_eps", 0.0), ("arch", 2)])
def test_invalid_configs_rejected(field, value):
    cfg = K.config_from(WL.by_name("whisper_small_f16_b16"))
    setattr(cfg, field, value)
    assert K.wd_workspace_bytes(cfg) == 0
    with pytest.raises(K.WdError) as e:
        K.wd_load(cfg, [], FAKE_WS, 1 << 40)
    assert e.value.status == 1


def _descs(w, drop=(), extra=(), numel_fix=None, dtype=None):
    out = []
    for name, shape, kind in WL.weight_specs(w):
        if name in drop:
            continue
        n = int(np.prod(shape))
        if numel_fix and name in numel_fix:
            n = numel_fix[name]
        dt = K.DTYPES[w.w_dtype] if dtype is None or kind != "mat" else dtype
        out.append(K.WdTensor(name.encode(), FAKE_DATA, n, dt))
    for name, n in extra:
        out.append(K.WdTensor(name.encode(), FAKE_DATA, n, 0))
    return out


def _load_err(w, descs, ws=FAKE_WS, nbytes=None):
    cfg = K.config_from(w)
    nbytes = K.wd_workspace_bytes(cfg) if nbytes is None else nbytes
    with pytest.raises(K.WdError) as e:
        K.wd_load(cfg, descs, ws, nbytes)
    return e.value


def test_load_argument_errors():
    w = WL.reduced(WL.by_name("whisper_tiny_f32_b1"), layers=2, vocab=1000)
    e = _load_err(w, _descs(w, extra=[("dec.0.self.k.b", w.d)]))
    assert e.status == 1 and "no bias" in str(e)
    e = _load_err(w, _descs(w, drop=("dec.1.fc2.w",)))
    assert e.status == 1 and "missing" in str(e)
    e = _load_err(w, _descs(w, extra=[("dec.0.mystery.w", 4)]))
    assert e.status == 1 and "unknown" in str(e)
    e = _load_err(w, _descs(w, numel_fix={"embed": 5}))
    assert e.status == 1 and "elements" in str(e)
    e = _load_err(w, _descs(w, dtype=1))
    assert e.status == 1 and "w_dtype" in str(e)
    e = _load_err(w, _descs(w), ws=FAKE_WS + 8)
    assert e.status == 1 and "aligned" in str(e)
    e = _load_err(w, _descs(w), nbytes=1024)
    assert e.status == 5
    q = WL.reduced(WL.by_name("qwen3asr_bf16_b8"), layers=1, vocab=1000)
    e = _load_err(q, _descs(q, drop=("dec.0.k_norm.g",)))
    assert e.status == 1 and "k_norm" in str(e)


def test_null_context_calls_return_arg():
    L = K.lib()
    assert L.wd_step(None, None, None, 1, None, None) == 1
    assert L.wd_cross_kv(None, None, 1) == 1
    assert L.wd_cross_kv_ragged(None, None, None) == 1
    assert L.wd_topk(None, None, 1, 1, None, None, None) == 1
    assert L.wd_encode(None, None, 1, None) == 1
    assert L.wd_listen(None, None) == 1
    assert L.wd_load_encoder(None, 80, 3000, 1, 128, 1, None, 0, None, 0) == 1
    assert L.wd_encoder_workspace_bytes(None, 80, 3000, 1, 128, 1) == 0
    assert L.wd_reorder(None, None, 1, 1) == 1
    assert L.wd_beam_step(None, None, 1, 0, None, None, None, 0) == 1
    assert L.wd_prefill(None, None, 1, 1, None, 0, 0, None, None) == 1
    assert L.wd_check(None) == 1
    assert L.wd_set_option(None, K.WD_OPT_GRAPHS, 0) == 1
    # the allocation-free candidates entry point checks its arguments before any device call
    fake = ctypes.c_void_p(FAKE_DATA)
    assert L.wd_topk_noalloc(None, 1, 10, 10, 1, fake, fake, fake, None) == 1
    assert L.wd_topk_noalloc(fake, 65, 10, 10, 1, fake, fake, fake, None) == 1
    assert "scratch" in K.wd_last_error(None)
    assert L.wd_topk_noalloc(fake, 4, 10, 9, 1, fake, fake, fake, None) == 1
    assert L.wd_topk_noalloc(fake, 4, 10, 10, 9, fake, fake, fake, None) == 1
    # the machine-floor probe checks its arguments before creating a stream
    us = ctypes.c_double()
    assert L.wd_probe(6, None, None, 0, 1, None, ctypes.byref(us)) == 1
    assert L.wd_probe(2, fake, fake, 4095, 1, None, ctypes.byref(us)) == 1
    assert L.wd_probe(3, fake, None, 4096, 1, None, ctypes.byref(us)) == 1
    assert L.wd_probe(4, fake, fake, 100, 1, None, ctypes.byref(us)) == 1
    assert L.wd_probe(5, fake, ctypes.c_void_p(FAKE_DATA + 4), 4096, 1, None, ctypes.byref(us)) == 1
    assert L.wd_probe(0, None, None, 0, 0, None, ctypes.byref(us)) == 1
    assert L.wd_probe(0, None, None, 0, 1, None, None) == 1
    assert L.wd_probe(1, None, fake, 1 << 20, 1, fake, ctypes.byref(us)) == 1
    assert L.wd_probe(1, fake, fake, 1000, 1, fake, ctypes.byref(us)) == 1
    assert L.wd_probe(1, ctypes.c_void_p(FAKE_DATA + 8), fake, 1 << 20, 1, fake, ctypes.byref(us)) == 1
    assert "wd_probe" in K.wd_last_error(None)
    v = ctypes.c_int32()
    assert L.wd_get_option(None, K.WD_OPT_GRAPHS, ctypes.byref(v)) == 1
    L.wd_free(None)

"""Python binding of the MI355X decoder-step library (``libwd.so``).

The functions below carry the names of the C ABI in ``include/wd.h`` and only
marshal arguments through ctypes; every step of the decoder runs in the
library's HIP kernels.  PyTorch is used for device memory and streams only
(``Decoder`` allocates the workspace and uploads weights with it).

The library must have been built (``python -m kv_cached_autoregressive_amd._build``
or ``__graft_entry__.build()``); importing a missing library raises at once --
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Dict, Iterable, Optional, Sequence

__all__ = [
    "WdError", "WdConfig", "WdTensor", "lib", "lib_path", "declared_functions",
    "wd_abi_version", "wd_workspace_bytes", "wd_load", "wd_cross_kv", "wd_cross_kv_ragged", "wd_step", "wd_reorder",
    "wd_topk", "wd_prefill", "wd_encoder_workspace_bytes", "wd_load_encoder", "wd_encode", "wd_listen", "wd_check", "wd_last_error", "wd_free", "wd_profile", "wd_profile_read", "wd_probe",
    "wd_debug_cache", "wd_set_option", "wd_get_option", "WD_OPT_GRAPHS", "wd_topk_noalloc", "wd_beam_step",
    "config_from", "Decoder", "DTYPES", "STATUS",
]

HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(HERE)
HEADER = os.path.join(_ROOT, "include", "wd.h")
DTYPES = {"f32": 0, "f16": 1, "bf16": 2}
ARCHS = {"whisper": 0, "qwen3": 1}
STATUS = {0: "WD_OK", 1: "WD_ERR_ARG", 2: "WD_ERR_STATE", 3: "WD_ERR_RANGE", 4: "WD_ERR_HIP",
          5: "WD_ERR_OOM", 6: "WD_ERR_INTERNAL"}
# kernel classes for wd_profile
K_CROSS_ATTN, K_SELF_ATTN, K_LOGITS, K_XKV_GEMM, K_FC1 = 0, 1, 2, 3, 4
# context options (wd_set_option)
WD_OPT_GRAPHS = 0


class WdError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class WdConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "arch", "d_model", "n_heads", "n_kv_heads", "head_dim", "n_layers", "d_ff", "vocab",
        "context", "max_frames", "max_batch", "n_enc", "w_dtype", "cache_dtype")] + [
        ("norm_eps", ctypes.c_float), ("rope_base", ctypes.c_float)]


class WdTensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("data", ctypes.c_void_p), ("numel", ctypes.c_int64),
                ("dtype", ctypes.c_int32)]


def lib_path() -> str:
    """The in-tree build, or the library the WD_LIB environment variable names (another build
    of the same sources, e.g. one compiled with different flags); there is no other fallback."""
    return os.environ.get("WD_LIB", os.path.join(HERE, "libwd.so"))


_LIB = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        p = lib_path()
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is missing: build it with `python -m kv_cached_autoregressive_amd._build`")
        L = ctypes.CDLL(p)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        sig = {
            "wd_abi_version": (i32, []),
            "wd_workspace_bytes": (sz, [ctypes.POINTER(WdConfig)]),
            "wd_load": (i32, [ctypes.POINTER(WdConfig), ctypes.POINTER(WdTensor), i32, vp, sz, vp,
                              ctypes.POINTER(vp)]),
            "wd_cross_kv": (i32, [vp, vp, i32]),
            "wd_cross_kv_ragged": (i32, [vp, vp, ctypes.POINTER(i32)]),
            "wd_step": (i32, [vp, vp, vp, i32, vp, vp]),
            "wd_reorder": (i32, [vp, ctypes.POINTER(i32), i32, i32]),
            "wd_topk": (i32, [vp, vp, i32, i32, vp, vp, vp]),
            "wd_beam_step": (i32, [vp, vp, i32, i32, vp, vp, vp, i32]),
            "wd_encoder_workspace_bytes": (sz, [vp, i32, i32, i32, i32, i32]),
            "wd_load_encoder": (i32, [vp, i32, i32, i32, i32, i32, ctypes.POINTER(WdTensor), i32, vp, sz]),
            "wd_encode": (i32, [vp, vp, i32, vp]),
            "wd_listen": (i32, [vp, vp]),
            "wd_prefill": (i32, [vp, vp, i32, i32, vp, i32, i32, vp, vp]),
            "wd_check": (i32, [vp]),
            "wd_last_error": (ctypes.c_char_p, [vp]),
            "wd_free": (None, [vp]),
            "wd_profile": (i32, [vp, i32, i32, i32]),
            "wd_profile_read": (i32, [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]),
            "wd_probe": (i32, [i32, vp, vp, i64, i32, vp, ctypes.POINTER(ctypes.c_double)]),
            "wd_debug_cache": (i32, [vp, i32, i32, ctypes.POINTER(vp)]),
            "wd_set_option": (i32, [vp, i32, i32]),
            "wd_topk_noalloc": (i32, [vp, i32, i32, i64, i32, vp, vp, vp, vp]),
            "wd_get_option": (i32, [vp, i32, ctypes.POINTER(i32)]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _LIB = L
    return _LIB


def declared_functions() -> list:
    """Names of the functions include/wd.h declares."""
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(wd_[a-z_]+)\s*\(", txt)))


def _check(st: int, ctx=None):
    if st != 0:
        raise WdError(st, wd_last_error(ctx))


# ---- the C ABI, one wrapper per entry point --------------------------------------------------

def wd_abi_version() -> int:
    return lib().wd_abi_version()


def wd_workspace_bytes(cfg: WdConfig) -> int:
    return lib().wd_workspace_bytes(ctypes.byref(cfg))


def wd_load(cfg: WdConfig, tensors: Sequence[WdTensor], workspace: int, ws_bytes: int,
            stream: int = 0):
    arr = (WdTensor * max(1, len(tensors)))(*tensors)
    out = ctypes.c_void_p()
    st = lib().wd_load(ctypes.byref(cfg), arr if tensors else None, len(tensors),
                       ctypes.c_void_p(workspace), ws_bytes, ctypes.c_void_p(stream), ctypes.byref(out))
    _check(st)
    return out.value


def wd_cross_kv(ctx, enc: int, frames: int):
    _check(lib().wd_cross_kv(ctx, ctypes.c_void_p(enc), frames), ctx)


def wd_cross_kv_ragged(ctx, enc: int, frames: Iterable[int]):
    f = [int(x) for x in frames]
    arr = (ctypes.c_int32 * max(1, len(f)))(*f)
    _check(lib().wd_cross_kv_ragged(ctx, ctypes.c_void_p(enc), arr), ctx)


def wd_step(ctx, tokens: int, positions: int, B: int, logits: int, argmax: int):
    _check(lib().wd_step(ctx, ctypes.c_void_p(tokens), ctypes.c_void_p(positions), B,
                         ctypes.c_void_p(logits) if logits else None, ctypes.c_void_p(argmax)), ctx)


def wd_reorder(ctx, beam_idx: Iterable[int], n_rows: int):
    idx = list(beam_idx)
    arr = (ctypes.c_int32 * max(1, len(idx)))(*idx)
    _check(lib().wd_reorder(ctx, arr, len(idx), n_rows), ctx)


def wd_topk(ctx, logits: int, B: int, W: int, top_val: int, top_id: int, lse: int):
    _check(lib().wd_topk(ctx, ctypes.c_void_p(logits), B, W, ctypes.c_void_p(top_val), ctypes.c_void_p(top_id),
                         ctypes.c_void_p(lse)), ctx)


def wd_beam_step(ctx, logits: int, W: int, first: bool, scores: int, beam_idx: int, tokens: int, n_rows: int):
    _check(lib().wd_beam_step(ctx, ctypes.c_void_p(logits), W, 1 if first else 0, ctypes.c_void_p(scores),
                              ctypes.c_void_p(beam_idx), ctypes.c_void_p(tokens), n_rows), ctx)


def wd_encoder_workspace_bytes(ctx, n_mels: int, frames: int, n_layers: int, d_ff: int, max_sets: int) -> int:
    return lib().wd_encoder_workspace_bytes(ctx, n_mels, frames, n_layers, d_ff, max_sets)


def wd_load_encoder(ctx, n_mels: int, frames: int, n_layers: int, d_ff: int, max_sets: int,
                    tensors: Sequence[WdTensor], workspace: int, ws_bytes: int):
    arr = (WdTensor * max(1, len(tensors)))(*tensors)
    _check(lib().wd_load_encoder(ctx, n_mels, frames, n_layers, d_ff, max_sets, arr if tensors else None,
                                 len(tensors), ctypes.c_void_p(workspace), ws_bytes), ctx)


def wd_encode(ctx, mel: int, n_sets: int, enc: int):
    _check(lib().wd_encode(ctx, ctypes.c_void_p(mel), n_sets, ctypes.c_void_p(enc)), ctx)


def wd_listen(ctx, mel: int):
    _check(lib().wd_listen(ctx, ctypes.c_void_p(mel)), ctx)


def wd_prefill(ctx, tokens: int, B: int, T: int, embeds: int, A: int, offset: int, logits: int,
               argmax: int):
    _check(lib().wd_prefill(ctx, ctypes.c_void_p(tokens), B, T,
                            ctypes.c_void_p(embeds) if embeds else None, A, offset,
                            ctypes.c_void_p(logits) if logits else None, ctypes.c_void_p(argmax)), ctx)


def wd_check(ctx) -> int:
    """Returns the status (0, or WD_ERR_RANGE == 3 when the device flag was set)."""
    return lib().wd_check(ctx)


def wd_last_error(ctx=None) -> str:
    r = lib().wd_last_error(ctx)
    return r.decode() if r else ""


def wd_free(ctx):
    lib().wd_free(ctx)


def wd_profile(ctx, kernel: int, layer: int = -1, repeats: int = 1):
    _check(lib().wd_profile(ctx, kernel, layer, repeats), ctx)


def wd_profile_read(ctx):
    t = ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib().wd_profile_read(ctx, ctypes.byref(t), ctypes.byref(n)), ctx)
    return t.value, n.value


def wd_probe(kind: int, a: int = 0, b: int = 0, nbytes: int = 0, iters: int = 1, sink: int = 0) -> float:
    """Microseconds per launch of a machine-floor probe (kind 0: empty dependent launches in a
    graph; kind 1: one read of nbytes from each of the device buffers a and b)."""
    us = ctypes.c_double()
    _check(lib().wd_probe(kind, a or None, b or None, nbytes, iters, sink or None, ctypes.byref(us)), None)
    return us.value


def wd_debug_cache(ctx, which: int, layer: int) -> int:
    p = ctypes.c_void_p()
    _check(lib().wd_debug_cache(ctx, which, layer, ctypes.byref(p)), ctx)
    return p.value


def wd_topk_noalloc(logits: int, B: int, V: int, ld: int, W: int, top_val: int, top_id: int, lse: int,
                    stream: int = 0):
    _check(lib().wd_topk_noalloc(ctypes.c_void_p(logits), B, V, ld, W, ctypes.c_void_p(top_val),
                                 ctypes.c_void_p(top_id), ctypes.c_void_p(lse), ctypes.c_void_p(stream)))


def wd_set_option(ctx, option: int, value: int):
    _check(lib().wd_set_option(ctx, option, value), ctx)


def wd_get_option(ctx, option: int) -> int:
    v = ctypes.c_int32()
    _check(lib().wd_get_option(ctx, option, ctypes.byref(v)), ctx)
    return v.value


# ---- convenience: config and a torch-backed holder -------------------------------------------

def config_from(w, max_batch: Optional[int] = None) -> WdConfig:
    """WdConfig from any object with the workload attribute names (d, heads, ...)."""
    c = WdConfig()
    c.arch = ARCHS[w.arch]
    c.d_model, c.n_heads, c.n_kv_heads, c.head_dim = w.d, w.heads, w.kv_heads, w.head_dim
    c.n_layers, c.d_ff, c.vocab, c.context = w.layers, w.d_ff, w.vocab, w.context
    c.max_frames = w.frames if w.arch == "whisper" else 0
    c.max_batch = w.batch if max_batch is None else max_batch
    c.n_enc = w.n_enc if w.arch == "whisper" else 0
    c.w_dtype, c.cache_dtype = DTYPES[w.w_dtype], DTYPES[w.cache_dtype]
    c.norm_eps = w.eps
    c.rope_base = w.rope_base
    return c


def _torch_dtype(name: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[name]


class Decoder:
    """Owns one context: the workspace (a torch uint8 tensor), the loaded weights
    and the caches.  ``weights`` maps canonical names to arrays/tensors holding
    values representable in the workload's w_dtype."""

    def __init__(self, w, weights: Dict[str, object], device: str = "cuda", stream=None):
        import numpy as np
        import torch
        self.w = w
        self.cfg = config_from(w)
        self.device = torch.device(device)
        # a stream of our own (default priority): the library captures each step into a
        # HIP graph, which the legacy null stream does not allow
        self.stream = stream if stream is not None else torch.cuda.Stream(self.device)
        nbytes = wd_workspace_bytes(self.cfg)
        if nbytes == 0:
            raise WdError(1, "invalid configuration")
        self.workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        base = self.workspace.data_ptr()
        self.ws_ptr = (base + 255) & ~255
        wdt = _torch_dtype(w.w_dtype)
        up, descs = [], []
        with torch.cuda.stream(self.stream):
            for name, arr in weights.items():
                t = arr if isinstance(arr, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(arr))
                t = t.to(device=self.device, dtype=wdt).contiguous()
                up.append(t)
                descs.append(WdTensor(name.encode(), t.data_ptr(), t.numel(), DTYPES[w.w_dtype]))
        self.ctx = wd_load(self.cfg, descs, self.ws_ptr, nbytes, self.stream.cuda_stream)
        self.stream.synchronize()
        del up

    def load_encoder(self, weights: Dict[str, object], n_mels: int, frames: int, n_layers: int, d_ff: int,
                     max_sets: int):
        """Loads the audio encoder (canonical ``enc.*`` names) into a second workspace."""
        import numpy as np
        import torch
        nbytes = wd_encoder_workspace_bytes(self.ctx, n_mels, frames, n_layers, d_ff, max_sets)
        if nbytes == 0:
            raise WdError(1, "invalid encoder configuration")
        self.enc_workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        ptr = (self.enc_workspace.data_ptr() + 255) & ~255
        wdt = _torch_dtype(self.w.w_dtype)
        up, descs = [], []
        with torch.cuda.stream(self.stream):
            for name, arr in weights.items():
                t = arr if isinstance(arr, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(arr))
                t = t.to(device=self.device, dtype=wdt).contiguous()
                up.append(t)
                descs.append(WdTensor(name.encode(), t.data_ptr(), t.numel(), DTYPES[self.w.w_dtype]))
        wd_load_encoder(self.ctx, n_mels, frames, n_layers, d_ff, max_sets, descs, ptr, nbytes)
        self.stream.synchronize()
        del up
        self.enc_frames = frames

    def encode(self, mel, out=None):
        """mel: device tensor [n_sets, frames, n_mels] in w_dtype.  Returns [n_sets, P, d]."""
        import torch
        n, frames = mel.shape[0], mel.shape[1]
        assert frames == self.enc_frames and mel.is_contiguous()
        P = (frames - 1) // 2 + 1
        if out is None:
            out = torch.empty(n, P, self.w.d, dtype=mel.dtype, device=self.device)
        cur = self._enter()
        wd_encode(self.ctx, mel.data_ptr(), n, out.data_ptr())
        self._leave(cur)
        return out

    def listen(self, mel):
        """mel: device tensor [n_enc, frames, n_mels]; encodes and fills the cross caches."""
        assert mel.shape[0] == self.w.n_enc and mel.is_contiguous()
        assert mel.shape[1] == getattr(self, "enc_frames", mel.shape[1])
        cur = self._enter()
        wd_listen(self.ctx, mel.data_ptr())
        self._leave(cur)

    def close(self):
        """Frees the context (wd_free waits for its stream first); the workspace is
        released only after that, when this object goes away."""
        if getattr(self, "ctx", None):
            self.stream.synchronize()
            wd_free(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ordering against torch's current stream: a call waits for the work queued there
    # before it, and work queued there after it waits for the call (no-ops when the
    # caller already runs on self.stream)
    def _enter(self):
        import torch
        cur = torch.cuda.current_stream(self.device)
        if cur != self.stream:
            self.stream.wait_stream(cur)
        return cur

    def _leave(self, cur):
        if cur != self.stream:
            cur.wait_stream(self.stream)

    def cross_kv(self, enc, frames: Optional[int] = None):
        cur = self._enter()
        wd_cross_kv(self.ctx, enc.data_ptr(), enc.shape[1] if frames is None else frames)
        self._leave(cur)

    def cross_kv_ragged(self, enc, frames: Sequence[int]):
        """enc: device tensor [n_enc, max(frames), d]; set e has frames[e] valid rows."""
        assert enc.shape[0] == self.w.n_enc and enc.shape[1] == max(frames) and len(frames) == self.w.n_enc
        cur = self._enter()
        wd_cross_kv_ragged(self.ctx, enc.data_ptr(), frames)
        self._leave(cur)

    def step(self, tokens, positions, logits=None, argmax=None):
        """tokens, positions: int32 device tensors [B].  Returns (logits, argmax)."""
        import torch
        B = tokens.shape[0]
        if argmax is None:
            argmax = torch.empty(B, dtype=torch.int32, device=self.device)
        cur = self._enter()
        wd_step(self.ctx, tokens.data_ptr(), positions.data_ptr(), B,
                logits.data_ptr() if logits is not None else 0, argmax.data_ptr())
        self._leave(cur)
        return logits, argmax

    def prefill(self, tokens, embeds=None, offset: int = 0, logits=None, argmax=None):
        import torch
        B, T = tokens.shape
        if argmax is None:
            argmax = torch.empty(B, dtype=torch.int32, device=self.device)
        A = 0 if embeds is None else embeds.shape[1]
        cur = self._enter()
        wd_prefill(self.ctx, tokens.data_ptr(), B, T, embeds.data_ptr() if embeds is not None else 0,
                   A, offset, logits.data_ptr() if logits is not None else 0, argmax.data_ptr())
        self._leave(cur)
        return logits, argmax

    def reorder(self, beam_idx, n_rows: int):
        cur = self._enter()
        wd_reorder(self.ctx, [int(i) for i in beam_idx], n_rows)
        self._leave(cur)

    def beam_step(self, logits, W: int, first: bool, scores, beam_idx, tokens, n_rows: int):
        """One beam step on the device (wd_beam_step): logits fp32 [>= W, vocab], scores float64
        [W] (updated in place), beam_idx and tokens int32 [W] (written), then the self-cache
        rearrangement of rows 0..n_rows-1."""
        import torch
        assert logits.dtype == torch.float32 and logits.is_contiguous() and logits.shape[1] == self.w.vocab
        assert scores.dtype == torch.float64 and beam_idx.dtype == torch.int32 and tokens.dtype == torch.int32
        cur = self._enter()
        wd_beam_step(self.ctx, logits.data_ptr(), W, first, scores.data_ptr(), beam_idx.data_ptr(),
                     tokens.data_ptr(), n_rows)
        self._leave(cur)

    def topk(self, logits, W: int):
        """logits: fp32 device tensor [B, vocab].  Returns device tensors (top values [B, W],
        top ids [B, W] int32, lse [B])."""
        import torch
        B = logits.shape[0]
        assert logits.dtype == torch.float32 and logits.is_contiguous() and logits.shape[1] == self.w.vocab
        vals = torch.empty(B, W, dtype=torch.float32, device=self.device)
        ids = torch.empty(B, W, dtype=torch.int32, device=self.device)
        lse = torch.empty(B, dtype=torch.float32, device=self.device)
        cur = self._enter()
        wd_topk(self.ctx, logits.data_ptr(), B, W, vals.data_ptr(), ids.data_ptr(), lse.data_ptr())
        self._leave(cur)
        return vals, ids, lse

    def check(self) -> int:
        return wd_check(self.ctx)

    def set_graphs(self, on: bool):
        """Step graphs on (capture once, replay) or off (eager launches)."""
        wd_set_option(self.ctx, WD_OPT_GRAPHS, 1 if on else 0)

    def cache(self, which: int, layer: int):
        """A torch view of one cache block (test hook): which 0/1 self K/V
        [max_batch, Hkv, context, hd], 2/3 cross K/V [n_enc, H, max_frames, hd]."""
        import torch
        w = self.w
        ptr = wd_debug_cache(self.ctx, which, layer)
        shape = ((w.batch, w.kv_heads, w.context, w.head_dim) if which < 2
                 else (w.n_enc, w.heads, w.frames, w.head_dim))
        dt = _torch_dtype(w.cache_dtype)
        n = 1
        for s_ in shape:
            n *= s_
        base = self.workspace.view(torch.uint8)
        off = ptr - base.data_ptr()
        esz = torch.tensor([], dtype=dt).element_size()
        return base[off:off + n * esz].view(dt).view(*shape)

    def last_error(self) -> str:
        return wd_last_error(self.ctx)

#!/usr/bin/env python3
"""Decoder-step throughput on one MI355X.

One bench step is one whole audio window of the workload: the cross K/V
projection of every layer (once per window), then every decode position of the
window, each a wd_step over the B rows, greedy on the device (the argmax of a
step is the next step's token buffer; the 4-token prompt is fed first), with no
host synchronisation inside the window.  Inputs (weights, encoder states,
prompts) are resident in HBM before the timed region.

Printed: one JSON line.  value = B * positions * K / (time of K windows),
tokens/s including the cross K/V projection; decode-only tokens/s, the
algorithmic HBM bytes per window (weights once per step + self-cache rows
0..pos + cross cache once per encoder set) and their rate against the 8 TB/s
peak are extra fields.  `roofline` reports the dominant kernel (the
cross-attention) from HIP events recorded around its launches in one layer
over a window run right after the timed ones; `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads as WL  # noqa: E402

HBM_PEAK = 8.0e12
DEFAULT = "whisper_large_bf16_b64"
DT_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
# the cross-attention kernel's source: its file and the headers it includes
ATTN_SRC = [os.path.join(ROOT, "kv_cached_autoregressive_amd", "csrc", f)
            for f in ("k_attn.hip", "wd_common.h", "wd_kernels.h")]


def attn_source_sha() -> str:
    h = hashlib.sha256()
    for f in ATTN_SRC:
        h.update(open(f, "rb").read())
    return h.hexdigest()
TRAFFIC_WORKLOAD = "whisper_large_bf16_b64"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", f"k_attn_cross_{TRAFFIC_WORKLOAD}_traffic.json")


def whisper_bytes_per_step(w, pos: int) -> int:
    """Algorithmic HBM bytes of one decode step at position `pos`: every weight
    once (projections, norms, biases, the tied head), the B embedding and
    position rows, self-cache rows 0..pos of every row and layer, the cross
    cache once per encoder set."""
    d, ff, L = w.d, w.d_ff, w.layers
    wb, cb = DT_BYTES[w.w_dtype], DT_BYTES[w.cache_dtype]
    per_layer = (6 * d * d + 2 * d * ff + 12 * d + ff) * wb
    glob = w.vocab * d * wb + 2 * d * wb + 2 * w.batch * d * wb
    self_c = w.batch * L * (pos + 1) * 2 * d * cb
    cross = w.n_enc * L * w.frames * 2 * d * cb
    return L * per_layer + glob + self_c + cross


def cross_attn_bytes_per_launch(w) -> int:
    """Algorithmic bytes of one cross-attention launch (one layer): the K and V
    blocks of every encoder set, read once."""
    return w.n_enc * w.heads * w.frames * w.head_dim * 2 * DT_BYTES[w.cache_dtype]


def traffic_per_launch(workload: str):
    """HBM bytes per cross-attention launch from the committed rocprofv3 counter
    summary, or None when absent, taken on a different kernel source, or taken on
    another workload (the counters cover the large-v3 window only)."""
    if workload != TRAFFIC_WORKLOAD:
        return None
    try:
        t = json.load(open(TRAFFIC_FILE))
        if t.get("kernel_source_sha256") != attn_source_sha():
            return None
        return int(t["hbm_bytes_per_launch"])
    except Exception:
        return None


COPY_PROBE_BYTES = 256 << 20
# the cross-attention instantiation: k_attn<cache type, head dim, queries, CROSS = true, waves>
CROSS_ATTN_NAME = re.compile(r"k_attn<[^<>]*?,\s*true\s*,")


def summarize_traffic(fetch_csv: str, write_csv: str, commands: list) -> dict:
    """HBM bytes per cross-attention launch from two rocprofv3 --pmc runs of
    `bench.py --traffic-probe` (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch).
    Each counter is scaled by what it reads for the probe's device copy of
    COPY_PROBE_BYTES (the largest copy dispatch of the run), so the result is in
    the copy's bytes."""
    import csv

    def per_kernel(path, counter):
        attn, copies = [], []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name, v = r["Kernel_Name"], float(r["Counter_Value"])
            if CROSS_ATTN_NAME.search(name):
                attn.append(v)
            elif "copyBuffer" in name:
                copies.append(v)
        if not attn or not copies:
            raise SystemExit(f"{path}: no cross-attention or copy dispatches with {counter}")
        return sum(attn) / len(attn), max(copies), len(attn)

    fa, fc, n = per_kernel(fetch_csv, "FETCH_SIZE")
    wa, wc, _ = per_kernel(write_csv, "WRITE_SIZE")
    ref_kib = COPY_PROBE_BYTES / 1024
    f_fac, w_fac = fc / ref_kib, wc / ref_kib
    fetch_b, write_b = fa * 1024 / f_fac, wa * 1024 / w_fac
    return {"kernel": "k_attn (cross-attention)", "dispatches": n,
            "fetch_kib_per_dispatch": fa, "write_kib_per_dispatch": wa,
            "copy_probe_bytes": COPY_PROBE_BYTES, "copy_fetch_kib": fc, "copy_write_kib": wc,
            "fetch_scale": f_fac, "write_scale": w_fac,
            "hbm_fetch_bytes_per_launch": int(fetch_b), "hbm_write_bytes_per_launch": int(write_b),
            "hbm_bytes_per_launch": int(fetch_b + write_b),
            "kernel_source_sha256": attn_source_sha(),
            "commands": commands}


def qwen_bytes_per_step(w, pos: int) -> int:
    """Algorithmic HBM bytes of one Qwen3 decode step at position `pos`: every weight once
    (q, k, v, o, gate, up, down, the norms, the tied head), the B embedding rows and the
    K/V rows 0..pos of every row and layer."""
    d, ff, L, hd = w.d, w.d_ff, w.layers, w.head_dim
    wb, cb = DT_BYTES[w.w_dtype], DT_BYTES[w.cache_dtype]
    qd, kvd = w.heads * hd, w.kv_heads * hd
    per_layer = (d * qd + 2 * d * kvd + qd * d + 3 * d * ff) * wb + (2 * d + 2 * hd) * 4
    glob = w.vocab * d * wb + d * 4 + w.batch * d * wb
    kv = w.batch * L * (pos + 1) * 2 * kvd * cb
    return L * per_layer + glob + kv


def qwen_cpu_baseline(w, budget_s: float):
    """The Qwen3 oracle on the host cores: one stream's decode steps from position 0 for
    about `budget_s` seconds (no prefill; bounded sample)."""
    from threadpoolctl import threadpool_info

    from oracle import qwen3 as OQ
    W = WL.make_weights(w)
    O = OQ.QwenOracle(OQ.dims_of(w), W, round_cache=True)
    del W
    O.reset(1)
    ids = WL.random_ids(w, 64)[:1]
    n, t = 0, 0.0
    while n < ids.shape[1] and (n < 2 or t < budget_s):
        t0 = time.perf_counter()
        O.step(ids[:, n], [n])
        t += time.perf_counter() - t0
        n += 1
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": n / t, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"1 of {w.batch} streams, decode steps at positions 0..{n - 1} (float64 numpy, no prefill)"}


def run_qwen(args, w):
    """Qwen3-ASR: prefill of 900 positions (audio rows spliced in), then the greedy decode
    steps to the context end, argmax on the device.  value = decode tokens/s; the prefill
    (batched: chunks of positions through dense MFMA GEMMs and a causal prefill attention)
    is timed separately."""
    import torch

    import kv_cached_autoregressive_amd as K
    dev = torch.device("cuda:0")
    W = WL.make_weights(w)
    ids_np, audio_np = WL.make_qwen_prefill(w)
    dec = K.Decoder(w, W)
    del W
    wdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.w_dtype]
    B, T, S = w.batch, w.prefill_len, w.steps
    ids = torch.from_numpy(np.ascontiguousarray(ids_np)).to(dev, torch.int32)
    audio = torch.from_numpy(np.ascontiguousarray(audio_np)).to(dev, wdt)
    pos_all = (T + torch.arange(S, dtype=torch.int32, device=dev))[:, None].repeat(1, B).contiguous()
    amax = torch.zeros(B, dtype=torch.int32, device=dev)
    stream, ctx = dec.stream, dec.ctx

    def prefill():
        K.wd_prefill(ctx, ids.data_ptr(), B, T, audio.data_ptr(), audio.shape[1], w.audio_offset, 0,
                     amax.data_ptr())

    def steps(n):
        for p in range(n):
            K.wd_step(ctx, amax.data_ptr(), pos_all[p].data_ptr(), B, 0, amax.data_ptr())

    torch.cuda.synchronize()
    torch.cuda.set_stream(stream)
    for _ in range(args.warmup):
        prefill()
        steps(S)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * args.steps)]
    pre_ms, dec_ms = 0.0, 0.0
    wall0 = time.perf_counter()
    for i in range(args.steps):
        ev[3 * i].record(stream)
        prefill()
        ev[3 * i + 1].record(stream)
        steps(S)
        ev[3 * i + 2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    for i in range(args.steps):
        pre_ms += ev[3 * i].elapsed_time(ev[3 * i + 1]) / args.steps
        dec_ms += ev[3 * i + 1].elapsed_time(ev[3 * i + 2]) / args.steps
    if dec.check() != 0:
        raise RuntimeError(dec.last_error())
    # kernel timing: the gate|up projection of one layer (the largest weight stream of a layer)
    prefill()
    K.wd_profile(ctx, K.K_FC1, args.profile_layer, args.profile_repeats)
    steps(min(S, args.profile_positions))
    k_ms, k_n = K.wd_profile_read(ctx)
    K.wd_profile(ctx, -1, -1, 1)
    gu_bytes = 2 * w.d_ff * w.d * DT_BYTES[w.w_dtype]
    k_avg = k_ms / 1e3 / max(k_n, 1)
    bytes_dec = sum(qwen_bytes_per_step(w, T + p) for p in range(S))
    out = {
        "metric": "decoder tokens/sec at batch B; achieved HBM GB/s as % of MI355X peak",
        "value": B * S / (dec_ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": dec_ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.w_dtype,
        "data": "synthetic (seeded random-init weights N(0,0.02), N(0,1) audio rows, uniform ids)",
        "config": {"workload": w.name, "batch": B, "prefill": T, "positions": S, "layers": w.layers,
                   "d": w.d, "q_heads": w.heads, "kv_heads": w.kv_heads, "head_dim": w.head_dim,
                   "d_ff": w.d_ff, "vocab": w.vocab, "w_dtype": w.w_dtype, "cache_dtype": w.cache_dtype,
                   "step": "124 greedy decode steps after the prefill (prefill timed separately)"},
        "decode_tokens_per_s": B * S / (dec_ms / 1e3),
        "prefill_ms": pre_ms,
        "hbm_bytes_decode": bytes_dec,
        "hbm_gbps_decode": bytes_dec / (dec_ms / 1e3) / 1e9,
        "hbm_frac_decode": bytes_dec / (dec_ms / 1e3) / HBM_PEAK,
        "wall_s": wall,
        "roofline": {"kernel": "gate|up projection (MFMA skinny GEMM, one layer per launch)", "bound": "hbm",
                     "achieved": gu_bytes / k_avg / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": gu_bytes / k_avg / HBM_PEAK, "traffic": None, "bytes_per_launch": gu_bytes,
                     "avg_launch_us": k_avg * 1e6, "launches_timed": k_n},
        "cpu_baseline": None,
    }
    del dec
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = qwen_cpu_baseline(w, args.cpu_budget)
    print(json.dumps(out), flush=True)


def run_encoder(args, w):
    """The audio encoder of one window: every encoder set's 3000 synthetic mel frames through
    the stem and the encoder layers to its 1500 states (wd_encode), with seeded random-init
    weights generated on the device.  value = encoder states per second."""
    import torch

    import kv_cached_autoregressive_amd as K
    dev = torch.device("cuda:0")
    layers = args.encoder_layers or w.layers
    mels, frames, d, ff, n = args.mels, 2 * w.frames, w.d, w.d_ff, w.n_enc
    P = (frames - 1) // 2 + 1
    wdt = {"f16": torch.float16, "bf16": torch.bfloat16}[w.w_dtype]
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed * 1000 + 17)
    rnd = lambda *shape, std=0.02, mean=0.0: (torch.randn(*shape, generator=g, device=dev) * std + mean).to(wdt)
    W = {"enc.conv1.w": rnd(d, mels, 3), "enc.conv1.b": rnd(d), "enc.conv2.w": rnd(d, d, 3), "enc.conv2.b": rnd(d),
         "enc.pos": rnd(P, d, std=1.0), "enc.ln_post.g": rnd(d, mean=1.0), "enc.ln_post.b": rnd(d)}
    for i in range(layers):
        p = f"enc.{i}."
        for ln in ("ln1", "ln2"):
            W[p + ln + ".g"], W[p + ln + ".b"] = rnd(d, mean=1.0), rnd(d)
        for proj in ("q", "k", "v", "o"):
            W[p + f"attn.{proj}.w"] = rnd(d, d)
            if proj != "k":
                W[p + f"attn.{proj}.b"] = rnd(d)
        W[p + "fc1.w"], W[p + "fc1.b"], W[p + "fc2.w"], W[p + "fc2.b"] = rnd(ff, d), rnd(ff), rnd(d, ff), rnd(d)
    wr = WL.reduced(w, layers=1, vocab=1024)   # a decoder context to hold the encoder
    dec = K.Decoder(wr, WL.make_weights(wr))
    dec.load_encoder(W, mels, frames, layers, ff, max_sets=n)
    del W
    mel = torch.randn(n, frames, mels, generator=g, device=dev).to(wdt)
    out = torch.empty(n, P, d, dtype=wdt, device=dev)
    torch.cuda.synchronize()
    torch.cuda.set_stream(dec.stream)
    for _ in range(args.warmup):
        dec.encode(mel, out)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(dec.stream)
    for _ in range(args.steps):
        dec.encode(mel, out)
    t1.record(dec.stream)
    torch.cuda.synchronize()
    if dec.check() != 0:
        raise RuntimeError(dec.last_error())
    ms = t0.elapsed_time(t1) / args.steps
    # algorithmic flops: the two convolutions and, per layer, q|k|v, the attention, o, fc1, fc2
    per_set = 2 * frames * 3 * mels * d + 2 * P * 3 * d * d + \
        layers * (2 * P * d * 3 * d + 4 * P * P * d + 2 * P * d * d + 4 * P * d * ff)
    print(json.dumps({
        "metric": "encoder states/sec (audio encoder, one window of every encoder set)",
        "value": n * P / (ms / 1e3), "unit": "states/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "dtype": w.w_dtype,
        "data": "synthetic (seeded random-init weights N(0,0.02), mel N(0,1))",
        "config": {"workload": w.name + " encoder", "sets": n, "mel_frames": frames, "states": P, "mels": mels,
                   "layers": layers, "d": d, "heads": w.heads, "d_ff": ff},
        "tflops": n * per_set / (ms / 1e3) / 1e12}), flush=True)


def cpu_baseline(w, budget_s: float):
    """The oracle as it is, on the host cores: one stream of the workload, its
    cross K/V and as many decode steps as fit the time budget."""
    from threadpoolctl import threadpool_info

    from oracle import whisper as OW
    W = WL.make_weights(w)
    enc = WL.make_encoder_states(w, streams=[0])
    O = OW.WhisperOracle(OW.dims_of(w), W)
    del W
    t0 = time.perf_counter()
    O.cross_kv(enc)
    t_cross = time.perf_counter() - t0
    O.reset(1)
    prompt = WL.make_prompt(w)[:1]
    tok = prompt[:, 0]
    n, t_steps = 0, 0.0
    while n < w.steps and (n < 2 or t_steps < budget_s):
        t0 = time.perf_counter()
        lg = O.step(tok, [n])
        t_steps += time.perf_counter() - t0
        tok = prompt[:, n + 1] if n + 1 < prompt.shape[1] else np.argmax(lg, -1)
        n += 1
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": n / t_steps, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"1 of {w.batch} streams, positions 0..{n - 1} of {w.steps} (float64 numpy); "
                      f"the stream's cross K/V took {t_cross:.2f} s on top, not counted"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3, help="timed windows")
    ap.add_argument("--warmup", type=int, default=1, help="untimed windows")
    ap.add_argument("--config", default=DEFAULT)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle decode steps")
    ap.add_argument("--profile-layer", type=int, default=0, help="layer whose cross-attention launches are timed")
    ap.add_argument("--profile-positions", type=int, default=16, help="positions of the kernel-timing run")
    ap.add_argument("--profile-repeats", type=int, default=8, help="back-to-back launches per timed event pair")
    ap.add_argument("--positions", type=int, default=0,
                    help="profiling aid: decode only the first N positions of each window")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="after the run, one device copy of a known size (counter calibration)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the cross-attention traffic summary under profiles/ from two --pmc runs and exit")
    ap.add_argument("--commands", nargs="*", default=[], help="the profiler commands, recorded in the summary")
    ap.add_argument("--encoder", action="store_true",
                    help="time the audio encoder (wd_encode) of the workload's encoder sets instead of the decoder")
    ap.add_argument("--encoder-layers", type=int, default=0, help="encoder layers (default: the decoder's)")
    ap.add_argument("--mels", type=int, default=80, help="mel channels of the encoder's input")
    args = ap.parse_args()
    if args.summarize_traffic:
        out = summarize_traffic(*args.summarize_traffic, args.commands)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(out, f, indent=1)
        print(json.dumps(out))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU: the decoder step is measured on a single MI355X and no "
              "multi-GPU path is built (rows would shard by stream across GPUs).", file=sys.stderr)
        sys.exit(2)

    import torch

    import kv_cached_autoregressive_amd as K

    w = WL.by_name(args.config)
    if args.positions:
        w = WL.reduced(w, steps=min(args.positions, w.steps))
    K.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if w.arch == "qwen3":
        run_qwen(args, w)
        return
    if args.encoder:
        run_encoder(args, w)
        return
    if w.mode != "greedy":
        print(f"bench.py times greedy windows; {w.name} is a beam-search workload", file=sys.stderr)
        sys.exit(2)

    W = WL.make_weights(w)
    enc_np = WL.make_encoder_states(w)
    dec = K.Decoder(w, W)
    del W
    wdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.w_dtype]
    enc = torch.from_numpy(enc_np).to(dev, wdt)
    del enc_np
    B, S = w.batch, w.steps
    prompt = torch.from_numpy(WL.make_prompt(w).T.copy()).to(dev)          # [4, B]
    pos_all = torch.arange(S, dtype=torch.int32, device=dev)[:, None].repeat(1, B).contiguous()
    amax = torch.zeros(B, dtype=torch.int32, device=dev)
    stream = dec.stream
    ctx = dec.ctx

    def steps(n):
        for p in range(n):
            tok = prompt[p] if p < prompt.shape[0] else amax
            K.wd_step(ctx, tok.data_ptr(), pos_all[p].data_ptr(), B, 0, amax.data_ptr())

    def window(ev=None):
        K.wd_cross_kv(ctx, enc.data_ptr(), w.frames)
        if ev is not None:
            ev.record(stream)
        steps(S)

    torch.cuda.synchronize()
    torch.cuda.set_stream(stream)          # everything below is queued on the decoder's stream
    for _ in range(args.warmup):
        window()
    torch.cuda.synchronize()
    if dec.check() != 0:
        raise RuntimeError(dec.last_error())

    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    mids = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        starts[i].record(stream)
        window(mids[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    xkv_ms = sum(starts[i].elapsed_time(mids[i]) for i in range(args.steps)) / args.steps
    if dec.check() != 0:
        raise RuntimeError(dec.last_error())
    # kernel timing: HIP events on the decoder's stream around the cross-attention of one
    # layer, issued `repeats` times back to back per step (the launch is idempotent), over
    # the first positions of a window run right after the timed ones (steps are launched
    # one by one there, since a captured step replays without per-launch host hooks); the
    # cross-attention reads all frames at every position, so any positions will do
    K.wd_profile(ctx, K.K_CROSS_ATTN, args.profile_layer, args.profile_repeats)
    steps(min(S, args.profile_positions))
    attn_ms, attn_n = K.wd_profile_read(ctx)
    K.wd_profile(ctx, -1, -1, 1)
    if args.traffic_probe:
        src = torch.ones(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.zeros_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ms_window = total_ms / args.steps
    dec_ms = ms_window - xkv_ms
    tokens = B * S
    bytes_window = sum(whisper_bytes_per_step(w, p) for p in range(S))
    attn_bytes = cross_attn_bytes_per_launch(w)
    attn_avg_s = attn_ms / 1e3 / max(attn_n, 1)
    achieved = attn_bytes / attn_avg_s
    xkv_flops = 2.0 * w.n_enc * w.frames * w.d * 2 * w.d * w.layers
    traffic = traffic_per_launch(w.name)
    out = {
        "metric": "decoder tokens/sec at batch B; achieved HBM GB/s as % of MI355X peak",
        "value": tokens / (ms_window / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_window,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.w_dtype,
        "data": "synthetic (seeded random-init weights N(0,0.02), encoder states N(0,1))",
        "config": {"workload": w.name, "batch": B, "positions": S, "frames": w.frames,
                   "layers": w.layers, "d": w.d, "heads": w.heads, "d_ff": w.d_ff,
                   "vocab": w.vocab, "w_dtype": w.w_dtype, "cache_dtype": w.cache_dtype,
                   "step": "one window: cross K/V projection + all positions, greedy on device"},
        "decode_tokens_per_s": tokens / (dec_ms / 1e3),
        "decode_ms_per_window": dec_ms,
        "hbm_bytes_per_window": bytes_window,
        "hbm_gbps_decode": bytes_window / (dec_ms / 1e3) / 1e9,
        "hbm_frac_decode": bytes_window / (dec_ms / 1e3) / HBM_PEAK,
        "cross_kv_ms": xkv_ms,
        "cross_kv_tflops": xkv_flops / (xkv_ms / 1e3) / 1e12,
        "wall_s": wall,
        "roofline": {"kernel": "k_attn (cross-attention, one layer per launch)", "bound": "hbm",
                     "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK,
                     "traffic": traffic,
                     "bytes_per_launch": attn_bytes, "avg_launch_us": attn_avg_s * 1e6,
                     "launches_timed": attn_n},
        "cpu_baseline": None,
    }
    del dec, enc
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

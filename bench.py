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


def probe_scale(copy_kib: list, path: str, counter: str) -> float:
    """Counter reading of the probe's COPY_PROBE_BYTES device copy (its largest copy dispatch)
    over the copy's true KiB.  The counters read 0.5 (FETCH_SIZE) and 1.0 (WRITE_SIZE) of the
    copy on this GPU; a run without the probe has only small copies and would give a scale
    thousands of times too small, so it is refused."""
    ref_kib = COPY_PROBE_BYTES / 1024
    scale = max(copy_kib, default=0.0) / ref_kib
    if scale < 0.25:
        raise SystemExit(f"{path}: no {COPY_PROBE_BYTES >> 20} MiB copy probe among the {counter} dispatches "
                         "(run bench.py with --traffic-probe)")
    return scale


def traffic_probe_copy(dev) -> None:
    """The device copy of COPY_PROBE_BYTES that calibrates FETCH_SIZE / WRITE_SIZE."""
    import torch
    src = torch.ones(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.zeros_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


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
    f_fac, w_fac = probe_scale([fc], fetch_csv, "FETCH_SIZE"), probe_scale([wc], write_csv, "WRITE_SIZE")
    fetch_b, write_b = fa * 1024 / f_fac, wa * 1024 / w_fac
    return {"kernel": "k_attn (cross-attention)", "dispatches": n,
            "fetch_kib_per_dispatch": fa, "write_kib_per_dispatch": wa,
            "copy_probe_bytes": COPY_PROBE_BYTES, "copy_fetch_kib": fc, "copy_write_kib": wc,
            "fetch_scale": f_fac, "write_scale": w_fac,
            "hbm_fetch_bytes_per_launch": int(fetch_b), "hbm_write_bytes_per_launch": int(write_b),
            "hbm_bytes_per_launch": int(fetch_b + write_b),
            "kernel_source_sha256": attn_source_sha(),
            "commands": commands}


# ---- per-kernel HBM traffic against algorithmic bytes (two rocprofv3 --pmc runs) ----------------
EPI = {"store": 0, "resid": 1, "qkv": 3, "gelu_split": 5, "swiglu_split": 6}


def sk_shape(N: int, K: int, B: int, epi: int):
    """The split-K skinny GEMM's launch shape for a projection (the library's policy, restated
    for labelling counter rows): (NBW, NBB, NSC, G, workgroups) or None when the projection
    takes another kernel."""
    NB, KST = (N + 15) // 16, K // 32
    NBB = 1 if B <= 16 else 2 if B <= 32 else 4
    NBW = 2 if (NB >= 256 or KST >= 128 or epi == EPI["swiglu_split"]) else 1
    narrow = NBB == 1 and (epi != EPI["swiglu_split"] or KST > 16) and KST * ((NB + 3) // 4) >= 8 * 256
    if narrow:
        NBW = 1
    ncg = (NB + 4 * NBW - 1) // (4 * NBW)
    S = max(2, min((KST * ncg + 255) // 256, 16 if narrow else 8))
    G = (KST + S - 1) // S
    if narrow:
        if G > 32:
            return None
        nsc = max(4, (KST + G - 1) // G)
        return NBW, NBB, (16 if nsc > 8 else nsc), G, ncg * G
    if ncg * G > 256 and NBW == 1:
        NBW = 2
        ncg = (NB + 7) // 8
        S = max(2, min((KST * ncg + 255) // 256, 8))
        G = (KST + S - 1) // S
    if N <= 2048 and KST >= 16:
        G = 8 * ((KST + 63) // 64)
    if G > 32:
        return None
    nsc = max(4, (KST + G - 1) // G)
    return NBW, NBB, (16 if nsc > 8 else nsc), G, ncg * G


def projections(w):
    """(role, N, K, epilogue) of one layer's projections, in launch order."""
    d, ff = w.d, w.d_ff
    if w.arch == "whisper":
        return [("q|k|v", 3 * d, d, EPI["qkv"]), ("self out", d, d, EPI["resid"]), ("cross q", d, d, EPI["store"]),
                ("cross out", d, d, EPI["resid"]), ("fc1", ff, d, EPI["gelu_split"]), ("fc2", d, ff, EPI["resid"])]
    qd, kvd = w.heads * w.head_dim, w.kv_heads * w.head_dim
    return [("q|k|v", qd + 2 * kvd, d, EPI["store"]), ("out", d, qd, EPI["resid"]),
            ("gate|up", 2 * ff, d, EPI["swiglu_split"]), ("down", d, ff, EPI["resid"])]


def canon_kernel(name: str) -> str:
    """'base<int and bool template arguments>' of a kernel name, demangled by the profiler or
    not (instantiations over _Float16 come out mangled): the type arguments are dropped."""
    m = re.match(r"_ZN2wd(\d+)(\w+)", name)
    if m:
        base = m.group(2)[:int(m.group(1))]
        rest = m.group(2)[int(m.group(1)):]
        args = [("true" if a == "b1" else "false") if a.startswith("b") else a[1:]
                for a in re.findall(r"L(i\d+|b[01])E", rest)]
        return f"{base}<{','.join(args)}>" if args else base
    m = re.search(r"(?:wd::)?(\w+)<([^()]*)>\(", name)
    if m:
        args = [a.strip() for a in m.group(2).split(",") if re.fullmatch(r"\s*(-?\d+|true|false)\s*", a)]
        return f"{m.group(1)}<{','.join(args)}>"
    m = re.search(r"(?:wd::)?(\w+)\(", name)
    return m.group(1) if m else name[:60]


def summarize_counters(fetch_csv: str, write_csv: str, w, positions: int, commands: list,
                       mfma_csv: str = None) -> str:
    """Markdown table of HBM bytes per dispatch (FETCH_SIZE + WRITE_SIZE, each scaled by what it
    reads for the run's device copy of COPY_PROBE_BYTES) per kernel and launch shape, against the
    kernel's algorithmic bytes (weights read once, cache rows read) and the activation and
    partial-slab bytes its design adds."""
    import csv
    import collections

    def load(path, counter):
        groups, copies = collections.defaultdict(list), []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            if "copyBuffer" in r["Kernel_Name"]:
                copies.append(v)
                continue
            wg = max(1, int(r.get("Workgroup_Size", 1) or 1))
            grid = int(r.get("Grid_Size", 0) or 0) // wg
            groups[(r["Kernel_Name"], grid)].append(v)
        return groups, probe_scale(copies, path, counter)

    fg, ff_ = load(fetch_csv, "FETCH_SIZE")
    wg_, wf = load(write_csv, "WRITE_SIZE")
    mf = {}
    if mfma_csv:
        for r in csv.DictReader(open(mfma_csv)):
            if r["Counter_Name"] != "MfmaUtil" or "copyBuffer" in r["Kernel_Name"]:
                continue
            wgs = max(1, int(r.get("Workgroup_Size", 1) or 1))
            mf.setdefault((r["Kernel_Name"], int(r.get("Grid_Size", 0) or 0) // wgs), []).append(float(r["Counter_Value"]))
    wb, cb = DT_BYTES[w.w_dtype], DT_BYTES[w.cache_dtype]
    B, d = w.batch, w.d
    Bp = 16 if B <= 16 else 32 if B <= 32 else 64
    # labels of the projection shapes
    label = {}
    for role, N, K, epi in projections(w):
        sh = sk_shape(N, K, B, epi)
        if sh is None:
            continue
        NBW, NBB, NSC, G, grid = sh
        key = (f"k_mgemv_sk<{NBW},{NBB},{NSC},1>", grid)
        alg = N * K * wb
        extra = G * B * N * 4 if G > 1 else 0   # fp32 partial slabs written (read by the consumer)
        prev = label.get(key)
        if prev is None:
            label[key] = (f"{role} (K groups {G})", alg, extra, G)
        else:   # two projections with one launch shape: their mean
            label[key] = (f"{prev[0]}, {role} (K groups {G})", (prev[1] + alg) // 2, (prev[2] + extra) // 2, G)
    # partial slabs the attention prologues read (q, and the appended k, v) when the q
    # projection is split
    qkv_G = [sk_shape(N, K, B, e)[3] for r, N, K, e in projections(w) if r == "q|k|v"][0]
    cq_G = [sk_shape(N, K, B, e)[3] for r, N, K, e in projections(w) if r == "cross q"] if w.arch == "whisper" else [1]
    mean_rows = (positions + 1) / 2 if w.arch == "whisper" else w.prefill_len + (positions + 1) / 2
    rows = []
    for key in sorted(set(fg) | set(wg_), key=lambda k: -sum(fg.get(k, [0]))):
        name, grid = key
        f = fg.get(key, [])
        wr = wg_.get(key, [])
        n = max(len(f), len(wr))
        fb = (sum(f) / max(len(f), 1)) * 1024 / ff_
        wb_ = (sum(wr) / max(len(wr), 1)) * 1024 / wf
        short = canon_kernel(name)
        role, alg, extra = "", None, None
        if (short, grid) in label:
            role, alg, extra, G = label[(short, grid)]
        if "k_attn<" in short and ",true," in short:
            role, alg = "cross-attention", cross_attn_bytes_per_launch(w)
            if cq_G[0] > 1:
                extra = cq_G[0] * B * d * 4
                role += " (+ cross-q partials read)"
        elif "k_attn<" in short:
            role = "self-attention"
            alg = int(B * w.kv_heads * mean_rows * w.head_dim * 2 * cb)
            if qkv_G > 1:
                nqkv = 3 * d if w.arch == "whisper" else (w.heads + 2 * w.kv_heads) * w.head_dim
                extra = qkv_G * B * nqkv * 4
                role += " (+ q|k|v partials read)"
        elif "k_mgemv_lds" in short or "k_mgemv<" in short:
            role, alg = "tied head (logits + argmax keys)", w.vocab * d * wb
        elif "k_norm" in short:
            role = "row norm (+ partial fold)"
        elif "k_mgemv_finish" in short:
            role = "split-K finish (GELU / SwiGLU)"
        elif "k_attn_combine" in short:
            role = "attention split combine"
        elif "k_fgemm" in short:
            role = "prefill GEMM (" + {"<0>": "q|k|v", "<1>": "out / down + residual", "<2>": "gate|up + SwiGLU"}.get(
                short[short.index("<"):], "epilogue " + short[short.index("<"):]) + ")"
        elif "k_pf_attn" in short:
            role = "prefill causal attention"
        elif "k_qk_rope_append" in short:
            role = "prefill q/k norm + RoPE + K/V append"
        mu = mf.get(key)
        rows.append((short, grid, n, fb, wb_, role, alg, extra, None if not mu else sum(mu) / len(mu)))
    out = [f"# HBM traffic per kernel: {w.name} (decode window of positions "
           f"{'0' if w.arch == 'whisper' else w.prefill_len}..{(0 if w.arch == 'whisper' else w.prefill_len) + positions - 1})",
           "",
           "Commands (run from /tmp with TMPDIR=/tmp, repository at $R):", ""]
    out += [f"    {c}" for c in commands]
    out += ["",
            f"FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what each reads for the run's "
            f"{COPY_PROBE_BYTES >> 20} MiB device copy (fetch scale {ff_:.3f}, write scale {wf:.3f}).  "
            "`algorithmic` is the kernel's share of the step's bytes (weights read once; self-cache rows "
            "0..pos; the cross cache); `design extra` is what the launch shape adds in HBM traffic: "
            "the fp32 partial slabs a split-K projection writes, or the ones an attention prologue "
            "reads (activation tiles re-read by many workgroups come from the L2 and do not show "
            "here).  Kernels without an algorithmic figure move activations and partial slabs only "
            "(the norms fold the residual projections' slabs, the finish kernel the fc1 / gate|up "
            "slabs)." + ("  The run also holds the 900-position prefill that precedes the decode "
                         "window: its dense GEMMs, causal attention and q/k norm + RoPE + append, "
                         "one dispatch per chunk and layer." if w.arch == "qwen3" else ""), "",
            "| kernel | workgroups | dispatches | fetch B | write B | role | algorithmic B | design extra B | "
            "measured / (alg + extra) | MfmaUtil % |",
            "|---|---|---|---|---|---|---|---|---|---|"]
    for short, grid, n, fb, wb_, role, alg, extra, mu in rows:
        ratio = ""
        if alg:
            ratio = f"{(fb + wb_) / (alg + (extra or 0)):.2f}"
        out.append(f"| `{short[:70]}` | {grid} | {n} | {fb:,.0f} | {wb_:,.0f} | {role} | "
                   f"{'' if alg is None else f'{alg:,}'} | {'' if extra is None else f'{extra:,}'} | {ratio} | "
                   f"{'' if mu is None else f'{mu:.1f}'} |")
    return "\n".join(out) + "\n"


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


def host_info() -> dict:
    """The host the CPU baseline ran on: CPU model, cores available to this process, and
    the BLAS libraries numpy uses with their thread counts."""
    from threadpoolctl import threadpool_info
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = [{"library": p.get("internal_api"), "version": p.get("version"), "threads": p.get("num_threads")}
            for p in threadpool_info() if p.get("user_api") == "blas"]
    return {"cpu_model": model, "cores_available": len(os.sched_getaffinity(0)), "blas": blas}


def _blas_threads() -> int:
    from threadpoolctl import threadpool_info
    return int(max([p.get("num_threads", 1) for p in threadpool_info()] + [1]))


def _sample_positions(first: int, last: int, n: int):
    """n positions spread evenly over first..last (inclusive)."""
    return sorted({int(round(first + (last - first) * i / max(n - 1, 1))) for i in range(n)})


def cpu_baseline(w, budget_s: float):
    """The oracle as it is (float64 numpy) on the host cores: one stream of the workload,
    its cross K/V, then single decode steps at positions spread over the whole window
    (the self-cache rows below each sampled position hold seeded values of the cache dtype:
    a step's cost does not depend on them), as many as fit the time budget.  tokens/s =
    sampled steps / their time, i.e. the mean step cost over the window."""
    from oracle import whisper as OW
    W = WL.make_weights(w)
    enc = WL.make_encoder_states(w, streams=[0])
    O = OW.WhisperOracle(OW.dims_of(w), W)
    del W
    t0 = time.perf_counter()
    O.cross_kv(enc)
    t_cross = time.perf_counter() - t0
    O.reset(1)
    rng = np.random.default_rng(w.seed)
    for l in range(w.layers):
        O.Ks[l][:] = rng.standard_normal(O.Ks[l].shape).astype(np.float32)
        O.Vs[l][:] = rng.standard_normal(O.Vs[l].shape).astype(np.float32)
    tok = WL.make_prompt(w)[:1, 0]
    times = []
    for n in (128, 64, 32, 16, 8, 4, 2):   # as many spread positions as fit the budget
        pos = _sample_positions(0, w.steps - 1, n)
        t0 = time.perf_counter()
        O.step(tok, [pos[0]])
        one = time.perf_counter() - t0
        if one * n <= budget_s or n == 2:
            times = [one]
            for p_ in pos[1:]:
                t0 = time.perf_counter()
                O.step(tok, [p_])
                times.append(time.perf_counter() - t0)
            break
    hi = host_info()
    return {"value": len(times) / sum(times), "unit": "tokens/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"1 of {w.batch} streams, one decode step at each of {len(pos)} positions spread evenly over "
                      f"0..{w.steps - 1} (float64 numpy); its cross K/V took {t_cross:.2f} s on top, not counted",
            "cpu_model": hi["cpu_model"], "cores_available": hi["cores_available"], "blas": hi["blas"],
            "s_per_step": sum(times) / len(times)}


def qwen_cpu_baseline(w, budget_s: float):
    """The Qwen3 oracle on the host cores: one stream's decode steps at positions spread over
    the decode window (the K/V rows below each hold seeded values of the cache dtype; no
    prefill), as many as fit about `budget_s` seconds."""
    from oracle import qwen3 as OQ
    W = WL.make_weights(w)
    O = OQ.QwenOracle(OQ.dims_of(w), W, round_cache=True)
    del W
    O.reset(1)
    rng = np.random.default_rng(w.seed)
    for l in range(w.layers):
        O.K[l][:] = rng.standard_normal(O.K[l].shape).astype(np.float16)
        O.V[l][:] = rng.standard_normal(O.V[l].shape).astype(np.float16)
    ids = WL.random_ids(w, 1)[:1, 0]
    first, last = w.prefill_len, w.prefill_len + w.steps - 1
    times = []
    for n in (64, 32, 16, 8, 4, 2):
        pos = _sample_positions(first, last, n)
        t0 = time.perf_counter()
        O.step(ids, [pos[0]])
        one = time.perf_counter() - t0
        if one * n <= budget_s or n == 2:
            times = [one]
            for p_ in pos[1:]:
                t0 = time.perf_counter()
                O.step(ids, [p_])
                times.append(time.perf_counter() - t0)
            break
    hi = host_info()
    return {"value": len(times) / sum(times), "unit": "tokens/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"1 of {w.batch} streams, one decode step at each of {len(pos)} positions spread evenly over "
                      f"{first}..{last} (float64 numpy, no prefill)", "cpu_model": hi["cpu_model"], "cores_available": hi["cores_available"],
            "blas": hi["blas"], "s_per_step": sum(times) / len(times)}


WDT = {"f32": "float32", "f16": "float16", "bf16": "bfloat16"}


def _tdt(name):
    import torch
    return getattr(torch, WDT[name])


def bench_whisper_greedy(w, windows: int, warmup: int, args, graphs_off_windows: int = 0):
    """Greedy windows of a Whisper workload: each window is wd_cross_kv of every layer, then
    every position for all rows, the argmax of a step feeding the next (after the prompt).
    Returns the measured figures and the decoder (for the kernel timing)."""
    import torch

    import kv_cached_autoregressive_amd as K
    dev = torch.device("cuda:0")
    W = WL.make_weights(w)
    enc_np = WL.make_encoder_states(w)
    dec = K.Decoder(w, W)
    del W
    enc = torch.from_numpy(enc_np).to(dev, _tdt(w.w_dtype))
    del enc_np
    B, S = w.batch, w.steps
    prompt = torch.from_numpy(WL.make_prompt(w).T.copy()).to(dev)          # [4, B]
    pos_all = torch.arange(S, dtype=torch.int32, device=dev)[:, None].repeat(1, B).contiguous()
    amax = torch.zeros(B, dtype=torch.int32, device=dev)
    stream, ctx = dec.stream, dec.ctx

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
    for _ in range(warmup):
        window()
    torch.cuda.synchronize()
    if dec.check() != 0:
        raise RuntimeError(dec.last_error())
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(windows)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(windows):
        ev[i][0].record(stream)
        window(ev[i][1])
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    if dec.check() != 0:
        raise RuntimeError(dec.last_error())
    win_ms = [e[0].elapsed_time(e[2]) for e in ev]
    xkv_ms = [e[0].elapsed_time(e[1]) for e in ev]
    dec_ms = [a - b for a, b in zip(win_ms, xkv_ms)]
    total_ms = ev[0][0].elapsed_time(ev[-1][2])
    bytes_window = sum(whisper_bytes_per_step(w, p) for p in range(S))
    mean_dec = sum(dec_ms) / windows
    out = {"workload": w.name, "batch": B, "positions": S,
           "tokens_per_s": B * S * windows / (total_ms / 1e3), "ms_per_window": total_ms / windows,
           "ms_per_window_median": float(np.median(win_ms)),
           "decode_tokens_per_s": B * S / (mean_dec / 1e3), "decode_ms_per_window": mean_dec,
           "decode_ms_per_window_median": float(np.median(dec_ms)),
           "hbm_bytes_per_window": bytes_window,
           "hbm_gbps_decode": bytes_window / (mean_dec / 1e3) / 1e9,
           "hbm_frac_decode": bytes_window / (mean_dec / 1e3) / HBM_PEAK,
           "cross_kv_ms": sum(xkv_ms) / windows,
           "cross_kv_tflops": 2.0 * w.n_enc * w.frames * w.d * 2 * w.d * w.layers / (sum(xkv_ms) / windows / 1e3) / 1e12,
           "windows": windows, "wall_s": wall}
    if graphs_off_windows:
        # the same windows with every kernel launched eagerly (no captured step graphs)
        dec.set_graphs(False)
        window()
        torch.cuda.synchronize()
        off = []
        for _ in range(graphs_off_windows):
            e1, e2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            window(e1)
            e2.record(stream)
            torch.cuda.synchronize()
            off.append(e1.elapsed_time(e2))
        dec.set_graphs(True)
        off_dec = sum(off) / len(off)
        out["graphs_off"] = {"decode_tokens_per_s": B * S / (off_dec / 1e3), "decode_ms_per_window": off_dec,
                             "hbm_frac_decode": bytes_window / (off_dec / 1e3) / HBM_PEAK,
                             "windows": graphs_off_windows}
        if dec.check() != 0:
            raise RuntimeError(dec.last_error())
    # the dominant kernel: HIP events on the decoder's stream around the cross-attention of
    # one layer, issued `repeats` times back to back per step (the launch is idempotent),
    # over the first positions of a window run right after the timed ones (steps are
    # launched one by one there: a captured step replays without per-launch host hooks);
    # the cross-attention reads all frames at every position, so any positions will do
    K.wd_profile(ctx, K.K_CROSS_ATTN, args.profile_layer, args.profile_repeats)
    steps(min(S, args.profile_positions))
    attn_ms, attn_n = K.wd_profile_read(ctx)
    K.wd_profile(ctx, -1, -1, 1)
    attn_bytes = cross_attn_bytes_per_launch(w)
    attn_avg_s = attn_ms / 1e3 / max(attn_n, 1)
    out["roofline"] = {"kernel": "k_attn (cross-attention, one layer per launch)", "bound": "hbm",
                       "achieved": attn_bytes / attn_avg_s / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                       "frac": attn_bytes / attn_avg_s / HBM_PEAK, "traffic": traffic_per_launch(w.name),
                       "bytes_per_launch": attn_bytes, "avg_launch_us": attn_avg_s * 1e6, "launches_timed": attn_n}
    return out, dec, enc


def bench_qwen(w, runs: int, warmup: int, args):
    """Qwen3-ASR: a 900-position prefill (audio rows spliced in), then the greedy decode steps
    to the context end, argmax on the device.  The prefill is timed separately."""
    import torch

    import kv_cached_autoregressive_amd as K
    dev = torch.device("cuda:0")
    W = WL.make_weights(w)
    ids_np, audio_np = WL.make_qwen_prefill(w)
    dec = K.Decoder(w, W)
    del W
    B, T, S = w.batch, w.prefill_len, w.steps
    ids = torch.from_numpy(np.ascontiguousarray(ids_np)).to(dev, torch.int32)
    audio = torch.from_numpy(np.ascontiguousarray(audio_np)).to(dev, _tdt(w.w_dtype))
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
    for _ in range(warmup):
        prefill()
        steps(S)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(runs)]
    wall0 = time.perf_counter()
    for i in range(runs):
        ev[i][0].record(stream)
        prefill()
        ev[i][1].record(stream)
        steps(S)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    if dec.check() != 0:
        raise RuntimeError(dec.last_error())
    pre = [e[0].elapsed_time(e[1]) for e in ev]
    dms = [e[1].elapsed_time(e[2]) for e in ev]
    dec_ms = sum(dms) / runs
    # kernel timing: the gate|up projection of one layer (the largest weight stream of a layer)
    prefill()
    K.wd_profile(ctx, K.K_FC1, args.profile_layer, args.profile_repeats)
    steps(min(S, args.profile_positions))
    k_ms, k_n = K.wd_profile_read(ctx)
    K.wd_profile(ctx, -1, -1, 1)
    gu_bytes = 2 * w.d_ff * w.d * DT_BYTES[w.w_dtype]
    k_avg = k_ms / 1e3 / max(k_n, 1)
    bytes_dec = sum(qwen_bytes_per_step(w, T + p) for p in range(S))
    out = {"workload": w.name, "batch": B, "prefill": T, "positions": S,
           "tokens_per_s": B * S / (dec_ms / 1e3), "decode_tokens_per_s": B * S / (dec_ms / 1e3),
           "decode_ms": dec_ms, "decode_ms_median": float(np.median(dms)),
           "prefill_ms": sum(pre) / runs, "prefill_ms_median": float(np.median(pre)),
           "hbm_bytes_decode": bytes_dec, "hbm_gbps_decode": bytes_dec / (dec_ms / 1e3) / 1e9,
           "hbm_frac_decode": bytes_dec / (dec_ms / 1e3) / HBM_PEAK, "runs": runs, "wall_s": wall,
           "roofline": {"kernel": "gate|up projection (MFMA skinny GEMM, one layer per launch)", "bound": "hbm",
                        "achieved": gu_bytes / k_avg / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                        "frac": gu_bytes / k_avg / HBM_PEAK, "traffic": None, "bytes_per_launch": gu_bytes,
                        "avg_launch_us": k_avg * 1e6, "launches_timed": k_n}}
    return out, dec


def _beam_merge(scores, vals, ids, lse, V, first):
    """One width-W beam step from per-row device candidates: scores S_b + (logit - lse_b) of
    the W x W candidates (only row 0 at the first generated position, where every row holds
    the same prefix), the W best kept, ties to the lower flat index b * V + v."""
    W = vals.shape[0]
    rows = 1 if first else W
    cand = np.asarray(scores, np.float64)[:rows, None] + (vals[:rows].astype(np.float64) -
                                                          lse[:rows, None].astype(np.float64))
    flat = (np.arange(rows)[:, None] * V + ids[:rows]).reshape(-1)
    c = cand.reshape(-1)
    keep = np.lexsort((flat, -c))[:W]
    return (flat[keep] // V).astype(np.int32), (flat[keep] % V).astype(np.int32), c[keep]


def bench_beam(w, runs: int, warmup: int):
    """Width-W beam search over one broadcast encoder set, all on the device: per position
    wd_step (logits) and wd_beam_step (candidates, W x W merge, cache rearrangement, the next
    tokens written into the step's token buffer), with no host round trip inside a run.
    tokens/s counts every row of every step.  One more run takes the candidates to the host
    for the merge and calls wd_reorder (the step without wd_beam_step), for comparison."""
    import torch

    import kv_cached_autoregressive_amd as K
    dev = torch.device("cuda:0")
    W = WL.make_weights(w)
    enc = torch.from_numpy(WL.make_encoder_states(w)).to(dev, _tdt(w.w_dtype))
    dec = K.Decoder(w, W)
    del W
    B, S, V = w.batch, w.steps, w.vocab
    prompt = WL.make_prompt(w)
    P = prompt.shape[1]
    prompt_dev = torch.from_numpy(np.ascontiguousarray(prompt.T, dtype=np.int32)).to(dev)   # [P, B]
    logits = torch.empty(B, V, dtype=torch.float32, device=dev)
    amax = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.zeros(B, dtype=torch.int32, device=dev)
    pos_all = torch.arange(S, dtype=torch.int32, device=dev)[:, None].repeat(1, B).contiguous()
    scores = torch.zeros(B, dtype=torch.float64, device=dev)
    bidx = torch.zeros(B, dtype=torch.int32, device=dev)
    stream, ctx = dec.stream, dec.ctx
    torch.cuda.set_stream(stream)

    def run():
        K.wd_cross_kv(ctx, enc.data_ptr(), w.frames)
        scores.zero_()
        for p in range(S):
            if p < P:
                tok.copy_(prompt_dev[p])
            K.wd_step(ctx, tok.data_ptr(), pos_all[p].data_ptr(), B, logits.data_ptr(), amax.data_ptr())
            if p >= P - 1:
                K.wd_beam_step(ctx, logits.data_ptr(), B, p == P - 1, scores.data_ptr(), bidx.data_ptr(),
                               tok.data_ptr(), p + 1 if p + 1 < S else 0)

    vals = torch.empty(B, B, dtype=torch.float32, device=dev)
    ids = torch.empty(B, B, dtype=torch.int32, device=dev)
    lse = torch.empty(B, dtype=torch.float32, device=dev)
    host = torch.empty(2 * B * B + B, dtype=torch.float32).pin_memory()

    def run_host_merge():
        K.wd_cross_kv(ctx, enc.data_ptr(), w.frames)
        sc_h = np.zeros(B)
        toks = prompt[:, 0]
        for p in range(S):
            if p < P:
                toks = prompt[:, p]
            tok.copy_(torch.from_numpy(np.ascontiguousarray(toks, dtype=np.int32)), non_blocking=False)
            K.wd_step(ctx, tok.data_ptr(), pos_all[p].data_ptr(), B, logits.data_ptr(), amax.data_ptr())
            if p >= P - 1:
                K.wd_topk(ctx, logits.data_ptr(), B, B, vals.data_ptr(), ids.data_ptr(), lse.data_ptr())
                host[:B * B].copy_(vals.view(-1), non_blocking=True)
                host[B * B:2 * B * B].copy_(ids.view(torch.float32).view(-1), non_blocking=True)
                host[2 * B * B:].copy_(lse, non_blocking=True)
                stream.synchronize()
                h = host.numpy()
                bi, tk, sc = _beam_merge(sc_h, h[:B * B].reshape(B, B), h[B * B:2 * B * B].view(np.int32).reshape(B, B),
                                         h[2 * B * B:], V, p == P - 1)
                if p + 1 < S:
                    K.wd_reorder(ctx, bi.tolist(), p + 1)
                sc_h, toks = sc, tk
        return np.asarray(toks)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record(stream)
    for _ in range(runs):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gpu_s = e0.elapsed_time(e1) / 1e3 / runs
    dev_tokens = tok.cpu().numpy().copy()
    run_host_merge()
    torch.cuda.synchronize()
    hm0 = time.perf_counter()
    host_tokens = run_host_merge()
    torch.cuda.synchronize()
    host_wall = time.perf_counter() - hm0
    if dec.check() != 0:
        raise RuntimeError(dec.last_error())
    bytes_run = sum(whisper_bytes_per_step(w, p) for p in range(S))
    out = {"workload": w.name, "beams": B, "positions": S,
           "tokens_per_s": B * S * runs / wall, "tokens_per_s_gpu": B * S / gpu_s,
           "ms_per_run_wall": wall / runs * 1e3, "ms_per_run_gpu": gpu_s * 1e3,
           "hbm_bytes_per_run": bytes_run, "hbm_frac_decode_gpu": bytes_run / gpu_s / HBM_PEAK,
           "runs": runs,
           "host_merge": {"tokens_per_s": B * S / host_wall, "ms_per_run_wall": host_wall * 1e3,
                          "same_final_tokens": bool(np.array_equal(dev_tokens, host_tokens))},
           "step": "wd_step + wd_beam_step (candidates, merge and cache rearrangement on the device) every "
                   "position, no host round trip; host_merge: the candidates merged on the host and "
                   "wd_reorder, one run"}
    del dec
    return out


def _extra_workloads(args):
    """The other four workloads, at a fixed small number of windows each (their figures ride
    along the headline line)."""
    import torch
    out = {}
    for name, fn in (("whisper_small_f16_b16", lambda w: bench_whisper_greedy(w, 3, 1, args, graphs_off_windows=1)),
                     ("whisper_tiny_f32_b1", lambda w: bench_whisper_greedy(w, 5, 1, args, graphs_off_windows=1)),
                     ("qwen3asr_bf16_b8", lambda w: bench_qwen(w, 3, 1, args)),
                     ("whisper_base_f16_beam5", lambda w: (bench_beam(w, 2, 1),))):
        w = WL.by_name(name)
        r = fn(w)
        out[name] = r[0]
        del r
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def floors(w, full=True):
    """The costs the decode kernels are bounded by on this device, from wd_probe: the per-launch
    cost of a graph of dependent empty kernels (1280 blocks, like the large-v3 attention grids),
    and one kernel that only streams the bytes of one cross-attention launch of the workload (its
    K and V caches as two buffers, read with the attention's 16-byte nontemporal lane loads);
    with full, also the hand-off of the residual rows between dependent launches (same / other
    XCD) and an in-kernel fence reduction over 256 / 1024 workgroups.  Medians of five
    measurements each; the buffers are allocated once and stay resident."""
    import torch
    import kv_cached_autoregressive_amd as K
    kv = w.n_enc * w.heads * w.frames * (w.d // w.heads) * {"f32": 4, "f16": 2, "bf16": 2}[w.cache_dtype]
    a = torch.empty(kv, dtype=torch.uint8, device="cuda")
    b = torch.empty(kv, dtype=torch.uint8, device="cuda")
    a.random_(0, 256)
    b.random_(0, 256)
    sink = torch.zeros(4096, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    launch = float(np.median([K.wd_probe(0, iters=1000) for _ in range(5)]))
    stream = float(np.median([K.wd_probe(1, a.data_ptr(), b.data_ptr(), kv, 20, sink.data_ptr()) for _ in range(5)]))
    rate = 2 * kv / stream / 1e3   # GB/s
    out = {"empty_dependent_launch_us": launch,
           "stream_bytes": 2 * kv, "stream_us": stream, "stream_gbps": rate,
           "stream_frac_of_8tbps": rate / 8000.0,
           # repeated reads of less than the 256 MB MALL come from it, not from HBM
           "stream_fits_mall": 2 * kv <= 256 * 2**20}
    probe = ("wd_probe kind 0 (1000 graph-captured launches of 1280 empty blocks), "
             "kind 1 (20 launches reading the K and V bytes of one cross-attention launch)")
    if full:
        # a decode step's hand-off: the B x d fp32 residual rows (rounded up to 4 KiB per 256 blocks)
        act = -(-w.batch * w.d * 4 // 4096) * 4096
        hand = {k: float(np.median([K.wd_probe(k, a.data_ptr(), b.data_ptr(), act, 1000) for _ in range(5)]))
                for k in (2, 3)}
        ctr = torch.zeros(2, dtype=torch.int32, device="cuda")
        fence = {k: float(np.median([K.wd_probe(k, a.data_ptr(), ctr.data_ptr(), 4096, 200) for _ in range(5)]))
                 for k in (4, 5)}
        out.update({"handoff_bytes": act, "handoff_same_xcd_us": hand[2], "handoff_cross_xcd_us": hand[3],
                    "fence_reduce_256_blocks_us": fence[4], "fence_reduce_1024_blocks_us": fence[5]})
        probe += (", kinds 2, 3 (1000 graph-captured dependent hand-offs of the residual rows, same / other "
                  "XCD) and kinds 4, 5 (200 in-kernel fence reductions over 256 / 1024 blocks)")
    out["probe"] = probe
    del a, b
    torch.cuda.empty_cache()
    return out


def run_floors(w):
    print(json.dumps({"metric": "machine floors", "workload": w.name, **floors(w)}))


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3, help="timed windows")
    ap.add_argument("--warmup", type=int, default=1, help="untimed windows")
    ap.add_argument("--config", default=DEFAULT)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="time the --config workload only (the default run also times the other four)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle decode steps")
    ap.add_argument("--profile-layer", type=int, default=0, help="layer whose dominant-kernel launches are timed")
    ap.add_argument("--profile-positions", type=int, default=16, help="positions of the kernel-timing run")
    ap.add_argument("--profile-repeats", type=int, default=8, help="back-to-back launches per timed event pair")
    ap.add_argument("--positions", type=int, default=0,
                    help="profiling aid: decode only the first N positions of each window")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="after the run, one device copy of a known size (counter calibration)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the cross-attention traffic summary under profiles/ from two --pmc runs and exit")
    ap.add_argument("--commands", nargs="*", default=[], help="the profiler commands, recorded in the summary")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/counters_<config>.md (HBM bytes per kernel against algorithmic bytes) "
                         "from two --pmc runs of the --config workload with --positions and exit")
    ap.add_argument("--mfma-csv", default=None, help="with --summarize-counters: a third --pmc MfmaUtil run")
    ap.add_argument("--encoder", action="store_true",
                    help="time the audio encoder (wd_encode) of the workload's encoder sets instead of the decoder")
    ap.add_argument("--encoder-layers", type=int, default=0, help="encoder layers (default: the decoder's)")
    ap.add_argument("--mels", type=int, default=80, help="mel channels of the encoder's input")
    ap.add_argument("--floors", action="store_true",
                    help="measure the machine floors the decode kernels run against (wd_probe) and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        w = WL.by_name(args.config)
        md = summarize_counters(*args.summarize_counters, w, args.positions or w.steps, args.commands, args.mfma_csv)
        with open(os.path.join(ROOT, "profiles", f"counters_{w.name}.md"), "w") as f:
            f.write(md)
        print(md)
        return
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
    if args.encoder:
        run_encoder(args, w)
        return
    if args.floors:
        run_floors(w)
        return
    metric = "decoder tokens/sec at batch B; achieved HBM GB/s as % of MI355X peak"
    common = {"metric": metric, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.w_dtype}
    if w.arch == "qwen3":
        r, dec = bench_qwen(w, args.steps, args.warmup, args)
        if args.traffic_probe:
            traffic_probe_copy(dev)
        del dec
        out = dict(common, value=r["decode_tokens_per_s"], ms_per_step=r["decode_ms"],
                   data="synthetic (seeded random-init weights N(0,0.02), N(0,1) audio rows, uniform ids)",
                   config={"workload": w.name, "batch": w.batch, "prefill": w.prefill_len, "positions": w.steps,
                           "layers": w.layers, "d": w.d, "q_heads": w.heads, "kv_heads": w.kv_heads,
                           "head_dim": w.head_dim, "d_ff": w.d_ff, "vocab": w.vocab, "w_dtype": w.w_dtype,
                           "cache_dtype": w.cache_dtype,
                           "step": "124 greedy decode steps after the prefill (prefill timed separately)"})
        out.update({k: v for k, v in r.items() if k not in ("workload", "batch", "positions", "tokens_per_s")})
        torch.cuda.empty_cache()
        out["cpu_baseline"] = None if args.no_cpu_baseline else qwen_cpu_baseline(w, args.cpu_budget)
        print(json.dumps(out), flush=True)
        return
    if w.mode != "greedy":
        r = bench_beam(w, args.steps, args.warmup)
        out = dict(common, value=r["tokens_per_s"], ms_per_step=r["ms_per_run_wall"],
                   data="synthetic (seeded random-init weights N(0,0.02), encoder states N(0,1))",
                   config={"workload": w.name, "beams": w.batch, "positions": w.steps, "layers": w.layers,
                           "d": w.d, "vocab": w.vocab, "w_dtype": w.w_dtype, "cache_dtype": w.cache_dtype})
        out.update(r)
        out["cpu_baseline"] = None
        print(json.dumps(out), flush=True)
        return

    r, dec, enc = bench_whisper_greedy(w, args.steps, args.warmup, args,
                                       graphs_off_windows=0 if args.no_extra else 1)
    if args.traffic_probe:
        traffic_probe_copy(dev)
    del dec, enc
    torch.cuda.empty_cache()
    out = dict(common, value=r["tokens_per_s"], ms_per_step=r["ms_per_window"],
               data="synthetic (seeded random-init weights N(0,0.02), encoder states N(0,1))",
               config={"workload": w.name, "batch": w.batch, "positions": w.steps, "frames": w.frames,
                       "layers": w.layers, "d": w.d, "heads": w.heads, "d_ff": w.d_ff,
                       "vocab": w.vocab, "w_dtype": w.w_dtype, "cache_dtype": w.cache_dtype,
                       "step": "one window: cross K/V projection + all positions, greedy on device"})
    out.update({k: v for k, v in r.items() if k not in ("workload", "batch", "positions", "tokens_per_s",
                                                        "ms_per_window", "windows")})
    if not args.no_extra and w.name == DEFAULT:
        out["workloads"] = _extra_workloads(args)
        # the plain read of one cross-attention launch's bytes: the practical ceiling of roofline.frac
        f = floors(w, full=False)
        out["floors"] = f
        if (out.get("roofline") or {}).get("avg_launch_us"):
            out["roofline"]["frac_of_plain_read"] = f["stream_us"] / out["roofline"]["avg_launch_us"]
    out["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input:
the dense causal prefill (B=4, H=16, S=2048, d=128, bf16) through mxfa_fwd,
and the latent-KV split decode (batch 128, q_len 4, 16 heads, 576/512,
kv_len 8192, bf16) through mxfa_decode_splitkv. Inputs are generated with the
seeded recipe of the ``workloads`` module and are resident in HBM before the
timed region. Each workload first runs back to back for about ``--settle-ms``
of GPU time (the chip's clock then settles at its sustained level for that
load, which the bench samples and reports), then ``--warmup`` untimed calls,
then ``--repeats`` timed regions of exactly ``--steps`` calls, each bracketed
by HIP events on the stream the calls are launched on.

Prints ONE JSON line. ``value`` is the prefill's algorithmic TFLOP/s (4*d
flops per visible (query, key) pair); the ``decode`` object carries the
decode's algorithmic HBM GB/s (Q + latent KV + O + LSE bytes, each once).
``roofline`` compares the prefill kernel with the bf16 MFMA peak;
``cpu_baseline`` times the fp64 oracle on a bounded sample of the same
prefill workload on the host cores.

Options: --gpus N (only 1 is supported), --steps K, --warmup W, --settle-ms T,
--workloads a,b,... (default: causal_prefill_bf16,mla_decode_bf16; "all"
adds the other configurations as extra lines in ``extra``),
--no-cpu-baseline, --cpu-seconds S.

Traffic counters: run the bench under ``rocprofv3 --pmc FETCH_SIZE`` and,
separately, ``--pmc WRITE_SIZE`` with ``--copy-probe-mb N`` (a device copy of
N MiB after the workloads, whose counter readings calibrate the counters),
then ``python bench.py --pmc-summarize FETCH_CSV WRITE_CSV --copy-probe-mb N``
writes profiles/pmc_traffic.json: measured HBM bytes per launch for each
kernel, tagged with a hash of the kernel's code (comments and whitespace
aside; the figures are ignored once that code changes).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s (prefill, % MFMA peak); decode HBM GB/s (% peak)"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
PRIMARY = "causal_prefill_bf16"
DECODE = "mla_decode_bf16"
KERNEL_SOURCES = {
    "fwd_bf16": "tiled_attention_amd/csrc/fwd_bf16.hip",
    "fwd_f32": "tiled_attention_amd/csrc/fwd_f32.hip",
    "decode_mla": "tiled_attention_amd/csrc/decode_mla.hip",
    "decode_mla_paged": "tiled_attention_amd/csrc/decode_mla.hip",
    "decode_mla_fp8": "tiled_attention_amd/csrc/decode_mla.hip",
    "decode_gqa": "tiled_attention_amd/csrc/decode_gqa.hip",
}


def visible_pairs(lens_q, lens_k, causal, window):
    """Exact number of visible (query, key) pairs (bottom-right alignment, inclusive window)."""
    total = 0
    wl, wr = window
    for sq, sk in zip(lens_q, lens_k):
        if sq == 0 or sk == 0:
            continue
        pos = np.arange(sq, dtype=np.int64) + (sk - sq)
        lo = np.zeros(sq, dtype=np.int64) if wl < 0 else np.maximum(0, pos - wl)
        hi = np.full(sq, sk - 1, dtype=np.int64)
        if causal:
            hi = np.minimum(hi, pos)
        if wr >= 0:
            hi = np.minimum(hi, pos + wr)
        total += int(np.maximum(0, hi - lo + 1).sum())
    return total


def work_of(w, inp):
    """Algorithmic flops and bytes of one call on workload w."""
    pairs = visible_pairs(inp["lens_q"], inp["lens_k"], w.causal, w.window) * w.heads_q
    flops = pairs * 2 * (w.d_qk + w.d_v)
    esz = 4 if w.dtype == "f32" else 2
    tq, tk = sum(inp["lens_q"]), sum(inp["lens_k"])
    q_b = tq * w.heads_q * w.d_qk * esz
    o_b = tq * w.heads_q * w.d_v * esz
    lse_b = tq * w.heads_q * 4
    if w.kind == "decode":
        kv_esz = 1 if w.kv_dtype == "fp8" else esz
        kv_b = tk * w.heads_kv * w.d_qk * kv_esz  # shared latent kv, read once
    else:
        kv_b = tk * w.heads_kv * (w.d_qk + w.d_v) * esz
    return pairs, flops, q_b + kv_b + o_b + lse_b


# Headers every kernel source includes: a change there changes the kernels too.
SHARED_SOURCES = ("tiled_attention_amd/csrc/mxfa_device.h", "tiled_attention_amd/csrc/mxfa_internal.h")


def _code_only(text):
    """C++ source without comments and whitespace (string literals kept)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"' or c == "'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            if not c.isspace():
                out.append(c)
            i += 1
    return "".join(out)


def source_sha(name):
    """Hash of the code (comments and whitespace aside) of a kernel's source and the shared headers."""
    h = hashlib.sha256()
    for rel in (KERNEL_SOURCES[name],) + SHARED_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


# rocprofv3 kernel names of each kernel family (one launch of mxfa_decode_splitkv
# is one split kernel plus one combine kernel).
PMC_KERNELS = {
    "fwd_bf16": ("fwd_bf16_kernel<128, 0>",),
    "decode_mla": ("decode_split_kernel<false, false, false>", "decode_combine_kernel"),
    "decode_mla_paged": ("decode_split_kernel<false, true, false>", "decode_combine_kernel"),
    "decode_mla_fp8": ("decode_split_kernel<false, false, true>", "decode_combine_kernel"),
    "decode_gqa": ("decode_gqa_split_kernel<128, false>", "decode_gqa_combine_kernel<128>"),
}
COPY_KERNEL_MARKERS = ("copyBuffer", "copy_kernel", "CopyKernel")


def _pmc_readings(csv_path, counter):
    """Counter values (KiB) of every dispatch, by kernel name."""
    import csv

    out = {}
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter:
                out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return out


def pmc_summarize(fetch_csv, write_csv, copy_mb):
    """Turn two rocprofv3 PMC runs into bytes per launch per kernel family."""
    fetch_all = _pmc_readings(fetch_csv, "FETCH_SIZE")
    write_all = _pmc_readings(write_csv, "WRITE_SIZE")
    fetch = {k: sum(v) / len(v) for k, v in fetch_all.items()}
    write = {k: sum(v) / len(v) for k, v in write_all.items()}

    def copy_reading(readings):
        cands = [x for k, v in readings.items() if any(m in k for m in COPY_KERNEL_MARKERS) for x in v]
        if not cands:
            raise SystemExit("no copy kernel in the counter file; run with --copy-probe-mb")
        return max(cands)  # the probe copy is the largest copy dispatch in the run

    copy_bytes = copy_mb * 2 ** 20
    f_scale = copy_bytes / (copy_reading(fetch_all) * 1024.0)
    w_scale = copy_bytes / (copy_reading(write_all) * 1024.0)
    out = {"_calibration": {"copy_bytes": copy_bytes, "fetch_scale": f_scale, "write_scale": w_scale,
                            "note": "bytes = counter KiB * 1024 * scale; scale = copy bytes / copy reading"}}
    for fam, names in PMC_KERNELS.items():
        fb = wb = 0.0
        raw = {}
        for n in names:
            fk = [v for k, v in fetch.items() if n in k]
            wk = [v for k, v in write.items() if n in k]
            if not fk or not wk:
                break
            raw[n] = {"FETCH_SIZE_KiB": fk[0], "WRITE_SIZE_KiB": wk[0]}
            fb += fk[0] * 1024.0 * f_scale
            wb += wk[0] * 1024.0 * w_scale
        else:
            out[fam] = {"source_sha": source_sha(fam), "bytes_per_launch": round(fb + wb),
                        "fetch_bytes": round(fb), "write_bytes": round(wb), "raw": raw}
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def trace_summarize(trace_csv, names, tail=1000, probes=8):
    """Per-dispatch durations of a rocprofv3 kernel trace of a bench run, by workload and kernel.

    The trace is cut into the bench's workloads (named in its order by
    ``names``): a workload ends once its ``probes`` clock probes have run and
    a kernel it did not launch appears. Prints one markdown row per
    (workload, kernel, grid): calls, mean over all dispatches, and median /
    min / max over the last ``tail`` dispatches (a workload's timed calls
    come last).
    """
    import csv

    rows = []
    with open(trace_csv) as f:
        for row in csv.DictReader(f):
            rows.append((int(row["Start_Timestamp"]), int(row["End_Timestamp"]), row["Kernel_Name"],
                         int(row["Grid_Size_X"]) // max(1, int(row["Workgroup_Size_X"]))))
    rows.sort()
    segments = [{"groups": {}, "probes": 0}]
    for st, en, name, wgs in rows:
        short = name.replace("(anonymous namespace)::", "").replace("mxfa::", "")
        short = (short[5:] if short.startswith("void ") else short).split("(")[0]
        if short.startswith("at::") or "copyBuffer" in short:
            continue  # torch's fills and copies of the harness
        seg = segments[-1]
        if short == "clock_probe_kernel":
            seg["probes"] += 1
            continue
        key = (short, wgs)
        if seg["probes"] >= probes and key not in seg["groups"]:
            seg = {"groups": {}, "probes": 0}
            segments.append(seg)
        seg["groups"].setdefault(key, []).append((en - st) / 1000.0)
    print("| Workload | Kernel | Work groups | Calls | Mean, all (us) | Median, last %d (us) | Min | Max |" % tail)
    print("|---|---|---|---|---|---|---|---|")
    for i, seg in enumerate(segments):
        label = names[i] if i < len(names) else f"segment {i}"
        for (short, wgs), v in seg["groups"].items():
            allv, last = np.array(v), np.array(v[-tail:])
            print(f"| {label} | `{short}` | {wgs} | {len(v)} | {allv.mean():.1f} | {np.median(last):.1f} | "
                  f"{last.min():.1f} | {last.max():.1f} |")


def load_traffic(kernel):
    """HBM traffic per launch from committed rocprofv3 PMC runs, if taken on this exact source."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != source_sha(kernel):
        return None
    return rec.get("bytes_per_launch")


class Runner:
    """Inputs resident on the GPU plus a closure that launches one call."""

    def __init__(self, name):
        import torch

        import tiled_attention_amd as mx
        import workloads

        self.w = w = workloads.get(name)
        inp = workloads.make_inputs(w)
        dev = torch.device("cuda:0")
        self.pairs, self.flops, self.bytes = work_of(w, inp)
        scale = w.softmax_scale
        if w.kind == "dense":
            q, k, v = (inp[x].to(dev) for x in "qkv")
            o = torch.empty_like(q)
            lse = torch.empty((w.batch, w.heads_q, w.seqlen_q), dtype=torch.float32, device=dev)
            self.call = lambda: mx.mxfa_fwd(q, k, v, causal=w.causal, window=w.window, softcap=w.softcap,
                                            scale=scale, out=o, lse=lse)
            self.kernel = "fwd_bf16" if w.dtype == "bf16" else "fwd_f32"
        elif w.kind == "gqa_decode":
            q, k, v = (inp[x].to(dev) for x in "qkv")
            cq, ck = inp["cu_seqlens_q"].to(dev), inp["cu_seqlens_k"].to(dev)
            o = torch.empty_like(q)
            lse = torch.empty((w.heads_q, q.shape[0]), dtype=torch.float32, device=dev)
            self.splits = mx.mxfa_decode_splitkv_gqa_num_splits(w.batch, w.seqlen_q, w.seqlen_k, w.heads_q,
                                                                w.heads_kv)
            nbytes = mx.mxfa_decode_splitkv_gqa_workspace_bytes(w.batch, w.seqlen_q, w.seqlen_k, w.heads_q,
                                                                w.heads_kv, w.d_qk)
            ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
            self.call = lambda: mx.mxfa_decode_splitkv_gqa(q, k, v, cq, ck, w.seqlen_q, w.seqlen_k, causal=w.causal,
                                                           window=w.window, softcap=w.softcap, scale=scale,
                                                           workspace=ws, out=o, lse=lse)
            self.kernel = "decode_gqa"
        elif w.kind == "varlen":
            q, k, v = (inp[x].to(dev) for x in "qkv")
            cq, ck = inp["cu_seqlens_q"].to(dev), inp["cu_seqlens_k"].to(dev)
            mq, mk = max(inp["lens_q"]), max(inp["lens_k"])
            o = torch.empty_like(q)
            lse = torch.empty((w.heads_q, q.shape[0]), dtype=torch.float32, device=dev)
            nbytes = mx.mxfa_fwd_varlen_workspace_bytes(w.batch, mq, w.heads_q, w.d_qk)
            ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
            self.call = lambda: mx.mxfa_fwd_varlen(q, k, v, cq, ck, mq, mk, causal=w.causal, window=w.window,
                                                   softcap=w.softcap, scale=scale, workspace=ws, out=o, lse=lse)
            self.kernel = "fwd_bf16"
        else:
            q = inp["q"].to(dev)
            cq = inp["cu_seqlens_q"].to(dev)
            o = torch.empty((q.shape[0], w.heads_q, w.d_v), dtype=q.dtype, device=dev)
            lse = torch.empty((w.heads_q, q.shape[0]), dtype=torch.float32, device=dev)
            self.splits = mx.mxfa_decode_splitkv_num_splits(w.batch, w.seqlen_q, w.seqlen_k, w.heads_q, w.heads_kv)
            nbytes = mx.mxfa_decode_splitkv_workspace_bytes(w.batch, w.seqlen_q, w.seqlen_k, w.heads_q,
                                                            w.heads_kv, w.d_v)
            ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            if w.kv_dtype == "fp8":
                kv8, ck = inp["kv8"].to(dev), inp["cu_seqlens_k"].to(dev)
                kv_scale = inp["kv_scale"]
                self.call = lambda: mx.mxfa_decode_splitkv_fp8(q, kv8, cq, ck, w.seqlen_q, w.seqlen_k, kv_scale,
                                                               head_dim_v=w.d_v, scale=scale, workspace=ws, out=o,
                                                               lse=lse)
                self.kernel = "decode_mla_fp8"
            elif w.page_size:
                cache = inp["kv_cache"].to(dev)
                seqlens, table = inp["cache_seqlens"].to(dev), inp["block_table"].to(dev)
                self.call = lambda: mx.mxfa_decode_splitkv_paged(q, cache, cq, seqlens, table, w.seqlen_q,
                                                                 w.seqlen_k, head_dim_v=w.d_v, scale=scale,
                                                                 workspace=ws, out=o, lse=lse)
                self.kernel = "decode_mla_paged"
            else:
                kv, ck = inp["kv"].to(dev), inp["cu_seqlens_k"].to(dev)
                self.call = lambda: mx.mxfa_decode_splitkv(q, kv, cq, ck, w.seqlen_q, w.seqlen_k,
                                                           head_dim_v=w.d_v, scale=scale, workspace=ws, out=o,
                                                           lse=lse)
                self.kernel = "decode_mla"
            del inp
        torch.cuda.synchronize()

    def settle(self, ms_target, probes=8):
        """Back-to-back calls for about ``ms_target`` ms of GPU time; returns (calls, ms, clock).

        The chip's shader clock follows its load: after an idle gap the first
        calls of a burst run at a clock the chip does not hold. The bench runs
        this before the warmup calls so that the timed calls see the sustained
        clock. The run is cut into ``probes`` chunks. While each chunk runs,
        the library's shader-clock probe (one wave counting shader cycles
        against the 100 MHz real-time counter for 1 ms) runs alongside it on a
        second stream and reads the clock under this load; ``clock``
        summarises those readings (MHz). A probe run between calls instead
        reads the idle clock (~2.4 GHz), since the clock recovers within
        microseconds; the side-by-side reading still counts the gaps between
        calls and so reads a few percent above the kernels' own clock.
        """
        import torch

        import tiled_attention_amd as mx

        if ms_target <= 0:
            return 0, 0.0, {"mhz": None, "note": "no settle run"}
        stream = torch.cuda.current_stream()
        side = torch.cuda.Stream()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(5):
            self.call()
        end.record(stream)
        torch.cuda.synchronize()
        per = max(start.elapsed_time(end) / 5, 1e-3)
        chunk = max(1, int(ms_target / per / probes))
        buf = torch.zeros(2 * probes, dtype=torch.int64, device="cuda:0")
        start.record(stream)
        for i in range(probes):
            for _ in range(chunk):
                self.call()
            # The host is ahead of the GPU here: the probe runs beside the
            # chunk's remaining calls.
            with torch.cuda.stream(side):
                mx.mxfa_clock_probe(buf[2 * i:2 * i + 2], 1000)
            if i + 1 < probes:
                torch.cuda.synchronize()  # keep the host within one chunk of the GPU
        end.record(stream)
        torch.cuda.synchronize()
        v = buf.cpu().numpy().reshape(-1, 2).astype(np.float64)
        mhz = [round(float(c / t * 100.0), 1) for c, t in v if t > 0]
        clock = {"mhz": round(float(np.median(mhz)), 1) if mhz else None, "probes_mhz": mhz,
                 "source": "in-kernel probe (s_memtime cycles / s_memrealtime ticks over 1 ms) on a second "
                           f"stream beside each of {probes} chunks of {chunk} back-to-back calls; reads a few "
                           "percent above the kernels' own clock (it also counts the gaps between calls)"}
        return chunk * probes, start.elapsed_time(end), clock

    def time(self, steps, warmup, repeats=1):
        """ms per call of each of ``repeats`` timed regions of exactly ``steps`` calls.

        ``warmup`` untimed calls come first. Each region is bracketed by HIP
        events on the stream the calls are launched on, with a device
        synchronisation on both sides.
        """
        import torch

        for _ in range(warmup):
            self.call()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        out = []
        for _ in range(repeats):
            start = torch.cuda.Event(enable_timing=True)
            end = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            start.record(stream)
            for _ in range(steps):
                self.call()
            end.record(stream)
            torch.cuda.synchronize()
            out.append(start.elapsed_time(end) / steps)  # ms per call
        return out


def clock_fields(res, peak):
    """Shader clock seen under sustained load of the workload, and the MFMA peak scaled to it.

    The dense bf16 MFMA peak assumes 2.4 GHz; at a lower clock the chip's
    attainable peak is lower in proportion.
    """
    mhz = (res.get("clock") or {}).get("mhz")
    out = {"clock_mhz": mhz, "clock_probes_mhz": (res.get("clock") or {}).get("probes_mhz"), "peak_clock_mhz": 2400.0}
    if mhz:
        peak_at = peak * mhz / 2400.0
        out["peak_at_clock"] = round(peak_at, 1)
        out["frac_at_clock"] = round(res["tflops"] / peak_at, 4)
    else:
        out["clock_note"] = (res.get("clock") or {}).get("note")
    return out


def cpu_baseline(name, target_s):
    """Time the fp64 oracle on a bounded, seeded sample of workload rows (host cores)."""
    import oracle
    import workloads

    w = workloads.get(name)
    inp = workloads.make_inputs(w)
    to_np = workloads.to_numpy_bits
    if w.kind == "dense":
        q = to_np(inp["q"]).reshape(-1, w.heads_q, w.d_qk)
        k = to_np(inp["k"]).reshape(-1, w.heads_kv, w.d_qk)
        v = to_np(inp["v"]).reshape(-1, w.heads_kv, w.d_v)
    elif w.kind in ("varlen", "gqa_decode"):
        q, k, v = to_np(inp["q"]), to_np(inp["k"]), to_np(inp["v"])
    else:
        q = to_np(inp["q"])
        k = to_np(inp["kv"])
        v = k[:, :, :w.d_v]
    cq, ck = inp["cu_seqlens_q"].numpy(), inp["cu_seqlens_k"].numpy()
    total_rows = q.shape[0] * w.heads_q
    rng = np.random.RandomState(12345)
    order = rng.permutation(total_rows)
    tok_of = order // w.heads_q
    head_of = order % w.heads_q
    # per-row visible key counts for the flop count of the sample
    starts = np.repeat(cq[:-1], np.diff(cq))
    seg = np.repeat(np.arange(len(cq) - 1), np.diff(cq))
    i = np.arange(q.shape[0]) - starts
    sk = (ck[1:] - ck[:-1])[seg]
    sq = (cq[1:] - cq[:-1])[seg]
    pos = i + sk - sq
    lo = np.zeros_like(pos) if w.window[0] < 0 else np.maximum(0, pos - w.window[0])
    hi = sk - 1
    if w.causal:
        hi = np.minimum(hi, pos)
    if w.window[1] >= 0:
        hi = np.minimum(hi, pos + w.window[1])
    cnt = np.maximum(0, hi - lo + 1)
    threads = oracle.threads_used(0)
    n = min(total_rows, 256)
    done = 0
    elapsed = 0.0
    pairs = 0
    while done < total_rows:
        rows = np.stack([tok_of[done:done + n], head_of[done:done + n]], axis=1)
        t0 = time.perf_counter()
        oracle.attention_rows(q, k, v, cq, ck, causal=w.causal, window=w.window, softcap=w.softcap,
                              scale=w.softmax_scale, rows=rows)
        elapsed += time.perf_counter() - t0
        pairs += int(cnt[rows[:, 0]].sum())
        done += n
        if elapsed >= target_s:
            break
        rate = done / max(elapsed, 1e-9)
        n = int(min(total_rows - done, max(256, rate * (target_s - elapsed))))
    flops = pairs * 2 * (w.d_qk + w.d_v)
    _, _, call_bytes = work_of(w, inp)
    return {
        "workload": name,
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "gflops": round(flops / elapsed / 1e9, 2),
        # algorithmic bytes of the sampled share of one call, per second
        "gbs": round(call_bytes * done / total_rows / elapsed / 1e9, 3),
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} of {total_rows} (token, head) rows of {name}, seeded random order; "
                  f"{pairs} visible pairs in {elapsed:.1f} s",
        "seconds": round(elapsed, 2),
        "cpu_model": _cpu_model(),
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def workload_names(spec):
    """The workloads a --workloads value runs, in the bench's order."""
    names = spec.split(",")
    if names == ["all"]:
        names = [PRIMARY, DECODE, "single_head_f32", "varlen_gqa_causal_bf16", "window_softcap_bf16",
                 "chunked_prefill_bf16", "paged_mla_decode_bf16", "gqa_decode_bf16", "mla_decode_fp8"]
    if PRIMARY not in names:
        names.insert(0, PRIMARY)
    return names


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # Long timed regions right after a long warmup: after any idle gap the
    # chip restarts at a lower shader clock and takes ~10-25 ms of continuous
    # load to reach its sustained one, which short regions would mostly miss.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed regions of --steps calls each; the figures are their median")
    ap.add_argument("--workloads", default=f"{PRIMARY},{DECODE}")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="GPU time of back-to-back calls before the warmup of each workload (sustained clock)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-probe-mb", type=int, default=0)
    ap.add_argument("--pmc-summarize", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--trace-summarize", metavar="KERNEL_TRACE_CSV",
                    help="print per-(kernel, grid) durations of a rocprofv3 --kernel-trace csv and exit")
    args = ap.parse_args()
    if args.trace_summarize:
        trace_summarize(args.trace_summarize, workload_names(args.workloads))
        return
    if args.pmc_summarize:
        if args.copy_probe_mb <= 0:
            raise SystemExit("--pmc-summarize needs --copy-probe-mb (the size of the calibration copy)")
        pmc_summarize(args.pmc_summarize[0], args.pmc_summarize[1], args.copy_probe_mb)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the library runs on one GPU; --gpus must be 1 "
              "(sharding across GPUs by (sequence, kv head) groups is designed but not implemented)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import tiled_attention_amd as mx

    mx.load_library()  # fails loudly when the HIP library is not built
    names = workload_names(args.workloads)

    results = {}
    for name in names:
        print(f"[bench] {name}: preparing inputs", file=sys.stderr, flush=True)
        r = Runner(name)
        settle_calls, settle_ms, clock = r.settle(args.settle_ms)
        reps = r.time(args.steps, args.warmup, max(1, args.repeats))
        ms = float(np.median(reps))
        res = {
            "workload": name,
            "settle_calls": settle_calls,
            "settle_ms": round(settle_ms, 1),
            "ms": round(ms, 4),
            "ms_mean": round(float(np.mean(reps)), 4),
            "ms_repeats": [round(x, 4) for x in reps],
            "clock": clock,
            "tflops": r.flops / (ms * 1e-3) / 1e12,
            "gbs": r.bytes / (ms * 1e-3) / 1e9,
            "flops_per_call": r.flops,
            "bytes_per_call": r.bytes,
            "kernel": r.kernel,
        }
        if r.w.kind in ("decode", "gqa_decode"):
            res["splits"] = r.splits
        results[name] = res
        clk = (res["clock"] or {}).get("mhz")
        print(f"[bench] {name}: {ms:.4f} ms/call (median of {len(reps)} x {args.steps}; mean {res['ms_mean']:.4f}), "
              f"{res['tflops']:.1f} TFLOP/s, {res['gbs']:.1f} GB/s, clock {clk} MHz", file=sys.stderr, flush=True)
        del r
        torch.cuda.empty_cache()

    if args.copy_probe_mb > 0:
        # Calibration copy for the traffic counters: reads and writes exactly
        # copy_probe_mb MiB (not part of the JSON line).
        src = torch.empty(args.copy_probe_mb * 2 ** 20, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy probe: {args.copy_probe_mb} MiB x 3", file=sys.stderr, flush=True)
        del src, dst

    p = results[PRIMARY]
    w = __import__("workloads").get(PRIMARY)
    line = {
        "metric": METRIC,
        "value": round(p["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": p["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), bf16 RNE)",
        "config": {"workload": PRIMARY, "batch": w.batch, "seqlen": w.seqlen_q, "heads_q": w.heads_q,
                   "heads_kv": w.heads_kv, "head_dim": w.d_qk, "causal": w.causal, "parallelism": "single GPU"},
        "roofline": {
            "bound": "mfma",
            "achieved": round(p["tflops"], 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(p["tflops"] / PEAK_BF16_TFLOPS, 4),
            "traffic": load_traffic(p["kernel"]),
            "kernel": p["kernel"],
            "flops_per_launch": p["flops_per_call"],
            "ms_median": p["ms"],
            "ms_mean": p["ms_mean"],
            "repeats": len(p["ms_repeats"]),
            **clock_fields(p, PEAK_BF16_TFLOPS),
        },
    }
    if DECODE in results:
        d = results[DECODE]
        line["decode"] = {
            "workload": DECODE,
            "value": round(d["gbs"], 1),
            "unit": "GB/s",
            "ms": d["ms"],
            "splits": d.get("splits"),
            "roofline": {"bound": "hbm", "achieved": round(d["gbs"], 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(d["gbs"] / PEAK_HBM_GBS, 4), "traffic": load_traffic("decode_mla"),
                         "bytes_per_launch": d["bytes_per_call"], "ms_median": d["ms"], "ms_mean": d["ms_mean"],
                         "repeats": len(d["ms_repeats"]), "clock_mhz": (d["clock"] or {}).get("mhz"),
                         "note": "one call = split kernel + combine kernel; the HBM peak does not scale "
                                 "with the shader clock"},
        }
    extra = [v for k, v in results.items() if k not in (PRIMARY, DECODE)]
    if extra:
        line["extra"] = extra
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline: fp64 oracle on a sample of the prefill workload", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(PRIMARY, args.cpu_seconds)
        # The same oracle on bounded samples of the other headline workloads
        # (reported only; the headline figure is the prefill's).
        others = []
        for name in ("single_head_f32", "varlen_gqa_causal_bf16", DECODE, "window_softcap_bf16"):
            print(f"[bench] cpu baseline: fp64 oracle on a sample of {name}", file=sys.stderr, flush=True)
            others.append(cpu_baseline(name, args.cpu_seconds / 2))
        line["cpu_baseline"]["others"] = others
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

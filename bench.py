#!/usr/bin/env python3
"""Bench: exact tiled attention forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3] [--no-cpu-baseline]
    python bench.py --workload decode     (split-KV decode forward, GB/s against the HBM roofline)
    python bench.py --workload window     (local-window forward, TFLOP/s on the visible pairs)
    python bench.py --workload sparse     (block-sparse forward, TFLOP/s on the visible pairs)

One step = one pass of the whole hot path over one batch of synthetic inputs already resident
in HBM: fa_fwd (O and LSE) then fa_bwd (its stages fa_bwd_prep, fa_bwd_dkdv, fa_bwd_dq), bf16 with
fp32 accumulation.  The default workload is causal attention at B=2, H=16, N=8192, d=128 — the
shape the headline metric is quoted on — with Q, K, V, dO drawn N(0,1)*0.5 from seed 3.

Printed: ONE JSON line with whole-job TFLOP/s (forward 4*N^2*d*B*H halved for causal, backward
2.5x that: five GEMM-shaped products instead of two), per-kernel HIP-event durations, the
roofline of the dominant kernel and the fp64 CPU oracle timed on a bounded sample on the host's
cores (a reported baseline, not a target).

Also: --copy-calib runs a plain device copy of known size, the reference point that scales the
rocprofv3 FETCH_SIZE / WRITE_SIZE counters into bytes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
_CSRC = "exact_io_aware_68_amd/csrc/"
KERNEL_SRC = {                 # kernel -> sources whose hash guards stored counter data
    "fwd_bf16": [_CSRC + "fa_fwd_bf16.hip", _CSRC + "fa_device.h"],
    "bwd_prep": [_CSRC + "fa_bwd_bf16.hip", _CSRC + "fa_device.h"],
    "bwd_dkdv": [_CSRC + "fa_bwd_bf16.hip", _CSRC + "fa_device.h"],
    "bwd_dq": [_CSRC + "fa_bwd_dq.hip", _CSRC + "fa_device.h"],
    "splitkv": [_CSRC + "fa_splitkv.hip", _CSRC + "fa_device.h"],
    "fwd_window": [_CSRC + "fa_fwd_bf16.hip", _CSRC + "fa_device.h"],
    "fwd_sparse": [_CSRC + "fa_fwd_bf16.hip", _CSRC + "fa_device.h"],
    "splitkv_merge": [_CSRC + "fa_splitkv.hip", _CSRC + "fa_device.h"],
}
# rocprofv3 kernel-name fragment -> kernel key
KERNEL_MATCH = [("bwd_prep", "bwd_prep"), ("bwd_dkdv", "bwd_dkdv"), ("bwd_dq", "bwd_dq"),
                ("fwd_window", "fwd_window"), ("fwd_sparse", "fwd_sparse"), ("fwd_bf16", "fwd_bf16"),
                ("splitkv_merge", "splitkv_merge"),
                ("splitkv_bf16", "splitkv")]
COPY_CALIB_BYTES = 1 << 30


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")


# ------------------------------------------------------------------ work and byte models

def fwd_flops(B, Hq, N, d, causal):
    """Matmul flops of the forward: 4 N^2 d per head (QK^T and PV), halved when causal."""
    f = 4.0 * N * N * d * B * Hq
    return f / 2 if causal else f


def bwd_flops(B, Hq, N, d, causal):
    """Backward: recompute S, then dV, dP, dK, dQ: five products of the forward's size."""
    return 2.5 * fwd_flops(B, Hq, N, d, causal)


def fwd_bytes_compulsory(B, Hq, Hkv, N, d, elem=2):
    """Tiled IO count of the forward: read Q, K, V once, write O and the fp32 LSE once."""
    return (2 * B * Hq * N * d + 2 * B * Hkv * N * d) * elem + B * Hq * N * 4


def bwd_bytes_compulsory(B, Hq, Hkv, N, d, elem=2):
    """Backward: read Q, K, V, O, dO (bf16), LSE; write+read the two per-row statistics; write
    fp32 dQ, dK, dV."""
    reads = (3 * B * Hq * N * d + 2 * B * Hkv * N * d) * elem + B * Hq * N * 4
    d_rw = 2 * 2 * B * Hq * N * 4
    writes = (B * Hq * N * d + 2 * B * Hkv * N * d) * 4
    return reads + d_rw + writes


def bwd_kernel_bytes_compulsory(B, Hq, Hkv, N, d, elem=2):
    """Per backward kernel: prep reads O, dO, LSE and writes D and the base-2 LSE; dK/dV reads
    Q, dO, K, V and both statistics and writes fp32 dK, dV; dQ reads the same and writes fp32 dQ."""
    q = B * Hq * N * d * elem
    kv = B * Hkv * N * d * elem
    rows = B * Hq * N * 4
    return {"bwd_prep": 2 * q + rows + 2 * rows,
            "bwd_dkdv": 2 * q + 2 * kv + 2 * rows + 2 * B * Hkv * N * d * 4,
            "bwd_dq": 2 * q + 2 * kv + 2 * rows + B * Hq * N * d * 4}


def decode_kernel_bytes_compulsory(w, key_lens, splits, elem=2):
    """Decode (split-KV): the range kernel reads the valid K and V rows once and Q, and writes
    each range's fp32 partial output and LSE; the merge reads those and writes O and LSE."""
    L = [w.Nk] * w.B if key_lens is None else [int(x) for x in key_lens.tolist()]
    kv = sum(2 * w.Hkv * l * w.d * elem for l in L)
    rows = w.B * w.Hq * w.Nq
    part = splits * rows * (w.d + 1) * 4
    return {"splitkv": kv + rows * w.d * elem + part,
            "splitkv_merge": part + rows * w.d * elem + rows * 4}


def window_pairs(N, left, right, key_lens=None, B=1):
    """Number of visible (query, key) pairs of a local window, summed over the batches."""
    import numpy as np
    i = np.arange(N)
    lo = np.maximum(i - left, 0) if left >= 0 else np.zeros(N, dtype=np.int64)
    tot = 0
    for b in range(B):
        L = N if key_lens is None else int(key_lens[b])
        hi = np.minimum(i + right, L - 1) if right >= 0 else np.full(N, L - 1)
        tot += int(np.maximum(hi - lo + 1, 0).sum())
    return tot


def sparse_pairs(N, bm, causal, bq=128, bk=64):
    """Visible (query, key) pairs of one head under a block bitmap (and causal), exactly."""
    import numpy as np
    bm = np.asarray(bm) != 0
    tot = 0
    for qb in range(bm.shape[0]):
        r0, r1 = qb * bq, min(N, (qb + 1) * bq)
        for kb in np.nonzero(bm[qb])[0]:
            k0, k1 = int(kb) * bk, min(N, (int(kb) + 1) * bk)
            if not causal:
                tot += int((r1 - r0) * (k1 - k0))
            else:
                rows = np.arange(r0, r1)
                tot += int(np.clip(rows - k0 + 1, 0, k1 - k0).sum())
    return tot


def naive_bytes(B, Hq, N, elem=2):
    """Naive attention's score traffic alone: write S, read S, write P, read P (elem bytes)."""
    return 4 * N * N * elem * B * Hq


def noreuse_tiled_bytes(B, Hq, N, d, Br=128, elem=2, causal=False):
    """Tiled attention with no on-chip reuse of K/V across query tiles: every q-tile re-reads
    the K and V it needs (half of them on average when causal), plus Q and O once."""
    ntiles = -(-N // Br)
    kv = 2 * N * d * elem * ntiles * (0.5 if causal else 1.0)
    return B * Hq * (kv + 2 * N * d * elem)


# ------------------------------------------------------------------ helpers

def _src_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(kernel, workload):
    """Measured HBM bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE) from the committed
    rocprofv3 counter summary of this workload, or None when absent or when the kernel's sources
    changed since the counters were taken."""
    try:
        lines = open(traffic_file(workload)).read().splitlines()
    except OSError:
        return None
    for ln in lines:
        cells = [c.strip() for c in ln.strip().strip("|").split("|")]
        if len(cells) >= 6 and cells[0] == kernel:
            if cells[1] != _src_hash(KERNEL_SRC[kernel]):
                return None
            try:
                return int(cells[5])
            except ValueError:
                return None
    return None


def _counter_means(path):
    """Mean Counter_Value per kernel key from a rocprofv3 counter_collection.csv."""
    import csv
    acc = {}
    for r in csv.DictReader(open(path)):
        name = r["Kernel_Name"]
        key = next((k for frag, k in KERNEL_MATCH if frag in name), None)
        if key is None and "copyBuffer" in name:
            key = "copy"
        if key is not None:
            acc.setdefault(key, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def traffic_summary(d, workload, cmd_note):
    """Write profiles/hbm_traffic_<workload>.md from four rocprofv3 --pmc runs in directory d:
    bench_FETCH_SIZE, bench_WRITE_SIZE (this bench) and copy_FETCH_SIZE, copy_WRITE_SIZE (the
    --copy-calib copy of COPY_CALIB_BYTES).  Each counter (KiB per dispatch) is scaled by
    known bytes / what the same counter reads for the copy."""
    f = {n: _counter_means(os.path.join(d, f"{n}_counter_collection.csv"))
         for n in ("bench_FETCH_SIZE", "bench_WRITE_SIZE", "copy_FETCH_SIZE", "copy_WRITE_SIZE")}
    kib = COPY_CALIB_BYTES / 1024
    fr = kib / f["copy_FETCH_SIZE"]["copy"]
    fw = kib / f["copy_WRITE_SIZE"]["copy"]
    import fa_inputs as fi
    if workload in fi.DECODE_WORKLOADS:
        w = fi.DECODE_WORKLOADS[workload]
        x = fi.make_decode(w)
        import exact_io_aware_68_amd as fa
        splits = fa.fa_fwd_splitkv_splits(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, 0)
        comp = decode_kernel_bytes_compulsory(w, x["key_lens"], splits)
        kernels = ("splitkv", "splitkv_merge")
        title = (f"B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} Nk={w.Nk} d={w.d} bf16, key lengths "
                 f"U[Nk/2, Nk], {splits} key ranges")
        comp_note = ("Compulsory bytes: the range kernel reads the valid K and V rows once and Q "
                     "and writes each range's fp32 partial output and LSE; the merge reads those "
                     "and writes O and LSE.")
    elif workload in fi.SPARSE_WORKLOADS:
        w, density = fi.SPARSE_WORKLOADS[workload]
        comp = {"fwd_sparse": fwd_bytes_compulsory(w.B, w.Hq, w.Hkv, w.N, w.d)}
        kernels = ("fwd_sparse",)
        title = (f"B={w.B} Hq={w.Hq} N={w.N} d={w.d} block bitmap band 2 + random {density} "
                 f"{w.dtype}")
        comp_note = ("`vs compulsory` divides by the tiled IO count (read Q, K, V once, write O "
                     "and LSE once).")
    elif workload in fi.WINDOW_WORKLOADS:
        w, window = fi.WINDOW_WORKLOADS[workload]
        comp = {"fwd_window": fwd_bytes_compulsory(w.B, w.Hq, w.Hkv, w.N, w.d)}
        kernels = ("fwd_window",)
        title = f"B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} local window {window} {w.dtype}"
        comp_note = ("`vs compulsory` divides by the tiled IO count (read Q, K, V once, write O "
                     "and LSE once).")
    else:
        w = fi.WORKLOADS[workload]
        comp = {"fwd_bf16": fwd_bytes_compulsory(w.B, w.Hq, w.Hkv, w.N, w.d),
                **bwd_kernel_bytes_compulsory(w.B, w.Hq, w.Hkv, w.N, w.d)}
        kernels = ("fwd_bf16", "bwd_prep", "bwd_dkdv", "bwd_dq")
        title = f"B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} causal={w.causal} {w.dtype}"
        comp_note = ("`vs compulsory` divides by the tiled IO count (read Q, K, V once, write O "
                     "and LSE once).  Compulsory bytes of the backward kernels: prep reads O, dO, "
                     "LSE and writes D and the base-2 LSE; dK/dV reads Q, dO, K, V and both row "
                     "statistics and writes fp32 dK, dV; dQ reads the same and writes fp32 dQ.")
    rows = []
    for k in kernels:
        if k not in f["bench_FETCH_SIZE"]:
            continue
        rd, wr = f["bench_FETCH_SIZE"][k], f["bench_WRITE_SIZE"][k]
        byt = int(round((rd * fr + wr * fw) * 1024))
        c = comp[k]
        rows.append(f"| {k} | {_src_hash(KERNEL_SRC[k])} | {rd:.0f} | {wr:.0f} | "
                    f"{(rd * fr + wr * fw) / 1024:.1f} | {byt} | "
                    f"{'-' if c is None else f'{byt / c:.3f}'} |")
    txt = f"""# HBM traffic per launch — workload {workload}: {title}

Counters from four `rocprofv3 --pmc` runs (one counter each), averaged over the dispatches of
each kernel:

{cmd_note}

Calibration: a plain device copy of {COPY_CALIB_BYTES} bytes (`bench.py --copy-calib`) reads
FETCH_SIZE = {f['copy_FETCH_SIZE']['copy']:.0f} KiB and WRITE_SIZE =
{f['copy_WRITE_SIZE']['copy']:.0f} KiB per dispatch, so FETCH_SIZE is scaled by {fr:.3f} and
WRITE_SIZE by {fw:.3f}.  `bytes/launch` = calibrated FETCH + WRITE.  `src` is the hash
bench.py compares with the kernel's current sources: a stale row reads as unmeasured.
{comp_note}

| kernel | src | FETCH_SIZE KiB | WRITE_SIZE KiB | calibrated MiB | bytes/launch | vs compulsory |
|---|---|---|---|---|---|---|
""" + "\n".join(rows) + "\n"
    open(traffic_file(workload), "w").write(txt)
    print(txt)


# MI355X (gfx950): 8 XCDs x 4 shader engines, 256 CUs, 4 SIMDs per CU.
N_SE, N_CU, N_SIMD = 32, 256, 1024


def _kernel_key(name):
    key = next((k for frag, k in KERNEL_MATCH if frag in name), None)
    if key is None and "copyBuffer" in name:
        key = "copy"
    return key


def _trace_durations(path):
    """{dispatch id: (kernel key, duration ns, start ns)} from a rocprofv3 kernel_trace.csv."""
    import csv
    out = {}
    for r in csv.DictReader(open(path)):
        key = _kernel_key(r["Kernel_Name"])
        if key is not None:
            s0, s1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            out[r["Dispatch_Id"]] = (key, s1 - s0, s0)
    return out


def _dispatch_counters(path):
    """{dispatch id: (kernel key, {counter: value})} from a rocprofv3 counter_collection.csv
    (values of one counter within a dispatch summed)."""
    import csv
    out = {}
    for r in csv.DictReader(open(path)):
        key = _kernel_key(r["Kernel_Name"])
        if key is None:
            continue
        _, c = out.setdefault(r["Dispatch_Id"], (key, {}))
        c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def trace_summary(d, workload, steps, cmd_note):
    """Write profiles/kernels_<workload>.md from a rocprofv3 --kernel-trace run in directory d
    (run_kernel_trace.csv): per kernel the calls, average, min and max duration over every
    dispatch and the average over the last `steps` (the bench's timed steps), next to the
    HIP-event averages the traced bench printed (d/bench.json, if present)."""
    import statistics
    tr = sorted(_trace_durations(os.path.join(d, "run_kernel_trace.csv")).values(),
                key=lambda t: t[2])
    by = {}
    for key, dur, _ in tr:
        by.setdefault(key, []).append(dur / 1e3)
    live = None
    try:
        live = json.loads(open(os.path.join(d, "bench.json")).read().strip().splitlines()[-1])
    except (OSError, ValueError, IndexError):
        pass
    rows = []
    for key, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        last = v[-steps:]
        rows.append(f"| {key} | {len(v)} | {statistics.mean(v):.1f} | {min(v):.1f} | {max(v):.1f} "
                    f"| {statistics.mean(last):.1f} |")
    live_txt = ""
    if live:
        km = live.get("kernels_ms") or {}
        live_txt = ("\nLive HIP-event averages printed by the traced bench (timed steps): " +
                    ", ".join(f"{k} {v * 1e3:.1f} µs" for k, v in km.items()) + ".\n")
        if live.get("roofline"):
            r = live["roofline"]
            live_txt += (f"Its roofline line: kernel {r.get('kernel')}, achieved {r.get('achieved')} "
                         f"{r.get('unit')} of {r.get('peak')} (frac {r.get('frac')}).\n")
    txt = f"""# Kernel durations — workload {workload}

Command (from the repository root on the MI355X box; $REPO is the repository):

{cmd_note}

`run_kernel_trace.csv`, every dispatch of each kernel, and the average over the last {steps}
dispatches (the bench's timed steps; the warm-up dispatches come first):

| Kernel | Calls | Average, all (µs) | Min (µs) | Max (µs) | Average, last {steps} (µs) |
|---|---|---|---|---|---|
""" + "\n".join(rows) + "\n" + live_txt
    open(os.path.join(ROOT, "profiles", f"kernels_{workload}.md"), "w").write(txt)
    print(txt)


SQ_PASSES = {   # rocprofv3 --pmc passes of at most 8 SQ counters (and GRBM in the last)
    "p1": "SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS "
          "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_TRANS_F32",
    "p2": "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_ANY SQ_WAIT_INST_LDS SQ_WAIT_ANY "
          "SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_VMEM SQ_WAIT_INST_ANY",
    "p3": "SQ_LDS_DATA_FIFO_FULL SQ_LDS_ADDR_CONFLICT SQ_INSTS_SALU SQ_INSTS_VMEM_RD "
          "SQ_INSTS_VMEM_WR SQ_VALU_MFMA_COEXEC_CYCLES SQ_BUSY_CU_CYCLES SQ_INSTS_BRANCH",
    "p4": "SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS_LOAD_BANDWIDTH GRBM_GUI_ACTIVE",
}


def sq_summary(d, workload, cmd_note):
    """Write profiles/sq_counters_<workload>.md from the four --pmc passes (with --kernel-trace) in
    directory d: per kernel the mean of each counter over its dispatches, and derived rates.  The
    shader clock of a dispatch is SQ_BUSY_CYCLES / N_SE over the dispatch's own duration."""
    import statistics
    counters, dur = {}, {}
    for ps in SQ_PASSES:
        c = _dispatch_counters(os.path.join(d, f"{ps}_counter_collection.csv"))
        t = _trace_durations(os.path.join(d, f"{ps}_kernel_trace.csv"))
        for did, (key, vals) in c.items():
            for name, v in vals.items():
                counters.setdefault(key, {}).setdefault(name, []).append(v)
            if ps == "p1" and did in t and "SQ_BUSY_CYCLES" in vals:
                dur.setdefault(key, []).append((t[did][1], vals["SQ_BUSY_CYCLES"]))
            if ps == "p4" and did in t and "GRBM_GUI_ACTIVE" in vals:
                dur.setdefault(key + "#grbm", []).append((t[did][1], vals["GRBM_GUI_ACTIVE"]))
    kernels = [k for k in ("fwd_bf16", "bwd_prep", "bwd_dkdv", "bwd_dq", "fwd_window", "fwd_sparse",
                           "splitkv", "splitkv_merge") if k in counters]
    names = [n for ps in SQ_PASSES.values() for n in ps.split()]
    mean = {k: {n: statistics.mean(counters[k][n]) for n in names if n in counters[k]}
            for k in kernels}
    lines = ["| Counter | " + " | ".join(kernels) + " |", "|---" * (len(kernels) + 1) + "|"]
    for n in names:
        lines.append(f"| {n} | " + " | ".join(f"{mean[k][n]:,.0f}" if n in mean[k] else "-"
                                             for k in kernels) + " |")

    def derived(k):
        m = mean[k]
        cyc = m.get("SQ_BUSY_CYCLES", 0.0) / N_SE          # cycles of the dispatch per engine
        mf = m.get("SQ_INSTS_MFMA", 0.0)
        ghz = [b / N_SE / ns for ns, b in dur.get(k, []) if ns > 0]
        grbm = [g / 8 / ns for ns, g in dur.get(k + "#grbm", []) if ns > 0]
        wc = m.get("SQ_WAVE_CYCLES", 0.0) or 1.0
        out = {
            "duration (µs, counter run)": statistics.mean(ns for ns, _ in dur[k]) / 1e3 if dur.get(k) else None,
            "shader clock, SQ_BUSY_CYCLES / 32 per duration (GHz)": statistics.mean(ghz) if ghz else None,
            "GRBM_GUI_ACTIVE / 8 per duration (GHz)": statistics.mean(grbm) if grbm else None,
            "MFMA busy (of SIMD-cycles)": m.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (cyc * N_SIMD) if cyc else None,
            "MFMA and VALU co-executing (of MFMA busy)":
                m.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0.0) / m["SQ_VALU_MFMA_BUSY_CYCLES"]
                if m.get("SQ_VALU_MFMA_BUSY_CYCLES") else None,
            "VALU instructions per MFMA (excl. MFMA)": (m.get("SQ_INSTS_VALU", 0.0) - mf) / mf if mf else None,
            "LDS instructions per MFMA": m.get("SQ_INSTS_LDS", 0.0) / mf if mf else None,
            "LDS busy (SQ_LDS_IDX_ACTIVE / CU-cycles)": m.get("SQ_LDS_IDX_ACTIVE", 0.0) / (cyc * N_CU) if cyc else None,
            "wave time executing": m.get("SQ_ACTIVE_INST_ANY", 0.0) / wc,
            "wave time waiting": m.get("SQ_WAIT_ANY", 0.0) / wc,
            "wave time waiting to issue": m.get("SQ_WAIT_INST_ANY", 0.0) / wc,
        }
        return out

    der = {k: derived(k) for k in kernels}
    dl = ["| Metric | " + " | ".join(kernels) + " |", "|---" * (len(kernels) + 1) + "|"]
    for name in der[kernels[0]]:
        cells = []
        for k in kernels:
            v = der[k][name]
            if v is None:
                cells.append("-")
            elif "GHz" in name or "per MFMA" in name:
                cells.append(f"{v:.2f}")
            elif "µs" in name:
                cells.append(f"{v:.1f}")
            else:
                cells.append(f"{100 * v:.1f} %")
        dl.append(f"| {name} | " + " | ".join(cells) + " |")
    txt = f"""# Instruction and stall counters — workload {workload}

Four `rocprofv3 --pmc` passes (each with `--kernel-trace`, so that every dispatch's counters sit
beside its own duration), one counter group each, means over each kernel's dispatches; run from
/tmp with TMPDIR=/tmp ($REPO is the repository):

{cmd_note}

Counters: SQ_INSTS_VALU includes the MFMAs; ACTIVE / WAIT / WAVE cycle counters are summed over
waves; SQ_BUSY_CYCLES is summed over the {N_SE} shader engines, SQ_VALU_MFMA_BUSY_CYCLES over
the {N_SIMD} SIMDs and SQ_LDS_IDX_ACTIVE over the {N_CU} CUs.  One v_mfma_f32_32x32x16_bf16 keeps
a SIMD's matrix unit busy for 32 cycles.

""" + "\n".join(lines) + "\n\nDerived, per kernel:\n\n" + "\n".join(dl) + "\n"
    open(os.path.join(ROOT, "profiles", f"sq_counters_{workload}.md"), "w").write(txt)
    print(txt)


def cpu_baseline(x, w, budget_s=20.0):
    """Time the fp64 oracle (as written, untuned) forward + backward on whole heads of the same
    workload, as many as fit the time budget (at least one)."""
    from threadpoolctl import threadpool_info

    from oracle import attn_bwd, attn_fwd
    heads = []
    t0 = time.perf_counter()
    g = w.Hq // w.Hkv
    for b in range(w.B):
        for hkv in range(w.Hkv):
            sl = slice(hkv * g, (hkv + 1) * g)
            q, k, v, do = (x[n][b:b + 1, s] for n, s in
                           (("q", sl), ("k", slice(hkv, hkv + 1)), ("v", slice(hkv, hkv + 1)),
                            ("do", sl)))
            attn_fwd(q, k, v, x["scale"], w.causal)
            attn_bwd(q, k, v, do, x["scale"], w.causal)
            heads.append((b, hkv))
            if time.perf_counter() - t0 > budget_s / 2:
                break
        if time.perf_counter() - t0 > budget_s / 2:
            break
    dt = time.perf_counter() - t0
    nq = len(heads) * g
    flops = fwd_flops(1, nq, w.N, w.d, w.causal) + bwd_flops(1, nq, w.N, w.d, w.causal)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"fp64 numpy oracle fwd+bwd on {nq} of {w.B * w.Hq} heads "
                      f"(N={w.N}, d={w.d}, causal={w.causal}) in {dt:.1f} s; "
                      f"host affinity {len(os.sched_getaffinity(0))} cpus"}


def copy_calibration(nbytes=1 << 30, reps=5):
    """A plain device copy of known size for counter calibration (reads and writes nbytes)."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}))


# ------------------------------------------------------------------ main

# The counter recipe written into the summary ($REPO: the repository, $OUT: any writable
# directory for the counter CSVs).
TRAFFIC_CMD = """    cd /tmp && export TMPDIR=/tmp
    for C in FETCH_SIZE WRITE_SIZE; do
      rocprofv3 --pmc $C -T -f csv -d $OUT/pmc -o bench_$C -- \\
          python3 $REPO/bench.py --steps 2 --warmup 1 --no-cpu-baseline --cold-steps 0 --no-other-configs
      rocprofv3 --pmc $C -T -f csv -d $OUT/pmc -o copy_$C -- \\
          python3 $REPO/bench.py --copy-calib
    done
    python3 $REPO/bench.py --traffic-summary $OUT/pmc"""

def causal_pairs(N, L):
    """Visible (query, key) pairs of one causal head whose keys stop at L: row i sees
    min(i + 1, L) keys."""
    L = min(L, N)
    return L * (L + 1) // 2 + (N - L) * L


def time_launches(fn, reps=10, warmup=3):
    """Mean duration (ms) of fn's launches, HIP events on the current stream around each."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / len(evs)


def other_configs(reps=10):
    """The other bf16 workloads, each timed on its own (after the timed steps, outside them):
    c2 and c4 forwards, c5 forward and backward (prep + dK/dV + dQ).  c4's work is given both by
    the formula (4 N^2 d B H / 2, counting keys past each key length) and on the visible pairs."""
    import torch

    import exact_io_aware_68_amd as fa
    import fa_inputs as fi
    dev = "cuda:0"
    res = {}
    for name in ("c2", "c4", "c5"):
        w = fi.WORKLOADS[name]
        x = fi.make(w, want_do=name == "c5")
        q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
        kl = None if x["key_lens"] is None else x["key_lens"].to(dev)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
        sc = x["scale"]

        def fwd():
            fa.fa_fwd(q, k, v, scale=sc, causal=w.causal, key_lens=kl, o=o, lse=lse)

        ms = time_launches(fwd, reps)
        ff = fwd_flops(w.B, w.Hq, w.N, w.d, w.causal)
        r = {"workload": f"B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} causal={w.causal} "
                         f"key_lens={x['key_lens'].tolist() if w.padded else 'none'}",
             "fwd_ms": round(ms, 4), "fwd_flops": ff,
             "fwd_tflops": round(ff / (ms * 1e-3) / 1e12, 2),
             "fwd_pct_peak": round(100 * ff / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}
        if w.padded:
            pairs = sum(causal_pairs(w.N, int(L)) for L in x["key_lens"].tolist()) * w.Hq
            fv = 4.0 * w.d * pairs
            r.update(fwd_flops_visible_pairs=fv,
                     fwd_tflops_visible_pairs=round(fv / (ms * 1e-3) / 1e12, 2))
        if name == "c5":
            fa.fa_fwd(q, k, v, scale=sc, causal=w.causal, key_lens=kl, o=o, lse=lse)
            do = x["do"].to(dev)
            dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
            dk = torch.empty(k.shape, dtype=torch.float32, device=dev)
            dv = torch.empty(v.shape, dtype=torch.float32, device=dev)
            ws = torch.empty(fa.fa_bwd_workspace_size(w.B, w.Hq, w.N), dtype=torch.uint8,
                             device=dev)

            def bwd():
                fa.fa_bwd(q, k, v, o, do, lse, scale=sc, causal=w.causal, key_lens=kl, dq=dq,
                          dk=dk, dv=dv, workspace=ws)

            bms = time_launches(bwd, reps)
            bf = bwd_flops(w.B, w.Hq, w.N, w.d, w.causal)
            r.update(bwd_ms=round(bms, 4), bwd_flops=bf,
                     bwd_tflops=round(bf / (bms * 1e-3) / 1e12, 2),
                     bwd_pct_peak=round(100 * bf / (bms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2))
        res[name] = r
        del x, q, k, v, o, lse
        torch.cuda.empty_cache()
    return res


def bench_decode(args):
    """Split-KV decode forward on a decode workload: one step = one fa_fwd_splitkv call (the range
    kernel and the merge kernel) with inputs resident in HBM.  Bound by HBM: reports GB/s of the
    algorithmic bytes against the 8 TB/s peak."""
    import torch

    import exact_io_aware_68_amd as fa
    import fa_inputs as fi
    w = fi.DECODE_WORKLOADS[args.workload]
    x = fi.make_decode(w)
    dev = "cuda:0"
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    kl = None if x["key_lens"] is None else x["key_lens"].to(dev)
    splits = fa.fa_fwd_splitkv_splits(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, args.splits)
    ws = torch.empty(fa.fa_fwd_splitkv_workspace_size(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, splits),
                     dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    # The K/V cache (185 MB here) would fit the 256 MB Infinity Cache; a decode step in service
    # reads it cold, so a 512 MiB buffer is READ before every timed call (outside the events):
    # reading evicts the caches without leaving dirty lines whose write-back would compete with
    # the timed reads.
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)

    def call():
        fa.fa_fwd_splitkv(q, k, v, scale=x["scale"], key_lens=kl, num_splits=splits, o=o, lse=lse,
                          workspace=ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    evs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        torch.sum(flush, dim=0, out=sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
    comp = decode_kernel_bytes_compulsory(w, x["key_lens"], splits)
    byt = comp["splitkv"] + comp["splitkv_merge"]
    gbs = byt / (ms * 1e-3) / 1e9
    meas = [stored_traffic(n, args.workload) for n in ("splitkv", "splitkv_merge")]
    out = {
        "metric": "split-KV decode attention GB/s (algorithmic bytes), HBM roofline",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "wall_ms_per_step_with_cache_flush": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"split-KV decode B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} "
                               f"Nk={w.Nk} d={w.d} key_lens=U[Nk/2,Nk] splits={splits}",
                   "seed": w.seed, "parallelism": "single GPU"},
        "kernels_ms": {"splitkv+merge": round(ms, 4)},
        "algorithmic_bytes": byt,
        "roofline": {"kernel": "splitkv+merge", "bound": "hbm", "achieved": round(gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": None if None in meas else sum(meas)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info

        from oracle import attn_decode
        t1 = time.perf_counter()
        attn_decode(x["q"], x["k"], x["v"], x["scale"], x["key_lens"])
        dt = time.perf_counter() - t1
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        out["cpu_baseline"] = {"value": round(byt / dt / 1e9, 3), "unit": "GB/s",
                               "cores": int(threads), "kind": "oracle",
                               "sample": f"fp64 numpy oracle over the whole workload in {dt:.2f} s "
                                         f"(same byte count); host affinity "
                                         f"{len(os.sched_getaffinity(0))} cpus"}
    print(json.dumps(out), flush=True)


def bench_window(args):
    """Local-window forward on a windowed workload: one step = one fa_fwd_window call.  Work is
    counted on the visible pairs only (4 d flops per pair per head: Q K^T and P V), so TFLOP/s
    compare directly with the full forward's; the % of peak is against the bf16 MFMA peak."""
    import torch

    import exact_io_aware_68_amd as fa
    import fa_inputs as fi
    w, window = fi.WINDOW_WORKLOADS[args.workload]
    x = fi.make(w)
    dev = "cuda:0"
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def call():
        fa.fa_fwd_window(q, k, v, window=window, scale=x["scale"], o=o, lse=lse)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    evs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
    pairs = window_pairs(w.N, window[0], window[1]) * w.B
    flops = 4.0 * w.d * pairs * w.Hq
    tf = flops / (ms * 1e-3) / 1e12
    out = {
        "metric": "local-window attention forward TFLOP/s on visible pairs + % bf16 MFMA peak",
        "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"local window (left, right)={window}, B={w.B} H={w.Hq} N={w.N} "
                               f"d={w.d}", "seed": w.seed, "parallelism": "single GPU"},
        "visible_pairs_per_head": pairs // w.B, "flops": flops,
        "full_attention_flops": fwd_flops(w.B, w.Hq, w.N, w.d, False),
        "kernels_ms": {"fwd_window": round(ms, 4)},
        "roofline": {"kernel": "fwd_window", "bound": "mfma", "achieved": round(tf, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": stored_traffic("fwd_window", args.workload)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info

        from oracle import attn_fwd
        t1 = time.perf_counter()
        attn_fwd(x["q"][:1, :1], x["k"][:1, :1], x["v"][:1, :1], x["scale"], False, window=window)
        dt = time.perf_counter() - t1
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        out["cpu_baseline"] = {"value": round(4.0 * w.d * (pairs // w.B) / dt / 1e12, 5),
                               "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
                               "sample": f"fp64 numpy oracle on 1 of {w.B * w.Hq} heads in "
                                         f"{dt:.2f} s (visible-pair flops; the oracle forms full "
                                         f"score rows); host affinity "
                                         f"{len(os.sched_getaffinity(0))} cpus"}
    print(json.dumps(out), flush=True)


def bench_sparse(args):
    """Block-sparse forward on a sparse workload: one step = one fa_fwd_blocksparse call.  Work is
    counted on the visible pairs of the bitmap (4 d flops per pair per head)."""
    import torch

    import exact_io_aware_68_amd as fa
    import fa_inputs as fi
    w, density = fi.SPARSE_WORKLOADS[args.workload]
    x = fi.make(w)
    bm_cpu = fi.block_bitmap(w.N, density, w.seed)
    dev = "cuda:0"
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    bm = bm_cpu.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def call():
        fa.fa_fwd_blocksparse(q, k, v, bm, scale=x["scale"], causal=w.causal, o=o, lse=lse)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    evs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
    pairs = sparse_pairs(w.N, bm_cpu.numpy(), w.causal)
    flops = 4.0 * w.d * pairs * w.B * w.Hq
    tf = flops / (ms * 1e-3) / 1e12
    out = {
        "metric": "block-sparse attention forward TFLOP/s on visible pairs + % bf16 MFMA peak",
        "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"block-sparse bitmap (128x64 blocks, band 2 + random {density}) "
                               f"B={w.B} H={w.Hq} N={w.N} d={w.d} causal={w.causal}",
                   "seed": w.seed, "parallelism": "single GPU"},
        "active_blocks": int(bm_cpu.sum()), "blocks": int(bm_cpu.numel()),
        "visible_pairs_per_head": pairs, "flops": flops,
        "full_attention_flops": fwd_flops(w.B, w.Hq, w.N, w.d, w.causal),
        "kernels_ms": {"fwd_sparse": round(ms, 4)},
        "roofline": {"kernel": "fwd_sparse", "bound": "mfma", "achieved": round(tf, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": stored_traffic("fwd_sparse", args.workload)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info

        from oracle import attn_fwd
        t1 = time.perf_counter()
        attn_fwd(x["q"][:1, :1], x["k"][:1, :1], x["v"][:1, :1], x["scale"], w.causal,
                 block_mask=(bm_cpu.numpy(), 128, 64))
        dt = time.perf_counter() - t1
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        out["cpu_baseline"] = {"value": round(4.0 * w.d * pairs / dt / 1e12, 5),
                               "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
                               "sample": f"fp64 numpy oracle on 1 of {w.B * w.Hq} heads in "
                                         f"{dt:.2f} s (visible-pair flops; the oracle forms full "
                                         f"score rows); host affinity "
                                         f"{len(os.sched_getaffinity(0))} cpus"}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c3")
    ap.add_argument("--only", choices=["fwd", "bwd", "both"], default="both")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=3,
                    help="steps timed kernel by kernel after a 512 MiB cache-evicting read "
                         "(reported as kernels_ms_cold_cache; 0 for profiling runs)")
    ap.add_argument("--flush-mib", type=int, default=512, help=argparse.SUPPRESS)
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the event-timed launches of the other workloads (c2, c4, c5)")
    ap.add_argument("--splits", type=int, default=0,
                    help="decode workloads: number of key ranges (0: the library's choice)")
    ap.add_argument("--copy-calib", action="store_true")
    ap.add_argument("--traffic-summary", metavar="DIR",
                    help="write profiles/hbm_traffic_<workload>.md from rocprofv3 --pmc CSVs")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="write profiles/kernels_<workload>.md from a rocprofv3 kernel trace")
    ap.add_argument("--sq-summary", metavar="DIR",
                    help="write profiles/sq_counters_<workload>.md from rocprofv3 --pmc passes")
    args = ap.parse_args()
    if args.traffic_summary:
        cmd = TRAFFIC_CMD
        if args.workload != "c3":
            W = args.workload
            cmd = (f"    cd /tmp && export TMPDIR=/tmp\n"
                   f"    for C in FETCH_SIZE WRITE_SIZE; do\n"
                   f"      rocprofv3 --pmc $C -T -f csv -d $OUT/pmcd_{W} -o bench_$C -- \\\n"
                   f"          python3 $REPO/bench.py --workload {W} --steps 2 --warmup 1 --no-cpu-baseline\n"
                   f"    done\n"
                   f"    cp $OUT/pmc/copy_* $OUT/pmcd_{W}/   # the copy calibration runs of the c3 summary\n"
                   f"    python3 $REPO/bench.py --workload {W} --traffic-summary $OUT/pmcd_{W}")
        traffic_summary(args.traffic_summary, args.workload, cmd)
        return
    if args.trace_summary:
        wl = "" if args.workload == "c3" else f" --workload {args.workload}"
        extra = " --cold-steps 0 --no-other-configs" if args.workload in ("c1", "c2", "c3", "c4", "c5") else ""
        cmd = (f"    cd /tmp && export TMPDIR=/tmp\n"
               f"    rocprofv3 --kernel-trace --stats -T -f csv -d $OUT/trace_{args.workload} -o run -- \\\n"
               f"        python3 $REPO/bench.py{wl} --steps {args.steps} --warmup {args.warmup} "
               f"--no-cpu-baseline{extra} > $OUT/trace_{args.workload}/bench.json\n"
               f"    python3 $REPO/bench.py{wl} --steps {args.steps} --warmup {args.warmup} "
               f"--trace-summary $OUT/trace_{args.workload}")
        trace_summary(args.trace_summary, args.workload, args.steps, cmd)
        return
    if args.sq_summary:
        wl = "" if args.workload == "c3" else f" --workload {args.workload}"
        cmd = "\n".join(
            f"    timeout -s KILL 60 rocprofv3 --pmc {c} --kernel-trace -T -f csv -d $OUT/sq_{args.workload} "
            f"-o {ps} -- \\\n        python3 $REPO/bench.py{wl} --steps 2 --warmup 1 --no-cpu-baseline "
            f"--cold-steps 0 --no-other-configs" for ps, c in SQ_PASSES.items())
        cmd += f"\n    python3 $REPO/bench.py{wl} --sq-summary $OUT/sq_{args.workload}"
        sq_summary(args.sq_summary, args.workload, cmd)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the attention path is "
              "built and measured on a single MI355X", file=sys.stderr)
        sys.exit(2)
    if args.copy_calib:
        copy_calibration()
        return
    import fa_inputs as fi
    if args.workload in fi.DECODE_WORKLOADS:
        bench_decode(args)
        return
    if args.workload in fi.WINDOW_WORKLOADS:
        bench_window(args)
        return
    if args.workload in fi.SPARSE_WORKLOADS:
        bench_sparse(args)
        return

    import torch

    import exact_io_aware_68_amd as fa
    import fa_inputs as fi

    w = fi.WORKLOADS[args.workload]
    x = fi.make(w, want_do=True)
    dev = "cuda:0"
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    kl = None if x["key_lens"] is None else x["key_lens"].to(dev)
    sc, causal = x["scale"], w.causal
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
    dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
    dk = torch.empty(k.shape, dtype=torch.float32, device=dev)
    dv = torch.empty(v.shape, dtype=torch.float32, device=dev)
    ws = torch.empty(fa.fa_bwd_workspace_size(w.B, w.Hq, w.N), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    do_fwd = args.only in ("fwd", "both")
    do_bwd = args.only in ("bwd", "both")
    if do_bwd and not do_fwd:
        fa.fa_fwd(q, k, v, scale=sc, causal=causal, key_lens=kl, o=o, lse=lse)

    names = (["fwd_bf16"] if do_fwd else []) + (["bwd_prep", "bwd_dkdv", "bwd_dq"] if do_bwd else [])
    ev = {n: [] for n in names}

    fns = {"fwd_bf16": lambda: fa.fa_fwd(q, k, v, scale=sc, causal=causal, key_lens=kl, o=o, lse=lse),
           "bwd_prep": lambda: fa.fa_bwd_prep(o, do, lse, ws),
           "bwd_dkdv": lambda: fa.fa_bwd_dkdv(q, k, v, do, dk, dv, ws, scale=sc, causal=causal,
                                              key_lens=kl),
           "bwd_dq": lambda: fa.fa_bwd_dq(q, k, v, do, dq, ws, scale=sc, causal=causal, key_lens=kl)}

    def step(record, flush=None, store=None):
        if flush is not None:
            # a spin of a few ms first, so that the host has queued the whole step (flushes,
            # events, kernels) before the GPU reaches it: no launch gap inside an event pair
            torch.cuda._sleep(5_000_000)
        for n in names:
            if flush is not None:   # evict L2 and the Infinity Cache, outside the events
                torch.sum(flush[0], dim=0, out=flush[1])
            if record:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fns[n]()
                e1.record(stream)
                (ev if store is None else store)[n].append((e0, e1))
            else:
                fns[n]()

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    kern_ms = {n: sum(a.elapsed_time(b) for a, b in ev[n]) / len(ev[n]) for n in names}
    # Per-kernel times with cold caches: each launch follows a 512 MiB read that evicts L2 and
    # the Infinity Cache (after the timed steps, with the clocks already up; profiling runs pass
    # --cold-steps 0, so their last dispatches are the timed steps).
    cold = {n: [] for n in names}
    if args.cold_steps > 0:
        fl = (torch.ones(args.flush_mib << 18, dtype=torch.float32, device=dev),
              torch.empty((), dtype=torch.float32, device=dev))
        for _ in range(args.cold_steps):
            step(True, flush=fl, store=cold)
        torch.cuda.synchronize()
        del fl

    ff = fwd_flops(w.B, w.Hq, w.N, w.d, causal) if do_fwd else 0.0
    bf = bwd_flops(w.B, w.Hq, w.N, w.d, causal) if do_bwd else 0.0
    value = (ff + bf) / (ms_step * 1e-3) / 1e12
    # Per-kernel executed products (each the size of one forward product, ff / 2): dK/dV
    # recomputes S and dP and forms dV, dK (4); dQ recomputes S and dP and forms dQ (3).  The
    # step's value counts the method's 5 backward products only.
    flops_of = {"fwd_bf16": ff, "bwd_prep": 0.0,
                "bwd_dkdv": 2.0 * ff if do_bwd else 0.0, "bwd_dq": 1.5 * ff if do_bwd else 0.0}
    if do_bwd and not do_fwd:
        f1 = fwd_flops(w.B, w.Hq, w.N, w.d, causal)
        flops_of.update(bwd_dkdv=2.0 * f1, bwd_dq=1.5 * f1)
    # dominant kernel: the one with the most time per step
    dom = max(names, key=lambda n: kern_ms[n])
    tr = stored_traffic(dom, args.workload)
    if dom == "bwd_prep":
        byt = bwd_bytes_compulsory(w.B, w.Hq, w.Hkv, w.N, w.d)
        ach = byt / (kern_ms[dom] * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": ach / PEAK_HBM_GBS, "traffic": tr}
    else:
        ach = flops_of[dom] / (kern_ms[dom] * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": tr}
    out = {
        "metric": "attention fwd/bwd TFLOP/s + % bf16 MFMA peak, N=8192 d=128 causal",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"exact attention {args.only}, B={w.B} Hq={w.Hq} Hkv={w.Hkv} "
                               f"N={w.N} d={w.d} causal={causal} "
                               f"key_lens={'U[N/2,N]' if w.padded else 'none'}",
                   "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d, "causal": causal,
                   "seed": w.seed, "parallelism": "single GPU"},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "kernels_ms": {n: round(t, 4) for n, t in kern_ms.items()},
        "kernels_ms_median": {n: round(sorted(a.elapsed_time(b) for a, b in ev[n])[len(ev[n]) // 2], 4)
                              for n in names},
        "kernels_ms_cold_cache": None if args.cold_steps <= 0 else {
            n: round(sum(a.elapsed_time(b) for a, b in cold[n]) / len(cold[n]), 4) for n in names},
        "fwd": None if not do_fwd else {
            "tflops": round(ff / (kern_ms["fwd_bf16"] * 1e-3) / 1e12, 2),
            "pct_peak": round(100 * ff / (kern_ms["fwd_bf16"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "instance": fa.fa_fwd_kernel_name(w.d, causal, kl is not None, fa.FA_BF16),
            "compulsory_bytes": fwd_bytes_compulsory(w.B, w.Hq, w.Hkv, w.N, w.d),
            "naive_score_bytes": naive_bytes(w.B, w.Hq, w.N),
            "noreuse_tiled_bytes": noreuse_tiled_bytes(w.B, w.Hq, w.N, w.d, causal=causal),
            "measured_bytes": stored_traffic("fwd_bf16", args.workload)},
        "bwd": None if not do_bwd else {
            "tflops": round(bf / (sum(kern_ms[n] for n in ("bwd_prep", "bwd_dkdv", "bwd_dq"))
                                  * 1e-3) / 1e12, 2),
            "dkdv_executed_tflops": round(flops_of["bwd_dkdv"] / (kern_ms["bwd_dkdv"] * 1e-3) / 1e12, 2),
            "dq_executed_tflops": round(flops_of["bwd_dq"] / (kern_ms["bwd_dq"] * 1e-3) / 1e12, 2),
            "instance": [fa.fa_bwd_dkdv_kernel_name(w.d, causal, kl is not None, fa.FA_BF16),
                         fa.fa_bwd_dq_kernel_name(w.d, causal, kl is not None, fa.FA_BF16)],
            "compulsory_bytes": bwd_bytes_compulsory(w.B, w.Hq, w.Hkv, w.N, w.d),
            "measured_bytes": {n: stored_traffic(n, args.workload)
                               for n in ("bwd_prep", "bwd_dkdv", "bwd_dq")}},
        "roofline": roof,
        "other_configs": None,
        "cpu_baseline": None,
    }
    if args.workload == "c3" and not args.no_other_configs:
        del q, k, v, do, o, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()
        out["other_configs"] = other_configs()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

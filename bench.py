#!/usr/bin/env python3
"""Benchmark of the speculative-decoding verify step on one MI355X.

One step = spec_verify_attn (one attention layer) + spec_reject_sample +
spec_commit_lengths over one batch of the 8B-shaped workload (B=64, k=3,
Hq=32, Hkv=8, D=128, contexts U[1024, 8192] in 16-token pages, vocab 128256,
T=1). Inputs are seeded synthetic arrays resident in HBM before timing; the
committed lengths are restored before every step so each step does the same
work. Prints one JSON line:

  value     verified tokens/s = sum_b (a_b + 1) per step / wall time per step
  roofline  the dominant call (verify attention): algorithmic bytes / its
            average duration from HIP events on the launch stream, vs 8 TB/s
  cpu_baseline  the fp64 oracle on this host's cores, on a bounded sample

Also in that line, `cold_cache`: per-call HIP-event times of the same step with
a 512 MiB write between steps, so that no logits or cache lines are left in
the L2 or the 256 MiB MALL (the flush is outside the timed calls).

Other modes:
  --variant plain              k = 0 on the same workload: plain decoding
  --variant ragged             per-sequence draft lengths k_b ~ U{0..7}
  --variant tree [--tree T,D]  a full T-ary draft tree of depth D (default 2,2: six
                               nodes) through the tree attention and the tree walk
  --variant fused              RoPE + KV append, attention, the LM head (H = 4096),
                               rejection sampling on its logits, and the commit
  --workload 7b --sweep 256,64,16,4
                               the shrinking active batch: the same step on the
                               first B sequences of the workload's seeded batch
  --cpu-baseline-only          time the oracle (run in a single-threaded child)
  --copy-calibration           also run an elementwise kernel of known traffic
                               (negation of 512 MiB fp32: 512 MiB read, 512 MiB
                               written) for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE
  --summarize-rocprof DIR      turn rocprofv3 output in DIR into a text summary
  --write-counters             from a FETCH_SIZE run (--fetch-dir) and a WRITE_SIZE
                               run (--write-dir), both with --copy-calibration,
                               write the per-call HBM traffic file that the
                               roofline's `traffic` field is read from
"""

from __future__ import annotations

import argparse
import csv
import dataclasses
import glob
import hashlib
import json
import math
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
EVENT_STEPS = 30    # at least this many steps with per-call events for the averages
METRIC = "verified tokens/s + HBM GB/s (% of peak) for spec verify, 8B shape, k=3"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "verify_attn_8b_counters.txt")
LM_COUNTERS_FILE = os.path.join(ROOT, "profiles", "lm_head_8b_counters.txt")
# counter runs of the uniform step per workload, each taken at that workload's own batch and k
WORKLOAD_COUNTERS = {
    "8b": COUNTERS_FILE,
    "7b": os.path.join(ROOT, "profiles", "verify_7b_b256_counters.txt"),
    "longtail": os.path.join(ROOT, "profiles", "verify_longtail_counters.txt"),
    "262k": os.path.join(ROOT, "profiles", "verify_262k_counters.txt"),
}
# counter runs of other launches at the 8B shape: (variant, tree shape or None) -> summary
VARIANT_COUNTERS = {
    ("plain", None): os.path.join(ROOT, "profiles", "verify_plain_8b_counters.txt"),
    ("ragged", None): os.path.join(ROOT, "profiles", "verify_ragged_8b_counters.txt"),
    ("tree", "2,2"): os.path.join(ROOT, "profiles", "verify_tree_2x2_8b_counters.txt"),
    ("tree", "2,3"): os.path.join(ROOT, "profiles", "verify_tree_2x3_8b_counters.txt"),
}
# sources (and the build script, which holds per-file compiler flags) whose hash a counter
# summary records: counters taken before a change to any of them are not used
BUILD_SCRIPT = "speculative_decoding_verification_14_amd/build.py"
KERNEL_SOURCES = ["speculative_decoding_verification_14_amd/csrc/attention.hip",
                  "speculative_decoding_verification_14_amd/csrc/common.hpp", BUILD_SCRIPT]
LM_KERNEL_SOURCES = ["speculative_decoding_verification_14_amd/csrc/upstream.hip",
                     "speculative_decoding_verification_14_amd/csrc/common.hpp", BUILD_SCRIPT]
REJECT_KERNEL_SOURCES = [f"speculative_decoding_verification_14_amd/csrc/{f}"
                         for f in ("reject.hip", "common.hpp", "heavy.hpp", "softmax_step.hpp", "fastexp.hpp", "philox.hpp")] + [BUILD_SCRIPT]


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for rel in (KERNEL_SOURCES if sources is None else sources):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(preset, seq_lens, num_accepted, draft_lens=None):
    """Bytes the method itself must move (each K/V row, Q/O row, examined logits row once).

    draft_lens: per-sequence k_b (ragged); the preset's k for every sequence if None."""
    import numpy as np
    L = np.asarray(seq_lens, dtype=np.int64)
    a = np.asarray(num_accepted, dtype=np.int64)
    B, Hq, Hkv, D, bs, V = preset.B, preset.Hq, preset.Hkv, preset.D, preset.block_size, preset.V
    k = np.full(B, preset.k, dtype=np.int64) if draft_lens is None else np.asarray(draft_lens, dtype=np.int64)
    n_keys = L + k + 1
    attn = int(np.sum(n_keys) * Hkv * D * 2 * 2 + 2 * np.sum(k + 1) * Hq * D * 2
               + np.sum((n_keys + bs - 1) // bs) * 4 + B * 4 + (0 if draft_lens is None else (B + 1) * 4))
    rows = (a + 1) + np.minimum(a + 1, k)
    reject = int(np.sum(rows) * V * 4 + np.sum(k) * 4 + B * (8 + 4) + np.sum(k + 1) * 8 + B * 4 + np.sum(k) * 4
                 + (0 if draft_lens is None else (B + 1) * 4))
    commit = int(B * 4 * 3)
    return attn, reject, commit


def event_steps(step, n_events: int, steps: int) -> dict:
    """Per-call HIP events from a loop of its own, after the wall-clock loop: every event record
    leaves a bubble of a few microseconds, which belongs in the per-call averages but not in
    the wall-clock step time. At least EVENT_STEPS steps."""
    import torch
    evs = {i: [torch.cuda.Event(enable_timing=True) for _ in range(n_events)]
           for i in range(max(EVENT_STEPS, min(steps, 100)))}
    for e in evs.values():
        step(e)
    torch.cuda.synchronize()
    return evs


def reject_read_figure(B: int, k: int, V: int, seconds: float, algorithmic: int) -> dict:
    """How the sampling call ran this shape (spec_reject_sample_plan) and the logits bytes it
    read: the examined rows (the algorithmic count) when the levels run one after another,
    all 2k + 1 rows of every sequence when they run at once (small batches)."""
    import speculative_decoding_verification_14_amd as sv
    mode = sv.reject_sample_plan(B, k, V)
    read = B * (2 * k + 1) * V * 4 if mode == 2 else algorithmic
    gbs = read / seconds / 1e9
    return dict(launch=sv.REJECT_PLANS[mode], bytes_read=read, gbs_read=gbs, frac_of_peak_read=gbs / HBM_PEAK_GBS)


def dense_reject_figure(preset, seconds: float) -> dict:
    """Context only: the rate the sampling call would show if every logits row were read,
    all k + 1 target rows and all k draft rows (B * (2k + 1) * V * 4 bytes), whatever the
    acceptance outcome. The call reads only the rows its chain examines."""
    dense = preset.B * (2 * preset.k + 1) * preset.V * 4
    gbs = dense / seconds / 1e9
    return dict(bytes=dense, gbs=gbs, frac_of_peak=gbs / HBM_PEAK_GBS)


def workload_counters(workload: str, variant: str = "uniform", tree: str | None = None):
    """The counter summary that measured this bench line's launches, or None: the uniform step
    of each workload at its own shape, and at the 8B shape plain decoding (k = 0), the ragged
    step and the 2x2 and 2x3 trees (the fused pass has its own LM-head file)."""
    if variant == "uniform":
        return WORKLOAD_COUNTERS.get(workload)
    if workload != "8b":
        return None
    return VARIANT_COUNTERS.get((variant, tree if variant == "tree" else None))


def stored_traffic(path=None, sources=None, key="hbm_bytes_per_call"):
    """HBM bytes per call of a kernel from committed rocprofv3 counter runs, if still valid: the
    file records a hash of the attention kernel's sources, and of the sampling kernel's for
    key "reject_hbm_bytes_per_call"; a value whose sources have changed since is not used."""
    path = COUNTERS_FILE if path is None else path
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, _, v = line.partition(":")
                vals[k.strip()] = v.strip()
    if key == "reject_hbm_bytes_per_call":
        if vals.get("reject_source_sha256_16") != kernel_source_hash(REJECT_KERNEL_SOURCES):
            return None
    elif vals.get("kernel_source_sha256_16") != kernel_source_hash(sources):
        return None
    try:
        return int(float(vals[key]))
    except (KeyError, ValueError):
        return None


# ----------------------------------------------------------------------------- CPU baseline

# Inputs of the CPU baseline, set before its worker pool forks (the workers read them
# copy-on-write; the baseline runs in a child process that never touches the GPU).
_CB: dict = {}


def _cb_attention(pairs) -> int:
    from oracle import attention as oatt
    inp, p = _CB["inp"], _CB["p"]
    oatt.verify_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"], inp["seq_lens"], p.k,
                          p.Hq, p.Hkv, p.block_size, inp["sm_scale"], pairs=pairs)
    return len(pairs)


def _cb_reject(seqs) -> list:
    import numpy as np
    from oracle import reject as orej
    inp, p = _CB["inp"], _CB["p"]
    idx = np.asarray(seqs, dtype=np.int64)
    res = orej.verify_batch(inp["target_logits"][idx], inp["draft_logits"][idx], inp["draft_tokens"][idx],
                            inp["seq_ids"][idx], inp["seq_lens"][idx], p.k, p.temperature, inp["seed"])
    return res["num_accepted"].tolist()


def cpu_workers() -> int:
    """Worker processes for the pooled oracle: the cores this process may run on, at most 16
    (one GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(workload: str) -> dict:
    """The oracle on one whole step of the workload (every (sequence, KV head) pair of the
    attention, every sequence's rejection sampling, the commit), timed two ways on this host:
    (i) one process, one thread; (ii) a pool of worker processes, one BLAS thread each, the
    attention split by (sequence, KV head) pair and the sampling by sequence."""
    import multiprocessing

    import numpy as np
    from oracle import commit as ocommit
    from workloads import PRESETS, make_inputs
    p = PRESETS[workload]
    inp = make_inputs(workload)
    _CB.update(inp=inp, p=p)
    pairs = [(b, g) for b in range(p.B) for g in range(p.Hkv)]
    seqs = list(range(p.B))
    cap = inp["max_blocks"] * p.block_size

    t0 = time.perf_counter()
    _cb_attention(pairs)
    t_attn1 = time.perf_counter() - t0
    t0 = time.perf_counter()
    acc1 = np.asarray(_cb_reject(seqs), dtype=np.int32)
    t_rej1 = time.perf_counter() - t0
    t0 = time.perf_counter()
    ocommit.commit_lengths(inp["seq_lens"], acc1, cap)
    t_com1 = time.perf_counter() - t0

    n = cpu_workers()
    # pairs in order of decreasing key count, dealt round-robin, so the shares are even
    by_keys = sorted(pairs, key=lambda bg: -int(inp["seq_lens"][bg[0]]))
    attn_chunks = [by_keys[i::n] for i in range(n)]
    rej_chunks = [seqs[i::n] for i in range(n)]
    ctx = multiprocessing.get_context("fork")
    with ctx.Pool(n) as pool:
        pool.map(_cb_reject, [[0]] * n)            # workers started and warm before timing
        t0 = time.perf_counter()
        pool.map(_cb_attention, attn_chunks)
        t_attnN = time.perf_counter() - t0
        t0 = time.perf_counter()
        parts = pool.map(_cb_reject, rej_chunks)
        t_rejN = time.perf_counter() - t0
    accN = np.zeros(p.B, dtype=np.int32)
    for chunk, part in zip(rej_chunks, parts):
        accN[chunk] = part
    if not np.array_equal(acc1, accN):
        raise RuntimeError("the pooled oracle disagrees with the single-process one")
    t0 = time.perf_counter()
    ocommit.commit_lengths(inp["seq_lens"], accN, cap)
    t_comN = time.perf_counter() - t0
    tokens = int(np.sum(acc1 + 1))
    one = t_attn1 + t_rej1 + t_com1
    pooled = t_attnN + t_rejN + t_comN
    return dict(
        tokens_per_step=tokens, workers=n,
        single=dict(seconds_per_step=one, attn_seconds=t_attn1, reject_seconds=t_rej1, tokens_per_s=tokens / one),
        pooled=dict(seconds_per_step=pooled, attn_seconds=t_attnN, reject_seconds=t_rejN,
                    tokens_per_s=tokens / pooled),
        sample=(f"one whole step of the {workload} workload: attention of all {len(pairs)} (sequence, KV head) "
                f"pairs, rejection sampling of all {p.B} sequences, the commit; timed once in one process "
                f"(one thread) and once over a pool of {n} worker processes (one BLAS thread each)"))


def run_cpu_baseline_child(workload: str) -> dict | None:
    env = dict(os.environ)
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS",
                "NUMEXPR_NUM_THREADS"):
        env[var] = "1"
    cmd = [sys.executable, os.path.abspath(__file__), "--cpu-baseline-only", "--workload", workload]
    res = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=900)
    if res.returncode != 0:
        sys.stderr.write(res.stderr[-2000:])
        return None
    return json.loads(res.stdout.strip().splitlines()[-1])


# ----------------------------------------------------------------------------- rocprof summary

def _kernel_label(name: str) -> str:
    """Readable kernel name: namespaces and the argument list dropped, template arguments kept."""
    name = name.replace("(anonymous namespace)::", "").replace("specverify::", "")
    if name.startswith("void "):
        name = name[5:]
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    return name[:cut][:70]


def summarize_rocprof(path: str, out: str, command: str) -> None:
    """Summarise rocprofv3 kernel stats and/or counter CSVs found under ``path``."""
    lines = [f"# rocprofv3 summary", f"# command: {command}", ""]
    stats = sorted(glob.glob(os.path.join(path, "**", "*kernel_stats.csv"), recursive=True))
    for s in stats:
        lines.append(f"## kernel stats ({os.path.relpath(s, path)})")
        lines.append(f"{'kernel':70s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}")
        with open(s) as f:
            for row in csv.DictReader(f):
                short = _kernel_label(row["Name"])
                lines.append(f"{short:70s} {int(row['Calls']):6d} {float(row['AverageNs']) / 1e3:10.2f} "
                             f"{float(row['MinNs']) / 1e3:10.2f} {float(row['MaxNs']) / 1e3:10.2f} "
                             f"{float(row['Percentage']):6.2f}")
        lines.append("")
    ctrs = sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True))
    for c in ctrs:
        lines.append(f"## counters per dispatch, averaged by kernel ({os.path.relpath(c, path)})")
        agg = {}
        with open(c) as f:
            for row in csv.DictReader(f):
                key = (_kernel_label(row["Kernel_Name"]), row["Counter_Name"])
                agg.setdefault(key, []).append(float(row["Counter_Value"]))
        lines.append(f"{'kernel':70s} {'counter':>12s} {'dispatches':>10s} {'mean':>16s}")
        for (k, cn), v in sorted(agg.items()):
            lines.append(f"{k:70s} {cn:>12s} {len(v):10d} {sum(v) / len(v):16.1f}")
        lines.append("")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


CALIB_BYTES = 1 << 29   # bytes read and bytes written by one calibration dispatch


def _counter_means(path: str, counter: str) -> dict:
    """Mean value per dispatch of one rocprofv3 counter, by kernel label."""
    files = sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {path}")
    agg = {}
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] == counter:
                    agg.setdefault(_kernel_label(row["Kernel_Name"]), []).append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in agg.items()}


def write_counters(fetch_dir: str, write_dir: str, out: str, fetch_cmd: str, write_cmd: str,
                   kind: str = "attn", title: str = "") -> None:
    """Per-call HBM bytes of the verify attention (and, for reference, the reject
    kernel), or with kind "lm" of the LM head, from FETCH_SIZE / WRITE_SIZE runs, each
    scaled by what the same counter reads for the calibration kernel of known traffic."""
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")
    calib = lambda d: [v for k, v in d.items() if "neg" in k.lower()]
    cf, cw = calib(fetch), calib(write)
    if not cf or not cw:
        raise RuntimeError("calibration kernel not found in the counter runs (run them with --copy-calibration)")
    f_scale = CALIB_BYTES / (max(cf) * 1024.0)   # counters are in KiB per dispatch
    w_scale = CALIB_BYTES / (max(cw) * 1024.0)
    per_call = lambda ks: sum(fetch.get(k, 0.0) * 1024.0 * f_scale + write.get(k, 0.0) * 1024.0 * w_scale for k in ks)
    head = ["# FETCH_SIZE / WRITE_SIZE are KiB per dispatch; each is scaled by the factor that maps the",
            "# calibration kernel (fp32 negation: 512 MiB read, 512 MiB written) onto its known traffic."]
    if kind == "lm":
        lm = sorted(k for k in set(fetch) | set(write) if k.startswith("lm_head"))
        lines = ["# rocprofv3 hardware counters, LM head of the 8b fused pass (R=256, H=4096, V=128256)",
                 f"# fetch command: {fetch_cmd}", f"# write command: {write_cmd}", *head,
                 f"kernel_source_sha256_16: {kernel_source_hash(LM_KERNEL_SOURCES)}",
                 f"fetch_scale: {f_scale:.4f}", f"write_scale: {w_scale:.4f}"]
        for k in lm:
            lines.append(f"{k}: FETCH_SIZE {fetch.get(k, 0.0):.1f} KiB, WRITE_SIZE {write.get(k, 0.0):.1f} KiB "
                         "per dispatch")
        lines.append(f"hbm_bytes_per_call: {per_call(lm):.0f}")
    else:
        attn = sorted(k for k in set(fetch) | set(write) if k.startswith("attn_"))
        rej = sorted(k for k in set(fetch) | set(write) if k.startswith("reject_"))
        lines = [f"# rocprofv3 hardware counters, {title or '8b workload (B=64, k=3, V=128256)'}, "
                 "one call of each kernel per step",
                 f"# fetch command: {fetch_cmd}", f"# write command: {write_cmd}", *head,
                 f"kernel_source_sha256_16: {kernel_source_hash()}",
                 f"reject_source_sha256_16: {kernel_source_hash(REJECT_KERNEL_SOURCES)}",
                 f"fetch_scale: {f_scale:.4f}", f"write_scale: {w_scale:.4f}"]
        for k in attn + rej:
            lines.append(f"{k}: FETCH_SIZE {fetch.get(k, 0.0):.1f} KiB, WRITE_SIZE {write.get(k, 0.0):.1f} KiB "
                         "per dispatch")
        lines.append(f"hbm_bytes_per_call: {per_call(attn):.0f}")
        lines.append(f"reject_hbm_bytes_per_call: {per_call(rej):.0f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


MFMA_FILE = os.path.join(ROOT, "profiles", "verify_attn_8b_mfma_counters.txt")
MFMA_PEAK_BF16_TFLOPS = 2500.0   # dense bf16 MFMA peak of the chip
SIMDS = 256 * 4


def attention_flops(preset, seq_lens, draft_lens=None) -> int:
    """Algorithmic attention flops: 2*D for q.k and 2*D for p.v per (query row, visible key)."""
    import numpy as np
    L = np.asarray(seq_lens, dtype=np.int64)
    k = np.full(L.shape, preset.k, dtype=np.int64) if draft_lens is None else np.asarray(draft_lens, np.int64)
    # row i of sequence b sees L_b + i + 1 keys
    keys = np.sum((k + 1) * L + (k + 1) * (k + 2) // 2)
    return int(4 * preset.D * preset.Hq * keys)


def write_mfma(pmc_dir: str, out: str, command: str) -> None:
    """MFMA use of the verify attention from one rocprofv3 run with the MFMA counters and a
    kernel trace: bf16 matrix flops per dispatch (SQ_INSTS_VALU_MFMA_MOPS_BF16 counts units of
    512 flops), their rate over the traced duration, and the matrix pipes' busy fraction
    (SQ_VALU_MFMA_BUSY_CYCLES, summed over the 1024 SIMDs, over SIMDs x traced cycles at 2.4 GHz)."""
    mops = _counter_means(pmc_dir, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    busy = _counter_means(pmc_dir, "SQ_VALU_MFMA_BUSY_CYCLES")
    stats = sorted(glob.glob(os.path.join(pmc_dir, "**", "*kernel_stats.csv"), recursive=True))
    dur = {}
    for st in stats:
        with open(st) as f:
            for row in csv.DictReader(f):
                dur[_kernel_label(row["Name"])] = float(row["AverageNs"]) * 1e-9
    lines = ["# rocprofv3 MFMA counters, verify attention of the 8b workload (B=64, k=3, Hq=32, Hkv=8, D=128)",
             f"# command: {command}",
             "# flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512 per dispatch; rate over the average traced duration",
             "# of the same run (kernels are serialised while counters are read, so the duration can be longer",
             "# than in an unprofiled run); busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs * duration * 2.4 GHz)",
             f"kernel_source_sha256_16: {kernel_source_hash()}",
             f"mfma_peak_bf16_tflops: {MFMA_PEAK_BF16_TFLOPS:.0f}"]
    for kname in sorted(k for k in mops if k.startswith("attn_")):
        flops = mops[kname] * 512.0
        d = dur.get(kname)
        rate = flops / d / 1e12 if d else float("nan")
        b = busy.get(kname, float("nan"))
        bfrac = b / (SIMDS * d * 2.4e9) if d else float("nan")
        lines.append(f"{kname}: mfma_flops {flops:.4g} per dispatch, traced avg {d * 1e6 if d else float('nan'):.1f} us, "
                     f"{rate:.1f} TFLOP/s = {rate / MFMA_PEAK_BF16_TFLOPS:.4f} of bf16 peak, "
                     f"MFMA busy cycles {b:.4g} ({bfrac:.4f} of SIMD cycles)")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


XCDS = 8   # GRBM counters are summed over the chip's accelerator dies


def clock_table(pmc_csv_rows) -> dict:
    """Average shader clock per kernel label from rows of a counter_collection.csv holding
    GRBM_COUNT: the counter ticks once per engine clock in each of the 8 dies while the
    dispatch runs, so GRBM_COUNT / 8 / (end - start) is the dispatch's mean clock.
    Returns {label: (dispatches, median duration in us, median clock in GHz)}."""
    per = {}
    for row in pmc_csv_rows:
        if row["Counter_Name"] != "GRBM_COUNT":
            continue
        ns = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
        if ns <= 0:
            continue
        per.setdefault(_kernel_label(row["Kernel_Name"]), []).append(
            (ns * 1e-3, float(row["Counter_Value"]) / XCDS / ns))
    med = lambda v: sorted(v)[len(v) // 2]
    return {k: (len(v), med([x[0] for x in v]), med([x[1] for x in v])) for k, v in per.items()}


def write_clock(pmc_dir: str, out: str, command: str, title: str) -> None:
    """Shader clock per kernel from one rocprofv3 run with GRBM_GUI_ACTIVE and GRBM_COUNT."""
    files = sorted(glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {pmc_dir}")
    rows = []
    for fn in files:
        with open(fn) as f:
            rows.extend(csv.DictReader(f))
    max_mhz = ""
    for fn in glob.glob(os.path.join(pmc_dir, "**", "*agent_info.csv"), recursive=True):
        with open(fn) as f:
            for row in csv.DictReader(f):
                if row.get("Agent_Type") == "GPU":
                    max_mhz = row.get("Max_Engine_Clk_Fcompute", "")
    lines = [f"# rocprofv3 GRBM counters, {title}: mean shader clock per kernel",
             f"# command: {command}",
             f"# clock = GRBM_COUNT / {XCDS} dies / (End_Timestamp - Start_Timestamp) of the dispatch; "
             "medians over the dispatches",
             f"# maximum engine clock reported by the agent: {max_mhz} MHz",
             "# the counters' window outlasts a dispatch by a few microseconds (a 7 us kernel reads ~4.7 GHz),",
             "# so only dispatches over 100 us are listed; for those the clock reads at most ~2-3% high",
             f"kernel_source_sha256_16: {kernel_source_hash()}",
             f"lm_head_source_sha256_16: {kernel_source_hash(LM_KERNEL_SOURCES)}",
             f"{'kernel':70s} {'dispatches':>10s} {'median_us':>10s} {'clock_GHz':>10s}"]
    for k, (n, us, ghz) in sorted(clock_table(rows).items(), key=lambda kv: -kv[1][1]):
        if us < 100.0:
            continue   # the counters' window outlasts a dispatch by a few microseconds: short ones read high
        lines.append(f"{k:70s} {n:10d} {us:10.1f} {ghz:10.3f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# ----------------------------------------------------------------------------- GPU benchmark

def copy_calibration(dev) -> dict:
    """An elementwise kernel of known traffic for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = 1 << 27   # 128 Mi fp32 = 512 MiB read + 512 MiB written by one elementwise kernel
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    return dict(kernel="elementwise neg (fp32)", bytes_read=4 * n, bytes_written=4 * n, calls=3)


def cold_cache_calls(step, dev, n: int) -> dict | None:
    """Per-call HIP-event times over n steps, each preceded by a 512 MiB write that
    evicts the L2 and the MALL (the write itself is outside the timed calls)."""
    import torch
    if n <= 0:
        return None
    scratch = torch.empty(1 << 27, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    rows = []
    for _ in range(n):
        scratch.fill_(1.0)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        step(ev)
        rows.append(ev)
    torch.cuda.synchronize()
    del scratch
    us = lambda i: sum(e[i].elapsed_time(e[i + 1]) for e in rows) / len(rows) * 1e3
    return dict(steps=n, flush_bytes=1 << 29, verify_attn=dict(avg_us=us(0)), reject_sample=dict(avg_us=us(1)),
                commit_lengths=dict(avg_us=us(2)))


def gpu_bench_ragged(args, p, dev) -> dict:
    """The 8B step with per-sequence draft lengths k_b ~ U{0..7} (packed rows)."""
    import numpy as np
    import torch
    import speculative_decoding_verification_14_amd as sv
    from workloads import make_ragged_attention_inputs, make_ragged_reject_inputs

    k_max = 7
    print(f"[bench] generating ragged {args.workload} inputs (k_b in 0..{k_max})", file=sys.stderr, flush=True)
    a = make_ragged_attention_inputs(p, k_max)
    r = make_ragged_reject_inputs(p, k_max, draft_lens=a["draft_lens"])
    assert np.array_equal(a["seq_lens"], r["seq_lens"])
    bf16 = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    B = p.B
    q, kc, vc, bt = bf16(a["q"]), bf16(a["k_cache"]), bf16(a["v_cache"]), t(a["block_table"])
    del a["k_cache"], a["v_cache"]
    cu = t(a["cu_drafts"])
    seq_lens0 = t(a["seq_lens"])
    seq_lens = seq_lens0.clone()
    tl, dl, dt, sid = t(r["target_logits"]), t(r["draft_logits"]), t(r["draft_tokens"]), t(r["seq_ids"])
    T, K = tl.shape[0], dl.shape[0]
    attn_out = torch.empty_like(q)
    out_tokens = torch.empty(T, dtype=torch.int32, device=dev)
    out_probs = torch.empty(T, dtype=torch.float32, device=dev)
    acc_probs = torch.empty(K, dtype=torch.float32, device=dev)
    num_acc = torch.empty(B, dtype=torch.int32, device=dev)
    overflow = torch.empty(B, dtype=torch.int32, device=dev)
    cap = a["max_blocks"] * p.block_size
    msl = a["max_seq_len"]
    attn_ws = torch.zeros(max(256, sv.verify_attn_workspace_size(B, k_max, p.Hq, p.Hkv, p.D, msl)),
                          dtype=torch.uint8, device=dev)
    rej_ws = torch.zeros(sv.reject_sample_workspace_size(B, k_max, p.V), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(events=None):
        seq_lens.copy_(seq_lens0)
        if events is not None:
            events[0].record(stream)
        sv.verify_attn_ragged(q, kc, vc, bt, seq_lens, cu, attn_out, k_max, msl, None, attn_ws, stream)
        if events is not None:
            events[1].record(stream)
        sv.reject_sample_ragged(tl, dl, dt, cu, sid, seq_lens, k_max, p.temperature, r["seed"], out_tokens,
                                num_acc, out_probs, acc_probs, rej_ws, stream)
        if events is not None:
            events[2].record(stream)
        sv.commit_lengths(seq_lens, num_acc, k_max, cap, overflow, stream)
        if events is not None:
            events[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    acc_ref = num_acc.cpu().numpy().copy()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    evs = event_steps(step, 4, args.steps)
    acc = num_acc.cpu().numpy()
    if not np.array_equal(acc, acc_ref):
        raise RuntimeError("accepted lengths changed between steps; the step is not repeatable")
    mean = lambda v: sum(v) / len(v)
    attn_s = mean([e[0].elapsed_time(e[1]) for e in evs.values()]) / 1e3
    rej_s = mean([e[1].elapsed_time(e[2]) for e in evs.values()]) / 1e3
    com_s = mean([e[2].elapsed_time(e[3]) for e in evs.values()]) / 1e3
    a_bytes, r_bytes, _ = algorithmic_bytes(p, a["seq_lens"], acc, a["draft_lens"])
    tokens = int(np.sum(acc + 1))
    step_s = wall / args.steps
    attn_gbs, rej_gbs = a_bytes / attn_s / 1e9, r_bytes / rej_s / 1e9
    return dict(
        metric=METRIC, value=tokens / step_s, unit="verified tokens/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=step_s * 1e3, higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="bf16", data="synthetic",
        config=dict(workload=(f"{args.workload} with ragged draft lengths: B={B}, k_b ~ U{{0..{k_max}}} "
                              f"(sum {int(np.sum(a['draft_lens']))}), Hq={p.Hq}, Hkv={p.Hkv}, D={p.D}, "
                              f"contexts {p.ctx}, block_size={p.block_size}, V={p.V}, T={p.temperature}, "
                              "one attention layer + rejection sampling + commit"),
                    global_batch=B, k="ragged", parallelism="none (1 GPU)"),
        roofline=dict(bound="hbm", achieved=attn_gbs, peak=HBM_PEAK_GBS, unit="GB/s", frac=attn_gbs / HBM_PEAK_GBS,
                      traffic=stored_traffic(workload_counters(args.workload, "ragged"))
                      if workload_counters(args.workload, "ragged") else None,
                      kernel="spec_verify_attn_ragged (attn_streamk_kernel + attn_merge_kernel)",
                      algorithmic_bytes_per_call=a_bytes, avg_call_us=attn_s * 1e6),
        verified_tokens_per_step=tokens,
        kernels=dict(verify_attn=dict(avg_us=attn_s * 1e6, bytes=a_bytes, gbs=attn_gbs,
                                      frac_of_peak=attn_gbs / HBM_PEAK_GBS),
                     reject_sample=dict(avg_us=rej_s * 1e6, bytes=r_bytes, gbs=rej_gbs,
                                        frac_of_peak=rej_gbs / HBM_PEAK_GBS),
                     commit_lengths=dict(avg_us=com_s * 1e6)),
        cold_cache=cold_cache_calls(step, dev, args.cold_steps),
    )


def gpu_bench_fused(args, p, dev) -> dict:
    """The whole verify pass of one attention layer plus the output head on the 8B shape: RoPE and
    KV append of the k+1 new rows, verify attention, the LM head (hidden [B(k+1)][4096] x W
    [128256][4096]^T), rejection sampling on those logits, and the commit. The draft logits are the
    LM head's logits plus the 8B recipe's draft noise, and the draft tokens are sampled from them,
    so acceptance behaves as in the three-call step."""
    import numpy as np
    import torch
    import speculative_decoding_verification_14_amd as sv
    from workloads import (ROPE_THETA, draft_from_logits, make_attention_inputs, make_lm_head_inputs,
                           make_new_rows, verify_seed)

    B, k, H = p.B, p.k, 4096
    R = B * (k + 1)
    theta = ROPE_THETA.get(args.workload, 500000.0)
    print(f"[bench] generating {args.workload} inputs for the fused pass (R = {R}, H = {H}, V = {p.V})",
          file=sys.stderr, flush=True)
    a = make_attention_inputs(p)
    rows = make_new_rows(p, k, seed=p.index)
    lm = make_lm_head_inputs(R, H, p.V, seed=p.index)
    bf16 = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    q, kn, vn = bf16(rows["q"]), bf16(rows["k_new"]), bf16(rows["v_new"])
    kc, vc, bt = bf16(a["k_cache"]), bf16(a["v_cache"]), t(a["block_table"])
    del a["k_cache"], a["v_cache"]
    hidden, weight = bf16(lm["hidden"]), bf16(lm["weight"])
    del lm
    tl = torch.empty((B, k + 1, p.V), dtype=torch.float32, device=dev)
    sv.lm_head(hidden, weight, tl)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(1000 + p.index))
    target = tl.cpu().numpy()
    draft = np.ascontiguousarray(target[:, :k] + rng.standard_normal((B, k, p.V), dtype=np.float32)
                                 * np.float32(p.draft_sigma))
    tokens = draft_from_logits(rng, draft, p.temperature).astype(np.int32)
    dl, dt = t(draft), t(tokens)
    sid = t((np.arange(B, dtype=np.int64) * 7919 + 1_000_003 * (p.index + 1)).astype(np.int64))
    seq_lens0 = t(a["seq_lens"])
    seq_lens = seq_lens0.clone()
    attn_out = torch.empty_like(q)
    out_tokens = torch.empty((B, k + 1), dtype=torch.int32, device=dev)
    num_acc = torch.empty(B, dtype=torch.int32, device=dev)
    out_probs = torch.empty((B, k + 1), dtype=torch.float32, device=dev)
    acc_probs = torch.empty((B, k), dtype=torch.float32, device=dev)
    overflow = torch.empty(B, dtype=torch.int32, device=dev)
    cap = a["max_blocks"] * p.block_size
    msl = a["max_seq_len"]
    attn_ws = torch.zeros(max(256, sv.verify_attn_workspace_size(B, k, p.Hq, p.Hkv, p.D, msl)),
                          dtype=torch.uint8, device=dev)
    rej_ws = torch.zeros(sv.reject_sample_workspace_size(B, k, p.V), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    seed = verify_seed(p)

    def step(events=None):
        rec = (lambda i: events[i].record(stream)) if events is not None else (lambda i: None)
        seq_lens.copy_(seq_lens0)
        rec(0)
        sv.rope_append(q, kn, vn, kc, vc, bt, seq_lens, theta, None, stream)   # q turns again each step
        rec(1)
        sv.verify_attn(q, kc, vc, bt, seq_lens, attn_out, msl, None, attn_ws, stream)
        rec(2)
        sv.lm_head(hidden, weight, tl, stream)
        rec(3)
        sv.reject_sample(tl, dl, dt, sid, seq_lens, p.temperature, seed, out_tokens, num_acc, out_probs, acc_probs,
                         rej_ws, stream)
        rec(4)
        sv.commit_lengths(seq_lens, num_acc, k, cap, overflow, stream)
        rec(5)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    acc_ref = num_acc.cpu().numpy().copy()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    evs = event_steps(step, 6, args.steps)
    acc = num_acc.cpu().numpy()
    if not np.array_equal(acc, acc_ref):
        raise RuntimeError("accepted lengths changed between steps; the step is not repeatable")
    mean = lambda v: sum(v) / len(v)
    call_s = [mean([e[j].elapsed_time(e[j + 1]) for e in evs.values()]) / 1e3 for j in range(5)]
    vs_lib = lm_head_vs_library(hidden, weight, tl, stream)
    a_bytes, r_bytes, _ = algorithmic_bytes(p, a["seq_lens"], acc)
    lm_bytes = p.V * H * 2 + R * H * 2 + R * p.V * 4
    lm_flops = 2.0 * R * H * p.V
    rope_bytes = B * (k + 1) * (p.Hq * 2 + p.Hkv * 3) * p.D * 2
    tokens = int(np.sum(acc + 1))
    step_s = wall / args.steps
    gbs = lambda by, sec: by / sec / 1e9
    lm_gbs, lm_tf = gbs(lm_bytes, call_s[2]), lm_flops / call_s[2] / 1e12
    if args.copy_calibration:
        copy_calibration(dev)
    return dict(
        metric=METRIC, value=tokens / step_s, unit="verified tokens/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=step_s * 1e3, higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="bf16", data="synthetic",
        config=dict(workload=(f"{args.workload} fused pass: B={B}, k={k}, Hq={p.Hq}, Hkv={p.Hkv}, D={p.D}, "
                              f"contexts {p.ctx}, block_size={p.block_size}, H={H}, V={p.V}, T={p.temperature}, "
                              f"RoPE theta={theta:g}; RoPE + KV append, one attention layer, LM head, rejection "
                              "sampling, commit"),
                    global_batch=B, k=k, parallelism="none (1 GPU)"),
        roofline=dict(bound="hbm", achieved=lm_gbs, peak=HBM_PEAK_GBS, unit="GB/s", frac=lm_gbs / HBM_PEAK_GBS,
                      traffic=stored_traffic(LM_COUNTERS_FILE, LM_KERNEL_SOURCES),
                      kernel="spec_lm_head (lm_head_kernel)", algorithmic_bytes_per_call=lm_bytes,
                      avg_call_us=call_s[2] * 1e6,
                      mfma=dict(achieved=lm_tf, peak=2500.0, unit="TFLOP/s", frac=lm_tf / 2500.0)),
        verified_tokens_per_step=tokens,
        mean_emitted_per_sequence=tokens / B,
        kernels=dict(
            rope_append=dict(avg_us=call_s[0] * 1e6, bytes=rope_bytes, gbs=gbs(rope_bytes, call_s[0])),
            verify_attn=dict(avg_us=call_s[1] * 1e6, bytes=a_bytes, gbs=gbs(a_bytes, call_s[1]),
                             frac_of_peak=gbs(a_bytes, call_s[1]) / HBM_PEAK_GBS),
            lm_head=dict(avg_us=call_s[2] * 1e6, bytes=lm_bytes, gbs=lm_gbs, frac_of_peak=lm_gbs / HBM_PEAK_GBS,
                         tflops=lm_tf, frac_of_mfma_peak=lm_tf / 2500.0),
            reject_sample=dict(avg_us=call_s[3] * 1e6, bytes=r_bytes, gbs=gbs(r_bytes, call_s[3]),
                               frac_of_peak=gbs(r_bytes, call_s[3]) / HBM_PEAK_GBS),
            commit_lengths=dict(avg_us=call_s[4] * 1e6)),
        lm_head_vs_library=vs_lib,
    )


def lm_head_vs_library(hidden, weight, logits, stream, rounds: int = 6, calls: int = 10) -> dict:
    """spec_lm_head against torch's library GEMM (torch.nn.functional.linear, bf16 output) on the
    same operands, back to back: rounds of `calls` calls of each, interleaved, every call timed
    with events on the stream both run on; medians over all calls."""
    import torch
    import torch.nn.functional as F
    import speculative_decoding_verification_14_amd as sv
    times = {"spec_lm_head": [], "torch_linear": []}
    with torch.cuda.stream(stream):
        for _ in range(2):
            sv.lm_head(hidden, weight, logits, stream)
            F.linear(hidden, weight)
        for _ in range(rounds):
            for name in times:
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(calls + 1)]
                ev[0].record(stream)
                for i in range(calls):
                    if name == "spec_lm_head":
                        sv.lm_head(hidden, weight, logits, stream)
                    else:
                        F.linear(hidden, weight)
                    ev[i + 1].record(stream)
                torch.cuda.synchronize()
                times[name] += [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(calls)]
    med = {k: float(sorted(v)[len(v) // 2]) for k, v in times.items()}
    return dict(spec_lm_head_median_us=med["spec_lm_head"], torch_linear_median_us=med["torch_linear"],
                spec_lm_head_min_us=min(times["spec_lm_head"]), torch_linear_min_us=min(times["torch_linear"]),
                speedup=med["torch_linear"] / med["spec_lm_head"], calls_each=rounds * calls,
                library_call="torch.nn.functional.linear(hidden, weight): bf16 logits, half the output bytes")


def tree_shape(spec: str) -> tuple[int, int]:
    t, d = (int(x) for x in spec.split(","))
    return t, d


def gpu_bench_tree(args, p, dev) -> dict:
    """The 8B step over a full t-ary draft tree of depth d (the same tree for every sequence):
    tree attention, the tree walk, and the tree commit (the accepted path's KV rows move to
    L+1 .. L+a, then the lengths). The lengths are restored before every step; the moved rows
    only change attention outputs, which the walk does not read, so every step does the same work."""
    import numpy as np
    import torch
    import speculative_decoding_verification_14_amd as sv
    from workloads import make_tree_attention_inputs, make_tree_reject_inputs, tree_parents

    t_br, depth = tree_shape(args.tree)
    parents = tree_parents(t_br, depth)
    N = int(parents.shape[0])
    print(f"[bench] generating {args.workload} tree inputs (t = {t_br}, depth = {depth}, N = {N})",
          file=sys.stderr, flush=True)
    a = make_tree_attention_inputs(p, N)
    r = make_tree_reject_inputs(p, parents)
    assert np.array_equal(a["seq_lens"], r["seq_lens"])
    bf16 = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    B = p.B
    q, kc, vc, bt = bf16(a["q"]), bf16(a["k_cache"]), bf16(a["v_cache"]), t(a["block_table"])
    del a["k_cache"], a["v_cache"]
    par = t(r["parents"])
    seq_lens0 = t(a["seq_lens"])
    seq_lens = seq_lens0.clone()
    tl, dl, dt, sid = t(r["target_logits"]), t(r["draft_logits"]), t(r["draft_tokens"]), t(r["seq_ids"])
    del r["target_logits"], r["draft_logits"]
    attn_out = torch.empty_like(q)
    out_tokens = torch.empty((B, N + 1), dtype=torch.int32, device=dev)
    out_probs = torch.empty((B, N + 1), dtype=torch.float32, device=dev)
    acc_probs = torch.empty((B, N), dtype=torch.float32, device=dev)
    acc_nodes = torch.empty((B, N), dtype=torch.int32, device=dev)
    num_acc = torch.empty(B, dtype=torch.int32, device=dev)
    overflow = torch.empty(B, dtype=torch.int32, device=dev)
    cap = a["max_blocks"] * p.block_size
    msl = a["max_seq_len"]
    attn_ws = torch.zeros(max(256, sv.verify_attn_workspace_size(B, N, p.Hq, p.Hkv, p.D, msl)),
                          dtype=torch.uint8, device=dev)
    rej_ws = torch.zeros(sv.reject_sample_tree_workspace_size(B, N, p.V), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(events=None):
        seq_lens.copy_(seq_lens0)
        if events is not None:
            events[0].record(stream)
        sv.verify_attn_tree(q, kc, vc, bt, seq_lens, par, attn_out, msl, None, attn_ws, stream)
        if events is not None:
            events[1].record(stream)
        sv.reject_sample_tree(tl, dl, dt, par, sid, seq_lens, p.temperature, r["seed"], out_tokens, num_acc,
                              acc_nodes, out_probs, acc_probs, rej_ws, stream)
        if events is not None:
            events[2].record(stream)
        sv.commit_tree(kc, vc, bt, seq_lens, acc_nodes, num_acc, cap, overflow, stream)
        if events is not None:
            events[3].record(stream)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    acc_ref = num_acc.cpu().numpy().copy()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    evs = event_steps(step, 4, args.steps)
    acc = num_acc.cpu().numpy()
    nodes = acc_nodes.cpu().numpy()
    if not np.array_equal(acc, acc_ref):
        raise RuntimeError("accepted lengths changed between steps; the step is not repeatable")
    mean = lambda v: sum(v) / len(v)
    attn_s = mean([e[0].elapsed_time(e[1]) for e in evs.values()]) / 1e3
    rej_s = mean([e[1].elapsed_time(e[2]) for e in evs.values()]) / 1e3
    com_s = mean([e[2].elapsed_time(e[3]) for e in evs.values()]) / 1e3
    a_bytes, _, _ = algorithmic_bytes(dataclasses.replace(p, k=N), a["seq_lens"], acc)
    r_bytes = tree_reject_bytes(p, parents, acc, nodes)
    tokens = int(np.sum(acc + 1))
    step_s = wall / args.steps
    attn_gbs, rej_gbs = a_bytes / attn_s / 1e9, r_bytes / rej_s / 1e9
    return dict(
        metric=METRIC, value=tokens / step_s, unit="verified tokens/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=step_s * 1e3, higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="bf16", data="synthetic",
        config=dict(workload=(f"{args.workload} with a draft tree: B={B}, full {t_br}-ary tree of depth {depth} "
                              f"(N={N} draft nodes), Hq={p.Hq}, Hkv={p.Hkv}, D={p.D}, contexts {p.ctx}, "
                              f"block_size={p.block_size}, V={p.V}, T={p.temperature}, "
                              "one attention layer + tree walk + tree commit"),
                    global_batch=B, k=f"tree {t_br}x{depth}", parallelism="none (1 GPU)"),
        roofline=dict(bound="hbm", achieved=attn_gbs, peak=HBM_PEAK_GBS, unit="GB/s", frac=attn_gbs / HBM_PEAK_GBS,
                      traffic=stored_traffic(workload_counters(args.workload, "tree", args.tree))
                      if workload_counters(args.workload, "tree", args.tree) else None,
                      kernel="spec_verify_attn_tree (attn_streamk_kernel + attn_merge_kernel)",
                      algorithmic_bytes_per_call=a_bytes, avg_call_us=attn_s * 1e6),
        verified_tokens_per_step=tokens,
        mean_emitted_per_sequence=tokens / B,
        kernels=dict(verify_attn=dict(avg_us=attn_s * 1e6, bytes=a_bytes, gbs=attn_gbs,
                                      frac_of_peak=attn_gbs / HBM_PEAK_GBS),
                     reject_sample=dict(avg_us=rej_s * 1e6, bytes=r_bytes, gbs=rej_gbs,
                                        frac_of_peak=rej_gbs / HBM_PEAK_GBS),
                     commit_tree=dict(avg_us=com_s * 1e6)),
        cold_cache=cold_cache_calls(step, dev, args.cold_steps),
    )


def tree_reject_bytes(preset, parents, num_accepted, accepted_nodes) -> int:
    """Bytes the tree walk must read: the target row of every node on the walked path, and the
    draft row of those that have children (their candidates are tested against it), plus the
    token, parent, length and output arrays."""
    import numpy as np
    par = np.asarray(parents)
    N, V, B = int(par.shape[-1]), preset.V, preset.B
    has_kids = np.zeros(N + 1, dtype=bool)
    has_kids[par] = True
    rows = 0
    for b in range(B):
        path = [0] + [int(x) for x in accepted_nodes[b, :int(num_accepted[b])]]
        rows += sum(2 if has_kids[v] else 1 for v in path)
    return int(rows * V * 4 + B * N * 4 * 2 + B * (8 + 4) + B * (N + 1) * 8 + B * N * 8 + B * 4)


def gpu_bench(args) -> dict:
    import numpy as np
    import torch
    import speculative_decoding_verification_14_amd as sv
    from workloads import PRESETS, make_inputs

    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU (one MI355X)")
    sv.library()
    dev = torch.device("cuda:0")
    p = PRESETS[args.workload]
    if args.variant == "plain":
        p = dataclasses.replace(p, k=0)
    if args.variant in ("ragged", "tree") and args.copy_calibration:
        copy_calibration(dev)   # the counter runs' calibration kernel (the other paths run it themselves)
    if args.variant == "ragged":
        return gpu_bench_ragged(args, p, dev)
    if args.variant == "tree":
        return gpu_bench_tree(args, p, dev)
    if args.variant == "fused":
        return gpu_bench_fused(args, p, dev)
    if args.sweep:
        return gpu_bench_sweep(args, p, dev)
    print(f"[bench] generating {args.workload} inputs (k = {p.k})", file=sys.stderr, flush=True)
    inp = make_inputs(args.workload, preset=p)

    def bf16(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)

    def t(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    q, kc, vc = bf16(inp["q"]), bf16(inp["k_cache"]), bf16(inp["v_cache"])
    bt = t(inp["block_table"])
    seq_lens0 = t(inp["seq_lens"])
    seq_lens = seq_lens0.clone()
    tl, sid = t(inp["target_logits"]), t(inp["seq_ids"])
    dl = t(inp["draft_logits"]) if p.k > 0 else None
    dt = t(inp["draft_tokens"]) if p.k > 0 else None
    B, k = p.B, p.k
    attn_out = torch.empty_like(q)
    out_tokens = torch.empty((B, k + 1), dtype=torch.int32, device=dev)
    num_acc = torch.empty(B, dtype=torch.int32, device=dev)
    out_probs = torch.empty((B, k + 1), dtype=torch.float32, device=dev)
    acc_probs = torch.empty((B, k), dtype=torch.float32, device=dev) if k > 0 else None
    overflow = torch.empty(B, dtype=torch.int32, device=dev)
    cap = inp["max_blocks"] * p.block_size
    msl = inp["max_seq_len"]
    attn_ws = torch.zeros(max(256, sv.verify_attn_workspace_size(B, k, p.Hq, p.Hkv, p.D, msl)),
                          dtype=torch.uint8, device=dev)
    rej_ws = torch.zeros(sv.reject_sample_workspace_size(B, k, p.V), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    del inp["k_cache"], inp["v_cache"]

    def step(events=None):
        seq_lens.copy_(seq_lens0)
        if events is not None:
            events[0].record(stream)
        sv.verify_attn(q, kc, vc, bt, seq_lens, attn_out, msl, None, attn_ws, stream)
        if events is not None:
            events[1].record(stream)
        sv.reject_sample(tl, dl, dt, sid, seq_lens, p.temperature, inp["seed"], out_tokens, num_acc, out_probs,
                         acc_probs, rej_ws, stream)
        if events is not None:
            events[2].record(stream)
        sv.commit_lengths(seq_lens, num_acc, k, cap, overflow, stream)
        if events is not None:
            events[3].record(stream)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    acc_ref = num_acc.cpu().numpy().copy()

    # The timed steps carry no events (each event record is a barrier packet that leaves a
    # few-microsecond bubble in the stream); the per-call times come from the same steps
    # run again right after, with HIP events around every call of every step.
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    acc = num_acc.cpu().numpy()
    if not np.array_equal(acc, acc_ref):
        raise RuntimeError("accepted lengths changed between steps; the step is not repeatable")
    n_ev = max(args.steps, EVENT_STEPS)
    print(f"[bench] per-call events on {n_ev} steps", file=sys.stderr, flush=True)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_ev)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    attn_ms = [e[0].elapsed_time(e[1]) for e in evs]
    rej_ms = [e[1].elapsed_time(e[2]) for e in evs]
    com_ms = [e[2].elapsed_time(e[3]) for e in evs]
    cold = cold_cache_calls(step, dev, args.cold_steps)

    copy_info = copy_calibration(dev) if args.copy_calibration else None

    tokens = int(np.sum(acc + 1))
    a_bytes, r_bytes, c_bytes = algorithmic_bytes(p, np.asarray(seq_lens0.cpu()), acc)
    a_flops = attention_flops(p, np.asarray(seq_lens0.cpu()))
    mean = lambda v: sum(v) / len(v)
    med = lambda v: sorted(v)[len(v) // 2]
    pct = lambda v, f: sorted(v)[min(len(v) - 1, int(f * len(v)))]   # p10 / p90 of the sampled calls
    attn_avg_s = mean(attn_ms) / 1e3
    rej_avg_s = mean(rej_ms) / 1e3
    com_avg_s = mean(com_ms) / 1e3
    step_s = wall / args.steps
    attn_gbs = a_bytes / attn_avg_s / 1e9
    rej_gbs = r_bytes / rej_avg_s / 1e9
    cfile = workload_counters(args.workload, args.variant)
    traffic = stored_traffic(cfile) if cfile else None
    result = dict(
        metric=METRIC, value=tokens / step_s, unit="verified tokens/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=step_s * 1e3, higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype="bf16", data="synthetic",
        config=dict(workload=(f"{args.workload}: B={B}, k={k}, Hq={p.Hq}, Hkv={p.Hkv}, D={p.D}, "
                              f"contexts {p.ctx}, block_size={p.block_size}, V={p.V}, T={p.temperature}, "
                              "one attention layer + rejection sampling + commit"),
                    global_batch=B, k=k, parallelism="none (1 GPU)"),
        roofline=dict(bound="hbm", achieved=attn_gbs, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=attn_gbs / HBM_PEAK_GBS, traffic=traffic,
                      kernel="spec_verify_attn (attn_streamk_kernel + attn_merge_kernel)",
                      algorithmic_bytes_per_call=a_bytes, avg_call_us=attn_avg_s * 1e6, calls_timed=len(evs)),
        roofline_reject=dict(bound="hbm", achieved=rej_gbs, peak=HBM_PEAK_GBS, unit="GB/s",
                             frac=rej_gbs / HBM_PEAK_GBS,
                             traffic=stored_traffic(cfile, key="reject_hbm_bytes_per_call") if cfile else None,
                             kernel="spec_reject_sample", algorithmic_bytes_per_call=r_bytes,
                             avg_call_us=rej_avg_s * 1e6, calls_timed=len(evs)),
        verified_tokens_per_step=tokens,
        mean_emitted_per_sequence=tokens / B,
        step_gbs=(a_bytes + r_bytes + c_bytes) / step_s / 1e9,
        kernels=dict(
            verify_attn=dict(avg_us=attn_avg_s * 1e6, median_us=med(attn_ms) * 1e3,
                             p10_us=pct(attn_ms, 0.1) * 1e3, p90_us=pct(attn_ms, 0.9) * 1e3, bytes=a_bytes, gbs=attn_gbs,
                             frac_of_peak=attn_gbs / HBM_PEAK_GBS,
                             mfma=dict(algorithmic_flops=a_flops, tflops=a_flops / attn_avg_s / 1e12,
                                       frac_of_bf16_peak=a_flops / attn_avg_s / 1e12 / MFMA_PEAK_BF16_TFLOPS)),
            reject_sample=dict(avg_us=rej_avg_s * 1e6, median_us=med(rej_ms) * 1e3,
                               p10_us=pct(rej_ms, 0.1) * 1e3, p90_us=pct(rej_ms, 0.9) * 1e3, bytes=r_bytes, gbs=rej_gbs,
                               frac_of_peak=rej_gbs / HBM_PEAK_GBS,
                               dense_equivalent=dense_reject_figure(p, rej_avg_s),
                               read=reject_read_figure(p.B, p.k, p.V, rej_avg_s, r_bytes)),
            commit_lengths=dict(avg_us=com_avg_s * 1e6, bytes=c_bytes)),
        event_sum_ms_per_step=(attn_avg_s + rej_avg_s + com_avg_s) * 1e3,
        event_timed_steps=len(evs),
    )
    if cold:
        cold["verify_attn"]["frac_of_peak"] = a_bytes / (cold["verify_attn"]["avg_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS
        cold["reject_sample"]["frac_of_peak"] = r_bytes / (cold["reject_sample"]["avg_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS
        result["cold_cache"] = cold
    if args.variant == "plain":
        result["config"]["workload"] = result["config"]["workload"].replace(
            "one attention layer", "k = 0 (plain decoding): one attention layer")
    if copy_info:
        result["copy_calibration"] = copy_info
    return result


def gpu_bench_sweep(args, p, dev) -> dict:
    """The shrinking active batch: the workload's seeded batch is generated once and the
    same three calls are timed on its first B sequences for each B of --sweep (the
    sequences that remain are the first B of the full batch, so every point reads a
    subset of the same pages and rows)."""
    import dataclasses
    import numpy as np
    import torch
    import speculative_decoding_verification_14_amd as sv
    from workloads import make_inputs

    sizes = [int(x) for x in args.sweep.split(",")]
    if max(sizes) > p.B or min(sizes) < 1:
        raise ValueError(f"--sweep sizes must lie in [1, {p.B}]")
    print(f"[bench] generating {args.workload} inputs (B = {p.B}, k = {p.k})", file=sys.stderr, flush=True)
    inp = make_inputs(args.workload, preset=p)

    def bf16(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)

    def t(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    kc, vc = bf16(inp["k_cache"]), bf16(inp["v_cache"])
    del inp["k_cache"], inp["v_cache"]
    k = p.k
    cap = inp["max_blocks"] * p.block_size
    stream = torch.cuda.current_stream()
    points = []
    for Bs in sizes:
        pb = dataclasses.replace(p, B=Bs)
        q = bf16(inp["q"][:Bs])
        bt = t(inp["block_table"][:Bs])
        seq_lens0 = t(inp["seq_lens"][:Bs])
        seq_lens = seq_lens0.clone()
        tl, dl = t(inp["target_logits"][:Bs]), t(inp["draft_logits"][:Bs])
        dt, sid = t(inp["draft_tokens"][:Bs]), t(inp["seq_ids"][:Bs])
        msl = int(np.max(inp["seq_lens"][:Bs])) + k + 1
        attn_out = torch.empty_like(q)
        out_tokens = torch.empty((Bs, k + 1), dtype=torch.int32, device=dev)
        num_acc = torch.empty(Bs, dtype=torch.int32, device=dev)
        out_probs = torch.empty((Bs, k + 1), dtype=torch.float32, device=dev)
        acc_probs = torch.empty((Bs, k), dtype=torch.float32, device=dev)
        overflow = torch.empty(Bs, dtype=torch.int32, device=dev)
        attn_ws = torch.zeros(max(256, sv.verify_attn_workspace_size(Bs, k, p.Hq, p.Hkv, p.D, msl)),
                              dtype=torch.uint8, device=dev)
        rej_ws = torch.zeros(sv.reject_sample_workspace_size(Bs, k, p.V), dtype=torch.uint8, device=dev)

        def step(events=None):
            seq_lens.copy_(seq_lens0)
            if events is not None:
                events[0].record(stream)
            sv.verify_attn(q, kc, vc, bt, seq_lens, attn_out, msl, None, attn_ws, stream)
            if events is not None:
                events[1].record(stream)
            sv.reject_sample(tl, dl, dt, sid, seq_lens, p.temperature, inp["seed"], out_tokens, num_acc,
                             out_probs, acc_probs, rej_ws, stream)
            if events is not None:
                events[2].record(stream)
            sv.commit_lengths(seq_lens, num_acc, k, cap, overflow, stream)
            if events is not None:
                events[3].record(stream)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        for i in range(args.steps):
            step()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - w0) / args.steps
        evs = event_steps(step, 4, args.steps)
        mean = lambda v: sum(v) / len(v)
        attn_s = mean([e[0].elapsed_time(e[1]) for e in evs.values()]) / 1e3
        rej_s = mean([e[1].elapsed_time(e[2]) for e in evs.values()]) / 1e3
        com_s = mean([e[2].elapsed_time(e[3]) for e in evs.values()]) / 1e3
        acc = num_acc.cpu().numpy()
        a_bytes, r_bytes, _ = algorithmic_bytes(pb, inp["seq_lens"][:Bs], acc)
        tokens = int(np.sum(acc + 1))
        points.append(dict(B=Bs, verified_tokens_per_s=tokens / wall, ms_per_step=wall * 1e3,
                           tokens_per_step=tokens,
                           verify_attn=dict(avg_us=attn_s * 1e6, bytes=a_bytes,
                                            frac_of_peak=a_bytes / attn_s / 1e9 / HBM_PEAK_GBS),
                           reject_sample=dict(avg_us=rej_s * 1e6, bytes=r_bytes,
                                              frac_of_peak=r_bytes / rej_s / 1e9 / HBM_PEAK_GBS,
                                              read=reject_read_figure(Bs, k, p.V, rej_s, r_bytes)),
                           commit_lengths=dict(avg_us=com_s * 1e6)))
        print(f"[bench] B={Bs}: {tokens / wall:.0f} tokens/s, attn {attn_s * 1e6:.1f} us, "
              f"reject {rej_s * 1e6:.1f} us", file=sys.stderr, flush=True)
        del q, bt, seq_lens0, seq_lens, tl, dl, dt, sid, attn_out, attn_ws, rej_ws
    return dict(metric="verified tokens/s per batch size (shrinking active batch)", unit="verified tokens/s",
                n_gpus=1, steps=args.steps, warmup=args.warmup, higher_is_better=True, dtype="bf16",
                data="synthetic",
                config=dict(workload=(f"{args.workload}: first B of a seeded batch of {p.B}, k={k}, Hq={p.Hq}, "
                                      f"Hkv={p.Hkv}, D={p.D}, contexts {p.ctx}, block_size={p.block_size}, V={p.V}, "
                                      "one attention layer + rejection sampling + commit")),
                sweep=points)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="8b")
    ap.add_argument("--variant", choices=["uniform", "plain", "ragged", "tree", "fused"], default="uniform")
    ap.add_argument("--tree", default="2,2", metavar="T,D",
                    help="tree variant: branching factor and depth of the full draft tree")
    ap.add_argument("--sweep", metavar="B1,B2,...",
                    help="time the step on the first B sequences of the workload's batch for each B")
    ap.add_argument("--cold-steps", type=int, default=30,
                    help="steps timed per call after a cache-evicting write (0: skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-baseline-only", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-rocprof", metavar="DIR")
    ap.add_argument("--out", metavar="FILE")
    ap.add_argument("--command", default="", help="command line recorded in a rocprof summary")
    ap.add_argument("--write-counters", action="store_true")
    ap.add_argument("--write-mfma", metavar="PMC_DIR",
                    help="write the attention's MFMA counter summary from a rocprofv3 run in PMC_DIR")
    ap.add_argument("--write-clock", metavar="PMC_DIR",
                    help="summarise a rocprofv3 run with GRBM_GUI_ACTIVE and GRBM_COUNT: shader clock per kernel")
    ap.add_argument("--counters-kind", choices=["attn", "lm"], default="attn")
    ap.add_argument("--fetch-dir")
    ap.add_argument("--write-dir")
    ap.add_argument("--fetch-command", default="")
    ap.add_argument("--counters-title", default="", help="workload named in a counter summary's first line")
    ap.add_argument("--write-command", default="")
    args = ap.parse_args()

    if args.write_mfma:
        write_mfma(args.write_mfma, args.out or MFMA_FILE, args.command)
        return

    if args.write_clock:
        write_clock(args.write_clock, args.out or "/dev/stdout", args.command, args.counters_title or args.workload)
        return

    if args.write_counters:
        write_counters(args.fetch_dir, args.write_dir,
                       args.out or (LM_COUNTERS_FILE if args.counters_kind == "lm" else COUNTERS_FILE),
                       args.fetch_command, args.write_command, args.counters_kind, args.counters_title)
        return

    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof, args.out or "/dev/stdout", args.command)
        return
    if args.cpu_baseline_only:
        print(json.dumps(cpu_baseline(args.workload)))
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the verify step is data parallel over sequences, one GPU's share is measured here)",
              file=sys.stderr)
        sys.exit(2)

    result = gpu_bench(args)
    if not args.no_cpu_baseline and args.variant == "uniform" and not args.sweep:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        cb = run_cpu_baseline_child(args.workload)
        if cb is not None:
            result["cpu_baseline"] = dict(value=cb["pooled"]["tokens_per_s"], unit="verified tokens/s",
                                          cores=cb["workers"], kind="oracle", sample=cb["sample"],
                                          seconds_per_step=cb["pooled"]["seconds_per_step"],
                                          single_core=dict(value=cb["single"]["tokens_per_s"], cores=1,
                                                           seconds_per_step=cb["single"]["seconds_per_step"]),
                                          cpu=_cpu_model())
    print(json.dumps(result))


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()

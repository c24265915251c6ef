"""Decode-step benchmark of the ShadowKV sparse-KV decode on one MI355X.

python bench.py [--gpus 1] [--steps 60] [--warmup 4] [--shape llama3_8b_122k]

One step = one ShadowKV decode step (landmark scoring + top-K + index scan, key
rebuild of the misses, sparse attention) through every layer of the model
shape, i.e. one new token for each of the `batch` sequences.  Inputs are the
seeded synthetic caches of sparse_kv_cache_decode_amd.synth, already resident in
HBM when the timed region starts; queries drift as AR(1) so the temporal cache
sees hits.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
CALIB_BYTES = 512 << 20         # bytes read (and written) once by the counter-calibration kernel
CSRC = os.path.join(ROOT, "sparse_kv_cache_decode_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
SCORE_KERNELS = {"bf16": "skv::score_kernel<{G}>", "e5m2": "skv::score_fp8_kernel<{G}>"}


def score_kernel_name(shape) -> str:
    """The score kernel the library launches for this shape (templated on G)."""
    return SCORE_KERNELS[shape.landmark_format].format(G=shape.group)
FORMAT_BYTES = {"bf16": 2, "e5m2": 1}
METRIC = "decode tokens/s at S=122K batch 8 (Llama-3.1-8B shape); % HBM roofline"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# CPU baseline: the oracle, timed on the host cores, on a bounded sample


def cpu_baseline_child(shape_name: str, seed: int, min_seconds: float):
    """Child process: build the oracle for layer 0 / batch element 0, say 'ready',
    wait for 'go' on stdin, then time oracle decode steps for >= min_seconds."""
    import numpy as np
    import threadpoolctl
    import torch

    from oracle import shadowkv as O
    from sparse_kv_cache_decode_amd import synth

    shape = synth.SHAPES[shape_name].replace(batch=1)
    t0 = time.time()
    k, v = synth.layer_cache_np(shape, 0, seed)
    q = synth.queries_np(shape, k, 0, 64, seed)
    kb = k.view(torch.int16).numpy().view(np.uint16)
    vb = v.view(torch.int16).numpy().view(np.uint16)
    st = O.build(O.config_from(shape), kb, vb)
    qb = q.view(torch.int16).numpy().view(np.uint16)
    print(json.dumps({"ready": True, "prep_s": time.time() - t0}), flush=True)
    sys.stdin.readline()
    threads = max(i["num_threads"] for i in threadpoolctl.threadpool_info()) \
        if threadpoolctl.threadpool_info() else 1
    prev, n, t_start = None, 0, time.perf_counter()
    while True:
        res = O.decode_step(st, qb[n % 64], prev)
        prev = res.ids
        n += 1
        el = time.perf_counter() - t_start
        if el >= min_seconds and n >= 4:
            break
    print(json.dumps({"steps": n, "seconds": el, "threads": threads,
                      "affinity": len(os.sched_getaffinity(0))}), flush=True)


def start_cpu_baseline(shape_name, seed, min_seconds):
    cmd = [sys.executable, os.path.abspath(__file__), "--cpu-baseline-child", "--shape", shape_name,
           "--seed", str(seed), "--cpu-seconds", str(min_seconds)]
    return subprocess.Popen(cmd, stdin=subprocess.PIPE, stdout=subprocess.PIPE, text=True, cwd=ROOT)


# ----------------------------------------------------------------------------
# HBM traffic from rocprofv3 counters (FETCH_SIZE and WRITE_SIZE, KiB per dispatch),
# scaled by what the same counters read for a streaming kernel of known size.


def kernel_source_digest() -> str:
    """Digest of every native source: traffic figures taken from an older build
    than the one being timed are not reported."""
    h = hashlib.sha256()
    for n in sorted(os.listdir(CSRC)):
        if n.endswith((".hip", ".h", ".cpp")):
            h.update(n.encode())
            with open(os.path.join(CSRC, n), "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def calibration_copy():
    """Elementwise float32 multiply over CALIB_BYTES: reads and writes each byte once.
    Runs outside the timed region; only its counter readings are used."""
    import torch
    src = torch.full((CALIB_BYTES // 4,), 1.0, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()


def _short_kernel_name(name: str) -> str:
    name = name.strip()
    if name.startswith("void "):
        name = name[5:]
    depth, end = 0, len(name)
    for i, ch in enumerate(name):        # cut the argument list, keep template arguments
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            end = i
            break
    return name[:end]


def _counter_rows(path: str, counter: str) -> list:
    """(dispatch id, short kernel name, value) of every dispatch, in dispatch order."""
    rows = []
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") == counter:
                rows.append((int(row["Dispatch_Id"]), _short_kernel_name(row["Kernel_Name"]),
                             float(row["Counter_Value"])))
    return sorted(rows)


def _means(rows: list) -> dict:
    acc = {}
    for _, k, v in rows:
        s, n = acc.get(k, (0.0, 0))
        acc[k] = (s + v, n + 1)
    return {k: (s / n, n) for k, (s, n) in acc.items()}


def _calibration(rows: list):
    """The calibration kernel is the last three dispatches of the run."""
    last = rows[-3:]
    names = {k for _, k, _ in last}
    assert len(last) == 3 and len(names) == 1 and "MulFunctor<float>" in next(iter(names)), names
    return next(iter(names)), sum(v for _, _, v in last) / 3.0


def summarize_counters(fetch_csv: str, write_csv: str, command: str) -> str:
    """Markdown summary (with a JSON block that bench.py reads back) of two
    rocprofv3 --pmc runs of `command`, one with FETCH_SIZE and one with WRITE_SIZE."""
    fr, wr = _counter_rows(fetch_csv, "FETCH_SIZE"), _counter_rows(write_csv, "WRITE_SIZE")
    fetch, write = _means(fr), _means(wr)
    calib, cf = _calibration(fr)
    _, cw = _calibration(wr)
    f_fac = CALIB_BYTES / (cf * 1024.0)
    w_fac = CALIB_BYTES / (cw * 1024.0)
    kernels = {}
    for k in sorted(fetch):
        if not k.startswith("skv::") or k not in write:
            continue
        fb, wb = fetch[k][0] * 1024.0 * f_fac, write[k][0] * 1024.0 * w_fac
        kernels[k] = {"dispatches": fetch[k][1], "fetch_kib": round(fetch[k][0], 1),
                      "write_kib": round(write[k][0], 1), "hbm_read_bytes": int(fb),
                      "hbm_write_bytes": int(wb), "hbm_bytes_per_launch": int(fb + wb)}
    blob = {"workload": "llama3_8b_122k", "kernel_source_digest": kernel_source_digest(),
            "calibration_bytes": CALIB_BYTES, "fetch_factor": round(f_fac, 4),
            "write_factor": round(w_fac, 4), "kernels": kernels}
    lines = ["# HBM traffic per kernel launch: ShadowKV decode, Llama-3.1-8B shape (122 880 tokens, batch 8)",
             "", "Commands (repository root on the MI355X host, `export TMPDIR=/tmp` first):", "", "```"]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        lines.append(f"rocprofv3 --pmc {c} --output-format csv -d /tmp/pmc_{c.lower()} -o pmc -- {command}")
    lines += ["```", "",
              f"Scaling: the calibration kernel (`{calib}`, the run's last three dispatches) reads and "
              f"writes {CALIB_BYTES} bytes; FETCH_SIZE reads {cf:.0f} KiB and WRITE_SIZE {cw:.0f} KiB for it, "
              f"so bytes = KiB x 1024 x {f_fac:.4f} (reads) and x {w_fac:.4f} (writes).", "",
              "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB | HBM write MB |",
              "|---|---|---|---|---|---|"]
    for k, v in kernels.items():
        lines.append(f"| `{k}` | {v['dispatches']} | {v['fetch_kib']} | {v['write_kib']} | "
                     f"{v['hbm_read_bytes'] / 1e6:.1f} | {v['hbm_write_bytes'] / 1e6:.1f} |")
    lines += ["", "Read back by bench.py (used only while the native sources hash to the digest):", "",
              "```json", json.dumps(blob, indent=1), "```", ""]
    return "\n".join(lines)


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE")
SIMDS = 256 * 4          # 256 CUs of 4 SIMDs
XCDS = 8                 # GRBM_GUI_ACTIVE per dispatch comes summed over the 8 XCDs
MFMA_BF16_PEAK_TFLOPS = 2500.0


def summarize_mfma(pmc_csv: str, stats_csv: str, command: str) -> str:
    """Markdown summary of one rocprofv3 --pmc run with MFMA_COUNTERS (per-dispatch
    means per kernel), with the kernels' mean durations from a kernel-trace run of
    the same command: MFMA busy fraction = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE
    / XCDS x SIMDs) (the per-dispatch GRBM_GUI_ACTIVE is the sum of the XCDs' busy
    cycles: about 8 x 2.3 cycles per ns on long kernels), bf16 MFMA rate =
    SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 flops / duration."""
    vals = {}
    with open(pmc_csv, newline="") as f:
        for row in csv.DictReader(f):
            c = row.get("Counter_Name")
            if c in MFMA_COUNTERS:
                k = _short_kernel_name(row["Kernel_Name"])
                vals.setdefault(k, {}).setdefault(c, []).append(float(row["Counter_Value"]))
    dur = {}
    with open(stats_csv, newline="") as f:
        for row in csv.DictReader(f):
            dur[_short_kernel_name(row["Name"])] = float(row["AverageNs"]) / 1e3
    lines = ["# MFMA counters per kernel launch: ShadowKV decode", "",
             "Commands (repository root on the MI355X host, `export TMPDIR=/tmp` first):", "", "```",
             f"rocprofv3 --pmc {' '.join(MFMA_COUNTERS)} --output-format csv -d /tmp/pmc_mfma -o pmc -- {command}",
             f"rocprofv3 --kernel-trace --stats --output-format csv -d /tmp/prof_mfma -o bench -- {command}",
             "```", "",
             f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {XCDS} x {SIMDS} SIMDs), the "
             f"dispatch's GRBM_GUI_ACTIVE being the sum over the {XCDS} XCDs; bf16 rate = "
             f"SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / mean duration (kernel trace), against "
             f"{MFMA_BF16_PEAK_TFLOPS:.0f} TFLOP/s dense bf16.", "",
             "| kernel | dispatches | MFMA busy | bf16 MFMA GFLOP per launch | mean us | bf16 TFLOP/s | of peak |",
             "|---|---|---|---|---|---|---|"]
    blob = {}
    for k in sorted(vals):
        if not k.startswith("skv::"):
            continue
        v = {c: sum(x) / len(x) for c, x in vals[k].items()}
        if not all(c in v for c in MFMA_COUNTERS):
            continue
        busy = v["SQ_VALU_MFMA_BUSY_CYCLES"] / max(1.0, v["GRBM_GUI_ACTIVE"] / XCDS * SIMDS)
        gflop = v["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / 1e9
        us = dur.get(k)
        rate = gflop / (us * 1e-6) / 1e3 if us else None
        n = len(vals[k]["GRBM_GUI_ACTIVE"])
        lines.append(f"| `{k}` | {n} | {busy:.4f} | {gflop:.3f} | {us if us is not None else float('nan'):.2f} | "
                     f"{rate if rate is not None else float('nan'):.1f} | "
                     f"{(rate or 0) / MFMA_BF16_PEAK_TFLOPS:.4f} |")
        blob[k] = {"mfma_busy": round(busy, 5), "bf16_gflop_per_launch": round(gflop, 4), "mean_us": us,
                   "bf16_tflops": round(rate, 2) if rate else None}
    lines += ["", "```json", json.dumps({"kernel_source_digest": kernel_source_digest(), "kernels": blob}, indent=1),
              "```", ""]
    return "\n".join(lines)


def summarize_overlap(trace_csv: str, command: str) -> str:
    """Markdown summary of how the host-value gather (side stream) overlaps the
    main stream's kernels, from a rocprofv3 --kernel-trace kernel_trace.csv: per
    decode step and layer, the gather's span against the rebuild that runs beside
    it and the attention that waits for it."""
    rows = []
    with open(trace_csv, newline="") as f:
        for row in csv.DictReader(f):
            name = _short_kernel_name(row["Kernel_Name"])
            if name.startswith("skv::"):
                rows.append((int(row["Start_Timestamp"]), int(row["End_Timestamp"]), name))
    rows.sort()
    spans = []   # (gather, rebuild, attention) per step: the gather and the main-stream kernels around it
    last_rebuild = None
    pending = None
    for st, en, name in rows:
        if name.startswith("skv::rebuild_kernel"):
            last_rebuild = (st, en)
            if pending is not None and pending[2] is None:
                pending[2] = (st, en)
        elif name == "skv::value_gather_kernel":
            pending = [(st, en), None, None]
            if last_rebuild and last_rebuild[1] > st:
                pending[2] = last_rebuild
        elif name.startswith("skv::attn_kernel") and pending is not None:
            pending[1] = (st, en)
            if pending[2] is not None:
                spans.append(tuple(pending))
            pending = None
    if not spans:
        return "no gather / rebuild / attention triples found\n"
    ov, gap, gat, reb = [], [], [], []
    for (gs, ge), (as_, ae), (rs, re) in spans:
        gat.append((ge - gs) / 1e3)
        reb.append((re - rs) / 1e3)
        ov.append(max(0, min(ge, re) - max(gs, rs)) / 1e3)
        gap.append((as_ - ge) / 1e3)
    med = lambda v: sorted(v)[len(v) // 2]
    lines = ["# Side-stream overlap: host-value gather beside the key rebuild (Llama-3.1-8B shape, values in pinned host memory)",
             "", "Command (repository root on the MI355X host, `export TMPDIR=/tmp` first):", "", "```",
             f"rocprofv3 --kernel-trace --output-format csv -d /tmp/trace_overlap -o bench -- {command}", "```", "",
             "From `bench_kernel_trace.csv`: for every decode step of every layer, the zero-copy gather of the missed",
             "chunks' values (`value_gather_kernel`, side stream) against the key rebuild of the same step",
             "(`rebuild_kernel`, decode stream) and the attention (`attn_kernel`), which waits for the gather.", "",
             f"| steps x layers | gather us (median) | rebuild us (median) | rebuild time inside the gather (median) | attention start after gather end, us (median) |",
             "|---|---|---|---|---|",
             f"| {len(spans)} | {med(gat):.1f} | {med(reb):.1f} | {med(ov):.1f} ({100 * med(ov) / max(1e-9, med(reb)):.0f} % of the rebuild) | {med(gap):.1f} |",
             ""]
    return "\n".join(lines)


def summarize_trace(stats_csv: str, command: str, shape=None) -> str:
    """Markdown table of the library's kernels from a rocprofv3 kernel_stats.csv,
    with the score kernel's rate at its algorithmic bytes per launch for `shape`
    (default: the Llama-3.1-8B shape)."""
    from sparse_kv_cache_decode_amd import synth
    shape = shape or synth.SHAPES["llama3_8b_122k"]
    rows = []
    with open(stats_csv, newline="") as f:
        for row in csv.DictReader(f):
            name = _short_kernel_name(row["Name"])
            if name.startswith("skv::"):
                rows.append((name, int(row["Calls"]), float(row["AverageNs"]) / 1e3, float(row["MinNs"]) / 1e3,
                             float(row["MaxNs"]) / 1e3, float(row["TotalDurationNs"]) / 1e6))
    rows.sort(key=lambda r: -r[5])
    lines = [f"# Kernel timing: ShadowKV decode, {shape.name} (S = {shape.seq_len}, batch {shape.batch}, "
             f"G = {shape.group}, C = {shape.chunk}, K = {shape.top_k}, {shape.layers} layers)", "",
             "Command (repository root on the MI355X host, `export TMPDIR=/tmp` first):", "", "```",
             f"rocprofv3 --kernel-trace --stats --output-format csv -d /tmp/prof_bench -o bench -- {command}",
             "```", "",
             "Per-kernel summary from `bench_kernel_stats.csv` (library kernels only). The build kernels run "
             "once per layer; the decode kernels once per layer and step (warm-up, timed and phase-timing steps).",
             "", "| kernel | calls | avg us | min us | max us | total ms |", "|---|---|---|---|---|---|"]
    for n, c, a, lo, hi, t in rows:
        lines.append(f"| `{n}` | {c} | {a:.2f} | {lo:.2f} | {hi:.2f} | {t:.1f} |")
    for fmt in SCORE_KERNELS:
        fshape = shape.replace(landmark_format=fmt)
        score = [r for r in rows if r[0] == score_kernel_name(fshape)]
        if score:
            by = algorithmic_bytes(fshape, 0.0)["score"]
            lines += ["", f"Score kernel ({fmt} landmarks): {by} algorithmic bytes per launch / {score[0][2]:.2f} us "
                          f"average = {by / (score[0][2] * 1e-6) / 1e9:.0f} GB/s "
                          f"({by / (score[0][2] * 1e-6) / 1e9 / HBM_PEAK_GBPS:.3f} of {HBM_PEAK_GBPS / 1000:.0f} TB/s)."]
    return "\n".join(lines) + "\n"


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None
    when there is none for this workload or the sources have changed since."""
    for path in sorted(glob.glob(os.path.join(PROFILES, "*_hbm_traffic.md"))):
        try:
            text = open(path).read()
            blob = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
        except (OSError, IndexError, ValueError):
            continue
        if blob.get("workload") != workload or blob.get("kernel_source_digest") != kernel_source_digest():
            continue
        k = blob.get("kernels", {}).get(kernel)
        if k:
            return k["hbm_bytes_per_launch"]
    return None


def measure_h2d_gbps(nbytes: int = 256 << 20, reps: int = 8) -> float:
    """Pinned host -> device copy rate (the PCIe ceiling for host-resident values)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    rate = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return rate


# ----------------------------------------------------------------------------


def algorithmic_bytes(shape, rebuilt_per_layer_step: float, fused: bool = False, temporal: bool = True) -> dict:
    """Bytes the method must move per layer-step (HBM-resident values), given the
    chunks rebuilt per layer-step (the misses with the temporal cache, every
    selected chunk without it):
    - score: the candidates' landmarks and the queries;
    - rebuild: the rebuilt chunks' rows of A, B once per pair, and the rebuilt keys
      written to their slots (kept for later hits, or handed to a separate attention
      launch; a fused rebuild without the temporal cache writes none);
    - attention: the values of every attended token, the keys of every attended
      token that is read from memory (a fused rebuild attends its rebuilt keys where
      it made them), and the output."""
    d, C, r = shape.head_dim, shape.chunk, shape.rank
    P = shape.pairs
    landmarks = P * shape.n_cand * d * FORMAT_BYTES[shape.landmark_format]
    q_bytes = shape.batch * shape.n_q_heads * d * 2
    out_bytes = shape.batch * shape.n_q_heads * d * 4
    slot_writes = rebuilt_per_layer_step * C * d * 2 if (temporal or not fused) else 0.0
    rebuild = rebuilt_per_layer_step * C * r * FORMAT_BYTES[shape.a_format] + slot_writes + \
        P * r * d * FORMAT_BYTES[shape.b_format]
    tokens = P * shape.tokens_attended
    key_tokens = tokens - (rebuilt_per_layer_step * C if fused else 0.0)
    attn = tokens * d * 2 + key_tokens * d * 2
    return {"score": landmarks + q_bytes, "rebuild": rebuild, "attention": attn + out_bytes,
            "total": landmarks + q_bytes + rebuild + attn + out_bytes}


def phase_rates(by: dict, phase_us: dict) -> dict:
    """Achieved rate of each phase at its algorithmic bytes (GB/s, and the fraction
    of the HBM peak): scoring; the tail (key rebuild and attention, with the merge
    of the partials: one fused launch plus the merge, or the rebuild, attention and
    merge launches)."""
    tail_us = phase_us["rebuild"] + phase_us["attention"]
    out = {}
    for name, b, us in (("score", by["score"], phase_us["score"]),
                        ("rebuild_attention_merge", by["rebuild"] + by["attention"], tail_us)):
        if us > 0:
            g = b / (us * 1e-6) / 1e9
            out[name] = {"achieved_GBps": round(g, 1), "frac": round(g / HBM_PEAK_GBPS, 4), "us": round(us, 2)}
    out["select"] = {"us": round(phase_us["select"], 2), "note": "latency-bound: logits are scratch, not counted"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--shape", default="llama3_8b_122k")
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (0 = model's)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--values", choices=["hbm", "host"], default="hbm",
                    help="value store in HBM or in pinned host memory (gathered over PCIe)")
    ap.add_argument("--queries", choices=["drift", "independent"], default="drift",
                    help="AR(1)-drifting queries (temporal cache hits) or independent draws")
    ap.add_argument("--chunk", type=int, default=0,
                    help="chunk size C for the 1M-token shape (budget K and O follow C)")
    ap.add_argument("--append", choices=["none", "exact", "lowrank"], default="none",
                    help="append one generated token per layer before every decode step "
                         "(exact keys, or ShadowKV+ low-rank states)")
    ap.add_argument("--landmarks", choices=["bf16", "e5m2"], default="bf16",
                    help="landmark storage: bf16 (the pages' precision) or FP8 E5M2 (their precision study)")
    ap.add_argument("--a-format", choices=["bf16", "e5m2"], default="bf16",
                    help="storage of the rows of A: bf16 (the pages' precision) or FP8 E5M2")
    ap.add_argument("--b-format", choices=["bf16", "e5m2"], default="bf16",
                    help="storage of B (Psi^T): bf16 (the pages' precision) or FP8 E5M2")
    ap.add_argument("--rebuild", choices=["auto", "fused", "separate", "overlap"], default="auto",
                    help="missed chunks rebuilt and attended in one launch with the rest of the attention "
                         "(fused; auto with values in HBM) or rebuilt by their own launch before it (separate)")
    ap.add_argument("--select", choices=["auto", "full"], default="auto",
                    help="top-K selection: the library's choice, or a pass over every candidate's score")
    ap.add_argument("--temporal", choices=["on", "off"], default="on",
                    help="temporal cache on (rebuild only the chunks missed against the previous step) or off "
                         "(rebuild every selected chunk; with the fused rebuild, no key slot cache at all)")
    ap.add_argument("--graph", choices=["on", "off"], default="off",
                    help="replay each timed step (all layers) as one captured HIP graph; off: launch eagerly")
    ap.add_argument("--phase-steps", type=int, default=16,
                    help="eager steps after the timed region that record per-phase events on sampled layers")
    ap.add_argument("--phase-every", type=int, default=1,
                    help="record per-phase HIP events on every n-th layer during the phase-timing steps "
                         "(an event record between kernels costs a few microseconds)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calib-copy", action="store_true",
                    help="after the timed region, run a known-size streaming kernel for counter scaling")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "COMMAND"),
                    help="print the traffic summary of two rocprofv3 --pmc runs (no GPU needed)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("STATS_CSV", "COMMAND"),
                    help="print the per-kernel summary of a rocprofv3 --kernel-trace --stats run (no GPU needed)")
    ap.add_argument("--summarize-overlap", nargs=2, metavar=("TRACE_CSV", "COMMAND"),
                    help="print the side-stream overlap of a rocprofv3 --kernel-trace run (no GPU needed)")
    ap.add_argument("--summarize-mfma", nargs=3, metavar=("PMC_CSV", "STATS_CSV", "COMMAND"),
                    help="print the MFMA counter summary of a rocprofv3 --pmc run (no GPU needed)")
    ap.add_argument("--cpu-baseline-child", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()

    if args.summarize_counters:
        print(summarize_counters(*args.summarize_counters))
        return 0
    if args.summarize_overlap:
        print(summarize_overlap(*args.summarize_overlap))
        return 0
    if args.summarize_mfma:
        print(summarize_mfma(*args.summarize_mfma))
        return 0
    if args.summarize_trace:
        from sparse_kv_cache_decode_amd import synth
        tshape = synth.glm_chunk_variant(args.chunk) if args.chunk else synth.SHAPES[args.shape]
        print(summarize_trace(*args.summarize_trace, tshape.replace(layers=args.layers or tshape.layers)))
        return 0

    if args.cpu_baseline_child:
        cpu_baseline_child(args.shape, args.seed, args.cpu_seconds)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode step shards by batch element with no communication)",
              file=sys.stderr)
        return 2

    # the oracle child starts before this process touches the GPU
    child = None if args.no_cpu_baseline else start_cpu_baseline(args.shape, args.seed, args.cpu_seconds)

    import torch

    from sparse_kv_cache_decode_amd import skv, synth

    shape = synth.glm_chunk_variant(args.chunk) if args.chunk else synth.SHAPES[args.shape]
    if args.chunk and not args.shape.startswith("glm4"):
        print("--chunk applies to the 1M-token shape only", file=sys.stderr)
        return 2
    if args.layers:
        shape = shape.replace(layers=args.layers)
    if args.landmarks != "bf16" or args.a_format != "bf16" or args.b_format != "bf16":
        shape = shape.replace(landmark_format=args.landmarks, a_format=args.a_format, b_format=args.b_format)
    L, W, K = shape.layers, args.warmup, args.steps
    PH = max(1, args.phase_steps)
    total = W + K + PH            # warm-up, timed and phase-timing steps
    dev = torch.device("cuda")
    torch.cuda.init()
    skv.lib()
    layers, qs = [], []
    t0 = time.time()
    host = args.values == "host"
    placement = skv.SKV_VALUES_HOST if host else skv.SKV_VALUES_DEVICE
    pcie_peak = measure_h2d_gbps()     # before the value stores take pinned memory
    new_mode = {"exact": skv.SKV_NEW_EXACT, "lowrank": skv.SKV_NEW_LOWRANK}.get(args.append)
    news = []
    build_s = []       # wall time of each layer's skv_build (pre-fill factorisation and caches)
    for l in range(L):
        k_pre, v = synth.layer_cache_torch(shape, l, args.seed, dev)
        if host:
            vh = torch.empty(v.shape, dtype=v.dtype, pin_memory=True)
            vh.copy_(v)
            del v
            v = vh
        torch.cuda.synchronize()
        tb = time.perf_counter()
        rb = skv.REBUILD_MODES[args.rebuild]
        tc = 1 if args.temporal == "on" else 0
        sm = skv.SELECT_MODES[args.select]
        if new_mode is None:
            layers.append(skv.Layer(shape, k_pre, v, placement, tc, rebuild_mode=rb, select_mode=sm))
        else:
            layers.append(skv.Layer(shape, k_pre, v, placement, tc, max_new_tokens=total, new_token_mode=new_mode,
                                    rebuild_mode=rb, select_mode=sm))
        torch.cuda.synchronize()
        build_s.append(time.perf_counter() - tb)
        if new_mode is not None:
            news.append(synth.continuation_torch(shape, l, total, args.seed, dev))
        qs.append(synth.queries_torch(shape, k_pre, l, total, args.seed, mode=args.queries))
        del k_pre, v
        if l % 4 == 3 or l == L - 1:
            log(f"built layer {l + 1}/{L} ({time.time() - t0:.1f}s)")
    # queries step-major, so that one step's queries of every layer are one block
    qall = torch.stack([torch.stack([qs[l][t] for l in range(L)]) for t in range(total)])
    del qs
    torch.cuda.synchronize()
    out = torch.empty((shape.batch, shape.n_q_heads, shape.head_dim), dtype=torch.float32, device=dev)
    ids = torch.empty((shape.batch, shape.n_kv_heads, shape.top_k), dtype=torch.int32, device=dev)
    qbuf = torch.empty_like(qall[0])
    stream = torch.cuda.current_stream()

    def step_layers(q, t, st):
        for l in range(L):
            if news:
                layers[l].append(news[l][0][t], news[l][1][t], st)
            layers[l].decode(q[l], out, ids, st)

    for t in range(W):
        step_layers(qall[t], t, stream)
    torch.cuda.synchronize()
    graph = None
    if args.graph == "on" and not news:
        # the step reads its queries from qbuf; capture launches nothing
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step_layers(qbuf, 0, None)
        torch.cuda.synchronize()
    before = [ly.stats() for ly in layers]
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for t in range(W, W + K):
        if graph is not None:
            qbuf.copy_(qall[t])
            graph.replay()
        else:
            step_layers(qall[t], t, stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    log(f"timed {K} steps x {L} layers: {ms_total:.2f} ms ({'graph replay' if graph else 'eager launches'})")
    after = [ly.stats() for ly in layers]

    # per-phase device timing: eager steps after the timed region, events on the
    # sampled layers (which then run their phases back to back, as one pair group)
    sampled = list(range(0, L, max(1, args.phase_every)))
    for l in sampled:
        skv.skv_set_timing(layers[l].h, PH)
    for t in range(W + K, total):
        step_layers(qall[t], t, stream)
    torch.cuda.synchronize()
    phase_ms = {p: 0.0 for p in skv.PHASES}
    for l in sampled:
        ph, n = skv.skv_get_timing(layers[l].h)
        assert n == PH
        for p in ph:
            phase_ms[p] += ph[p]
    launches = K * L
    phase_avg_us = {p: 1000.0 * phase_ms[p] / (PH * len(sampled)) for p in phase_ms}
    misses = sum(a["total_misses"] - b["total_misses"] for a, b in zip(after, before)) / launches
    hits = sum(a["total_hits"] - b["total_hits"] for a, b in zip(after, before)) / launches
    alpha_timed = hits / (shape.pairs * shape.top_k)
    # hits over steps 1.. of the warm-up and timed steps (device counters)
    alpha_all = sum(a["total_hits"] for a in after) / (L * shape.pairs * shape.top_k * (W + K - 1))
    # chunks rebuilt per layer-step: the misses, or every selected chunk without
    # the temporal cache (whose hit / miss counters then stay at zero)
    rebuilt = misses if args.temporal == "on" else float(shape.pairs * shape.top_k)
    fused = (args.rebuild if args.rebuild != "auto" else ("separate" if host else "fused")) == "fused"
    by = algorithmic_bytes(shape, rebuilt, fused=fused, temporal=args.temporal == "on")

    ms_per_step = ms_total / K
    tok_s = shape.batch * K / (ms_total / 1000.0)
    layer_us = 1000.0 * ms_per_step / L
    step_gbps = by["total"] / (layer_us * 1e-6) / 1e9
    score_gbps = by["score"] / (phase_avg_us["score"] * 1e-6) / 1e9
    # the pages' equivalent bandwidth: with values in HBM the PCIe term is absent and
    # alpha does not enter; with the measured alpha and a PCIe rate (the gather's own
    # with host values, else the pinned host->device copy rate measured here) it is
    # what the formula gives for host-resident values.  Also the dense-attention
    # bytes per measured layer time.
    S, C, Kc, Oc = shape.seq_len, shape.chunk, shape.top_k, shape.n_outlier

    def b_tilde(b_pcie):
        pcie_term = (1 - alpha_timed) * Kc * C * HBM_PEAK_GBPS / b_pcie if b_pcie else 0.0
        return 2 * S * HBM_PEAK_GBPS / (S / C + 2 * (Kc + Oc) * C + pcie_term) / 1000.0

    pcie = None
    pcie_gbps = None
    if host:
        host_bytes = misses * C * shape.head_dim * 2          # values of the missed chunks
        gather_us = phase_avg_us["value_gather"]
        pcie_gbps = host_bytes / (gather_us * 1e-6) / 1e9 if gather_us > 0 else None
        pcie = {"host_bytes_per_layer_step": int(host_bytes), "gather_us_per_layer": round(gather_us, 2),
                "achieved_GBps": round(pcie_gbps, 2) if pcie_gbps else None,
                "pinned_h2d_peak_GBps": round(pcie_peak, 2),
                "frac_of_peak": round(pcie_gbps / pcie_peak, 4) if pcie_gbps else None}
    dense_bytes = 2 * S * shape.head_dim * 2 * shape.pairs
    bt_measured = dense_bytes / (layer_us * 1e-6) / 1e12

    cpu = None
    if child is not None:
        line = child.stdout.readline()
        ready = json.loads(line) if line else None
        if ready:
            child.stdin.write("go\n")
            child.stdin.flush()
            res = json.loads(child.stdout.readline())
            child.wait(timeout=600)
            t_step = res["seconds"] / res["steps"]     # one layer, one batch element
            cpu = {"value": 1.0 / (L * t_step), "unit": "tokens/s", "cores": res["threads"],
                   "kind": "oracle",
                   "sample": f"layer 0, batch element 0 of {shape.name} ({shape.pairs // shape.batch} KV heads, "
                             f"S={shape.seq_len}), {res['steps']} drifting decode steps in {res['seconds']:.1f}s "
                             f"(float64 NumPy, {res['threads']} BLAS threads, {res['affinity']} cores in affinity); "
                             f"tokens/s = batch / (batch * layers * t_step) = 1/(layers * t_step); build untimed"}
        else:
            log("cpu baseline child failed")

    rec = {
        "metric": METRIC,
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" + ("" if shape.landmark_format == "bf16" else ", e5m2 landmarks (fp16 MFMA scoring)")
                 + ("" if shape.a_format == "bf16" else ", e5m2 rows of A (widened to bf16 for the rebuild)")
                 + ("" if shape.b_format == "bf16" else ", e5m2 B (widened to bf16 for the rebuild)"),
        "data": "synthetic",
        "config": {"workload": f"{shape.name}: {L} layers, batch {shape.batch}, S={shape.seq_len}, "
                               f"{shape.n_q_heads} q / {shape.n_kv_heads} KV heads, d={shape.head_dim}, "
                               f"r={shape.rank}, C={shape.chunk}, K={shape.top_k}, O={shape.n_outlier}, "
                               f"window {shape.window}, {shape.landmark_format} landmarks, "
                               f"{shape.a_format} A, {shape.b_format} B, "
                               f"values in {'pinned host memory' if host else 'HBM'}, "
                               f"{'AR(1)-drifting' if args.queries == 'drift' else 'independent'} queries"
                               + ("" if new_mode is None else
                                  f", one generated token appended per layer and step ({args.append} keys; "
                                  f"{W + 1}..{W + K} generated tokens attended in the timed steps)"),
                   "global_batch": shape.batch, "seq_len": shape.seq_len, "layers": L,
                   "parallelism": "single GPU"},
        "roofline_reading": "roofline: the dominant kernel (landmark scoring) alone; the target (>= 0.60 of "
                            "HBM roofline for the sparse-attention step) is step_roofline.frac: every kernel's "
                            "algorithmic bytes over the measured layer time",
        "roofline": {"bound": "hbm", "kernel": f"{score_kernel_name(shape)} (landmark GEMV)",
                     "achieved": round(score_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(score_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(shape.name, score_kernel_name(shape)),
                     "algorithmic_bytes": int(by["score"])},
        "step_roofline": {"algorithmic_bytes_per_layer_step": int(by["total"]),
                          "achieved_GBps": round(step_gbps, 1),
                          "frac": round(step_gbps / HBM_PEAK_GBPS, 4), "target": 0.60,
                          "meets_target": step_gbps / HBM_PEAK_GBPS >= 0.60},
        "phase_rates_GBps": phase_rates(by, phase_avg_us),
        "phase_us_per_layer": {p: round(v, 2) for p, v in phase_avg_us.items()},
        "phase_timing": f"score: the kernel's own start and end, recorded into HIP events by its launch "
                        f"(hipExtLaunchKernel); the other phases: HIP events between launches on the decode stream; "
                        f"layers {sampled}, {PH} eager steps after the timed region",
        "launch": "one captured HIP graph per step (all layers), replayed" if graph is not None else "eager launches",
        "rebuild": args.rebuild if args.rebuild != "auto" else ("separate" if host else "fused"),
        "select": args.select,
        "layer_us": round(layer_us, 2),
        "build_ms_per_layer": {"mean": round(1000.0 * sum(build_s[1:] or build_s) / len(build_s[1:] or build_s), 1),
                               "first": round(1000.0 * build_s[0], 1),
                               "note": "skv_build wall time per layer (not part of the timed decode steps); "
                                       "mean over layers after the first"},
        "alpha": {"timed_steps": round(alpha_timed, 4), "steps_1_to_end": round(alpha_all, 4),
                  "misses_per_layer_step": round(misses, 1)},
        "equivalent_bandwidth_TBps": {
            "formula_no_pcie_term_at_8TBps": round(b_tilde(None), 2),
            "formula_measured_alpha_and_pcie": round(b_tilde(pcie_gbps or pcie_peak), 2),
            "pcie_GBps_used": round(pcie_gbps or pcie_peak, 2),
            "pcie_source": "host-value gather rate" if pcie_gbps else "pinned host->device copy rate (measured)",
            "dense_bytes_over_measured_time": round(bt_measured, 1)},
        "pcie": pcie,
        "cpu_baseline": cpu,
    }
    if args.calib_copy:
        calibration_copy()
    print(json.dumps(rec), flush=True)
    for ly in layers:
        ly.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())

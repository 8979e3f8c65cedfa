#!/usr/bin/env python3
"""Benchmark of the lbq hot path on one MI355X.

One step is one pass of the whole hot path over the page workloads, phase by
phase (each phase is named for its workload):

LLaMA-3-8B decoder layer (q, k, v, o 4096/1024 x 4096; gate, up 14336 x 4096;
down 4096 x 14336):
  gemv_m1      Y = X W^T at m = 1, INT4 g128, over R distinct weight copies
               (R * 118 MB > 2 x 256 MB Infinity Cache, so weights stream from
               HBM); q/k/v and gate/up share X and run as one grouped call each,
               o and down alone: 4 launches per layer
  gemv_m1_per_linear  the same with one launch per linear (7 per layer)
  gemv_m4, gemv_m16   m = 4 and 16, grouped like gemv_m1 (multi-row GEMV or the
               small-batch kernel plus its K-split reduce)
  quant_int4, quant_nf4dq  quantize + pack the 7 fp32 weights
  dequant      dequantize the 7 NF4-DQ weights to bf16
  gemm_m2048   INT4 g128 forward at m = 2048, grouped calls
  fwd_m4096    NF4-DQ forward at m = 4096 (2 x 2048 tokens)       <- headline
  fwd_m4096_per_linear, lora_m4096 (rank 16 on q, v), bwd_m4096,
  bwd_m4096_grouped, lora_bwd_m4096
LLaMA-3-70B-shaped layer (8192^2, 1024 x 8192, 28672 x 8192, 8192 x 28672):
  chmix_70b_m1, _m3, _m16, _m40, _m1024   channel mix, 25% INT4 g128 / 75% INT2
               g64 rows; the linears that share X in one grouped call (both
               formats in one launch at m <= 64, one GEMM launch per format above)
  lmix70_i4_m1, lmix70_i2_m1, lmix70_i2c_m1   layer mix: every linear INT4
               g128, or INT2 g64, or INT2 g64 with compact metadata, m = 1
  lmix70_i4_m1024, lmix70_i2_m1024            the same layers at m = 1024
Qwen1.5-110B-shaped layer (hidden 8192, intermediate 49152, 8 kv heads),
all 7 linears INT2 g64, Student-t weights:
  qwen_quant_int2  quantize the whole layer (5.44 GB of fp32)
  qwen_gemv_m1     GEMV at m = 1 over 2 copies (2 x 446 MB)
  qwen_gemm_m512   GEMM at m = 512
  copy_1g      (only with --phases) a plain 1 GiB device copy, the reference
               kernel for scaling hardware byte counters

Every decode phase rotates over enough distinct weight copies that its bytes
per step exceed 2 x 256 MB, so weights come from HBM, not the Infinity Cache.

Timing: each phase (or each launch of the headline phase) is captured once as
a HIP graph (torch.cuda.CUDAGraph) and replayed K times back to back between
two HIP events on the launch stream, so the timed region holds device work
only.  ``value`` is the dequant-GEMM TFLOP/s of fwd_m4096 (2*m*n*k over the 7
linears / phase time); ``gemv_m1_hbm_GBps`` is the other half of the metric.

Also in the JSON line, from the same run:
  ceilings     a plain streaming read over 1 GiB and hipBLASLt bf16 GEMMs
               (torch.matmul) at 4096^3 and 4096 x 14336 x 4096
  gemv_m1_shapes  per decode launch of the 8B layer (q+k+v, o, gate+up,
               down): bytes, median / p10 / p90 microseconds over >= 100 graph
               replays of R distinct copies, and the streaming read of the
               same bytes timed the same way
  roofline     the dominant kernel (the 256 x 256-tile NF4+DQ GEMM launches)
  cpu_baseline the oracle on the host cores (see cpu_baseline())

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       [--phases a,b] [--eager] [--mark-phases FILE]
       python bench.py --traffic-from FETCH_CSV WRITE_CSV
       python bench.py --trace-summary KERNEL_TRACE_CSV PHASES_JSON OUT_MD
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dequant-GEMM TFLOP/s at M=4096; GEMV HBM GB/s at M=1 (LLaMA-3-8B shapes)"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published
PROFILES = os.path.join(ROOT, "profiles")
MALL_BYTES = 256 << 20          # MI355X Infinity Cache
GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))  # linears that read the same activation


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "group_wise_minmax_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, or None
    when no summary exists or the kernels changed since it was taken."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    if data.get("kernel_source_hash") != kernel_source_hash():
        return None
    ent = data.get("kernels", {}).get(kernel)
    return None if ent is None else ent.get("hbm_bytes_per_launch")


ALL_PHASES = ("gemv_m1", "gemv_m1_per_linear", "gemv_m4", "gemv_m16",
              "chmix_70b_m1", "chmix_70b_m3", "chmix_70b_m16", "chmix_70b_m40", "lmix70_i4_m1", "lmix70_i2_m1", "lmix70_i2c_m1", "qwen_gemv_m1",
              "quant_int4", "quant_nf4dq", "dequant", "qwen_quant_int2",
              "gemm_m2048", "fwd_m4096", "fwd_m4096_per_linear", "lora_m4096", "bwd_m4096", "bwd_m4096_grouped",
              "lora_bwd_m4096", "chmix_70b_m1024", "lmix70_i4_m1024", "lmix70_i2_m1024", "qwen_gemm_m512")
EXTRA_PHASES = ("copy_1g",)  # opt-in: plain 1 GiB device copy (counter calibration)


# Kernel-name patterns (rocprofv3 demangled names) whose HBM traffic the
# counter summary reports, with the phase they are measured in.
TRAFFIC_KERNELS = {
    "fwd_m4096_big": ("k_gemm_fwd<5, 256, 256, 4, 2, false, false>", "k_gemm_fwd_set<5, 256, 256, 4, 2, false>"),
    "gemv_m1": ("k_gemv1<0,", "k_gemv1_set<0,"),
    "gemvm_m4": ("k_gemvm<0,", "k_gemvm_set<0,"),
    "skinny_m16": ("k_skinny<0,", "k_skinny_set<0,"),
    "skinny_reduce_m16": ("k_skinny_reduce",),
    "skinny_mix_m40": ("k_skinny_mix<",),
    "quant_int4": ("k_quant_minmax<4, 128, false>",),
    "quant_nf4dq": ("k_quant_nf4<1,",),
    "dequant_nf4dq": ("k_dequant<5>",),
    "bwd_m4096": ("k_bwd_dx<5, 256, 256",),
    "gemm_reduce_m1024": ("k_gemm_reduce",),
}


def write_traffic(fetch_csv: str, write_csv: str, commands=()) -> dict:
    """profiles/traffic.json from two rocprofv3 --pmc runs (FETCH_SIZE, then
    WRITE_SIZE, KiB per dispatch) of the same bench.py command (with copy_1g).
    Each counter is scaled by what it reads for the plain 1 GiB device copy
    (2^30 bytes read and 2^30 written)."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        return vals

    fe, wr = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    copy_f = max(v for k, vs in fe.items() if "copy" in k.lower() for v in vs)
    copy_w = max(v for k, vs in wr.items() if "copy" in k.lower() for v in vs)
    cf, cw = float(1 << 30) / copy_f, float(1 << 30) / copy_w
    out = {"kernel_source_hash": kernel_source_hash(),
           "commands": list(commands),
           "copy_1GiB": {"FETCH_SIZE_bytes": copy_f, "WRITE_SIZE_bytes": copy_w, "fetch_factor": cf, "write_factor": cw},
           "kernels": {}}
    for key, pats in TRAFFIC_KERNELS.items():
        f = [v for k, vs in fe.items() if any(p in k for p in pats) for v in vs]
        w = [v for k, vs in wr.items() if any(p in k for p in pats) for v in vs]
        if f and w:
            fb, wb = sum(f) / len(f) * cf, sum(w) / len(w) * cw
            out["kernels"][key] = {"dispatches": len(f), "fetch_bytes_per_launch": round(fb),
                                   "write_bytes_per_launch": round(wb), "hbm_bytes_per_launch": round(fb + wb)}
    with open(os.path.join(PROFILES, "traffic.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    return out


SIMDS = 256 * 4                 # MI355X: 256 CUs x 4 SIMDs
SCLK_HZ = 2.4e9                 # MI355X peak engine clock
XCDS = 8                        # MI355X: GRBM_COUNT sums one clock counter per XCD


def _short_kernel(name: str) -> str:
    return name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "").replace("lbq::", "")


def counter_summary(csvs, out_md: str, commands=(), match: str = "lbq::") -> None:
    """Per kernel (name + grid), the mean of every counter over its dispatches
    in one or more rocprofv3 --pmc CSVs (each pass its own run of the same
    bench.py command), and the figures derived from them:
      TF/s        SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 flop / duration
      MFMA busy   SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x duration x 2.4 GHz)
      VALU/MFMA   (SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA
      LDS conf    SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE
      wait, issue, valu, lds, vmem
                  SQ_WAIT_ANY, SQ_WAIT_INST_ANY, SQ_ACTIVE_INST_VALU,
                  SQ_ACTIVE_INST_LDS, SQ_ACTIVE_INST_VMEM / SQ_WAVE_CYCLES
      clock       GRBM_COUNT / 8 XCDs / duration: the engine clock while the
                  kernel ran, for dispatches of at least 500 us (an upper
                  bound: the counter window also covers some dispatch set-up,
                  which shorter kernels cannot absorb)
      busy@clk    SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_COUNT / 8):
                  MFMA busy against the cycles the clock actually ran
    Durations are the counter run's own (dispatches serialised)."""
    import csv
    import numpy as np
    acc = {}
    for path in csvs:
        disp = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if match not in r["Kernel_Name"]:
                    continue
                key = (_short_kernel(r["Kernel_Name"]), int(r["Grid_Size"]) // int(r["Workgroup_Size"]))
                d = disp.setdefault((key, r["Dispatch_Id"]), {"dur": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9})
                d[r["Counter_Name"]] = float(r["Counter_Value"])
        for (key, _), d in disp.items():
            for c, v in d.items():
                acc.setdefault(key, {}).setdefault(c, []).append(v)
    lines = ["# Hardware counters per kernel and grid (rocprofv3 --pmc)", ""]
    if commands:
        lines += ["Commands (on the MI355X box, from the repository root `$R`; one counter pass per run):", ""]
        lines += ["    " + c for c in commands] + [""]
    lines += ["Derived figures: TF/s = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / duration; MFMA busy = "
              "SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x duration x 2.4 GHz); VALU/MFMA = (SQ_INSTS_VALU - "
              "SQ_INSTS_MFMA) / SQ_INSTS_MFMA; LDS conf = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; wait / issue / "
              "valu / lds / vmem = SQ_WAIT_ANY / SQ_WAIT_INST_ANY / SQ_ACTIVE_INST_VALU / SQ_ACTIVE_INST_LDS / "
              "SQ_ACTIVE_INST_VMEM over SQ_WAVE_CYCLES; clock = GRBM_COUNT / 8 XCDs / duration (GHz; dispatches of "
              "at least 500 us only, and an upper bound: the counter window also covers dispatch set-up); "
              "busy@clk = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_COUNT / 8).  Durations (us) are the "
              "counter runs' own.", "",
              "| kernel | workgroups | n | us | TF/s | MFMA busy | VALU/MFMA | LDS conf | wait | issue | valu | lds | vmem "
              "| clock | busy@clk |",
              "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]

    def m(d, c):
        return float(np.mean(d[c])) if c in d else None

    def fmt(x, p=3):
        return "" if x is None else f"{x:.{p}f}"

    raw = {}
    for key, d in sorted(acc.items(), key=lambda kv: -sum(kv[1]["dur"])):
        dur = m(d, "dur")
        mops, busy = m(d, "SQ_INSTS_VALU_MFMA_MOPS_BF16"), m(d, "SQ_VALU_MFMA_BUSY_CYCLES")
        valu, mf = m(d, "SQ_INSTS_VALU"), m(d, "SQ_INSTS_MFMA")
        conf, act = m(d, "SQ_LDS_BANK_CONFLICT"), m(d, "SQ_LDS_IDX_ACTIVE")
        wc = m(d, "SQ_WAVE_CYCLES")
        share = {c: (m(d, c) / wc if wc and m(d, c) is not None else None)
                 for c in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM")}
        tf = mops * 512 / dur / 1e12 if mops else None
        mb = busy / (SIMDS * dur * SCLK_HZ) if busy is not None else None
        vpm = (valu - mf) / mf if valu is not None and mf else None
        lc = conf / act if conf is not None and act else None
        grbm = m(d, "GRBM_COUNT")
        long_run = dur >= 500e-6  # the set-up in the window is then at most a few per cent
        clk = grbm / XCDS / dur / 1e9 if grbm and long_run else None
        mbc = busy / (SIMDS * grbm / XCDS) if grbm and long_run and busy is not None else None
        lines.append(f"| `{key[0]}` | {key[1]} | {len(d['dur'])} | {dur * 1e6:.1f} | {fmt(tf, 0)} | {fmt(mb)} | {fmt(vpm, 2)} | "
                     f"{fmt(lc)} | " + " | ".join(fmt(share[c]) for c in share) + f" | {fmt(clk, 2)} | {fmt(mbc)} |")
        raw[f"{key[0]} [{key[1]}]"] = {c: round(float(np.mean(v)), 1) for c, v in d.items() if c != "dur"}
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n\nMean counter values per dispatch:\n\n```json\n" + json.dumps(raw, indent=1) + "\n```\n")


def stats_summary(stats_csv: str, out_md: str, command: str = "") -> None:
    """The library's rows of a rocprofv3 --stats kernel summary (all phases of
    one run pooled per kernel; the per-phase split is trace_summary's)."""
    import csv
    lines = [f"# rocprofv3 --stats kernel summary (liblbq kernels): {os.path.basename(stats_csv)}", ""]
    if command:
        lines += ["Command (on the MI355X box, from the repository root `$R`):", "", "    " + command, ""]
    lines += ["Each kernel pooled over every phase of the run; durations in microseconds.  Template arguments: "
              "first = weight kind (0 INT4 g128, 1 INT4 g64, 2 INT2 g64, 3 INT2 g128, 4 NF4, 5 NF4+DQ, "
              "6 compact INT4 g128, 7 compact INT2 g64, 8 NF4+DQ with offset).", "",
              "| kernel | calls | total us | avg us | min us | max us |", "|---|---:|---:|---:|---:|---:|"]
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            if "lbq::" not in r["Name"]:
                continue
            lines.append(f"| `{_short_kernel(r['Name'])}` | {r['Calls']} | {int(r['TotalDurationNs']) / 1e3:.1f} | "
                         f"{float(r['AverageNs']) / 1e3:.2f} | {int(r['MinNs']) / 1e3:.2f} | {int(r['MaxNs']) / 1e3:.2f} |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def trace_summary(trace_csv: str, phases_json: str, out_md: str, command: str = "") -> None:
    """Per phase and per launch shape (kernel name + grid), the count and the
    median / p10 / p90 / mean duration of the dispatches of a rocprofv3
    --kernel-trace CSV of a bench.py run with --mark-phases: bench.py launches
    a one-element fp64 fill before each phase's timed launches and after the
    last, so the dispatches between two such fills belong to one phase."""
    import csv
    import numpy as np
    rows = []
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            if "Grid_Size_X" in r:
                grid = "x".join(str(int(r[f"Grid_Size_{a}"]) // int(r[f"Workgroup_Size_{a}"]))
                                for a in "XYZ" if int(r[f"Grid_Size_{a}"]) > 1 or a == "X")
            else:
                grid = r.get("Grid_Size", "")
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"], grid))
    rows.sort()
    with open(phases_json) as f:
        order = json.load(f)["phases"]
    seg, segs = None, []
    for s, e, name, grid in rows:
        if "FillFunctor<double>" in name:  # the phase marker (nothing else here fills doubles)
            if seg:  # two markers in a row (an older run's zero-filled marker) bound no phase
                segs.append(seg)
            seg = []
            continue
        if seg is not None:
            seg.append((name, grid, (e - s) / 1000.0))
    lines = [f"# Kernel-trace summary per phase and launch shape: {os.path.basename(trace_csv)}", ""]
    if command:
        lines += ["Command (on the MI355X box, from the repository root `$R`):", "", "    " + command, ""]
    lines += ["Durations in microseconds; p10 / p90 are the 10th / 90th percentiles over the phase's timed "
              "dispatches of that kernel and grid size.", "",
              "| phase | kernel | workgroups | dispatches | median | p10 | p90 | mean |", "|---|---|---:|---:|---:|---:|---:|---:|"]
    for ph, sg in zip(order, segs):
        by = {}
        for name, grid, us in sg:
            short = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "").replace("lbq::", "")
            by.setdefault((short, grid), []).append(us)
        for (short, grid), v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
            a = np.array(v)
            lines.append(f"| {ph} | `{short}` | {grid} | {len(a)} | {np.median(a):.2f} | {np.percentile(a, 10):.2f} | "
                         f"{np.percentile(a, 90):.2f} | {a.mean():.2f} |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")


# ---------------------------------------------------------------------------
# Launch counts, from the public workspace queries and the library's split rule
# ---------------------------------------------------------------------------

def _fill(t):
    return t / (((t + 255) // 256) * 256)


def gemm_splits(n, k, m) -> int:
    """K ranges of an n x k weight's GEMM at m (the library's rule,
    k_gemm_fwd.hip): split when its 256x256 tiles fill at most half the chip."""
    t = ((n + 255) // 256) * ((m + 255) // 256)
    if t > 128:
        return 1
    unit = 512 if m <= 256 and t <= 32 else 1024
    ks = min(256 // t, 8, k // 512 if unit == 512 else k // 3200)
    if ks < 2:
        return 1
    per = ((k + ks - 1) // ks + unit - 1) // unit * unit
    return (k + per - 1) // per


def gemm_set_launches(ns, k, m, cuttable=True) -> int:
    """Launches of one weight kind's GEMM (m > 64) over weights of ns rows:
    the library's rule (k_gemm_fwd.hip) splits a set in two when two tile
    shapes fill the chip's rounds better by over 5% (between weights, or,
    when no weight splits K, inside the weight where whole rounds of 256x256
    tiles end; not for the offset kind), and a launch in which a weight
    splits K adds the reduce of its partials."""
    def cost(ns_):
        ks = [gemm_splits(n, k, m) for n in ns_]
        t0 = sum((n + 255) // 256 * ((m + 255) // 256) * s for n, s in zip(ns_, ks))
        t1 = sum((n + 255) // 256 * ((m + 127) // 128) * s for n, s in zip(ns_, ks))
        t2 = sum((n + 127) // 128 * ((m + 127) // 128) * s for n, s in zip(ns_, ks))
        return sum(n * m / 65536 for n in ns_) / max(_fill(t0), _fill(t1) * 0.78, _fill(t2) * 0.74)

    def launches(ns_):
        return 1 + (1 if any(gemm_splits(n, k, m) > 1 for n in ns_) else 0)
    best, best_cost = 0, 0.95 * cost(ns)
    for j in range(1, len(ns)):
        c = cost(ns[:j]) + cost(ns[j:])
        if c < best_cost:
            best, best_cost = j, c
    if cuttable and not any(gemm_splits(n, k, m) > 1 for n in ns):
        ny = (m + 255) // 256
        t0 = sum((n + 255) // 256 * ny for n in ns)
        if t0 > 256 and t0 % 256:
            left = (t0 // 256) * 256 // ny
            for jw, n in enumerate(ns):
                if left < (n + 255) // 256:
                    break
                left -= (n + 255) // 256
            else:
                jw = len(ns)
            if jw < len(ns) and left > 0:
                r = 256 * left
                if cost(ns[:jw] + [r]) + cost([ns[jw] - r] + ns[jw + 1:]) < best_cost:
                    return 2
    return launches(ns) if best == 0 else launches(ns[:best]) + launches(ns[best:])


def grouped_launches(L, qws, m) -> int:
    """Launches of one lbq_linear_fwd_grouped call (one per weight kind; the
    small-batch kernel adds its K-split reduce when it needs a workspace, and
    so does a GEMM launch in which a weight splits K)."""
    kinds = []
    for q in qws:
        key = (q.desc.format, q.desc.bits, q.desc.group, q.desc.double_quant, q.desc.meta)
        if key not in kinds:
            kinds.append(key)
    mix = {(0, 4, 128, 0, 0), (0, 2, 64, 0, 0)}
    if m == 1:
        return 1 if set(kinds) == mix else len(kinds)
    if set(kinds) == mix and m <= 64 and (m > 4 or qws[0].k > (15872 if m == 2 else 7936)):
        # the channel-mixed set in one small-batch launch (plus its reduce)
        return 1 + (1 if L.lbq_linear_fwd_grouped_workspace_bytes(qws, m) > 0 else 0)
    n = 0
    for key in kinds:
        sub = [q for q in qws if (q.desc.format, q.desc.bits, q.desc.group, q.desc.double_quant, q.desc.meta) == key]
        if m <= 64:
            n += 1 + (1 if L.lbq_linear_fwd_grouped_workspace_bytes(sub, m) > 0 else 0)
        else:
            n += gemm_set_launches([q.n for q in sub], sub[0].k, m, cuttable=key[3] != 2)
    return n


def single_launches(L, q, m) -> int:
    if m == 1:
        return 1
    # the small-batch kernel's reduce, or the reduce of a GEMM that splits K
    return 1 + (1 if L.lbq_linear_workspace_bytes(q, m) > 0 else 0)


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

def clone_qw(L, q):
    return L.QuantizedWeight(q.desc, q.packed.clone(),
                             None if q.scales is None else q.scales.clone(),
                             None if q.zeros is None else q.zeros.clone(),
                             None if q.absmax is None else q.absmax.clone(),
                             None if q.absmax_q is None else q.absmax_q.clone(),
                             None if q.absmax_scale is None else q.absmax_scale.clone(),
                             q.out_rows)


def copies_for(nbytes_one: int, minimum: int = 2) -> int:
    """Distinct copies so that one pass over them exceeds 2 x the Infinity Cache."""
    return max(minimum, -(-2 * MALL_BYTES // max(1, nbytes_one)) + 1)


def build_workload(L, SI, torch, dev, R, want):
    """Allocate the inputs/outputs of the phases in `want` once; return the phase list."""
    need = lambda *ph: any(p in want for p in ph)
    phases = []

    # ---- LLaMA-3-8B layer -------------------------------------------------
    shapes = SI.LLAMA3_8B
    names = list(shapes)
    K_of = {nm: shapes[nm][1] for nm in names}
    N_of = {nm: shapes[nm][0] for nm in names}
    p8 = ("gemv_m1", "gemv_m1_per_linear", "gemv_m4", "gemv_m16", "quant_int4", "quant_nf4dq", "dequant", "gemm_m2048",
          "fwd_m4096", "fwd_m4096_per_linear", "lora_m4096", "bwd_m4096", "bwd_m4096_grouped", "lora_bwd_m4096")
    if need(*p8):
        W = {nm: SI.dev_gaussian_weights(SI.seed_of(2, i, SI.SLOT_W), *shapes[nm], dev) for i, nm in enumerate(names)}
        q4 = {nm: L.QuantizedWeight.empty(L.make_desc("minmax", *shapes[nm], 4, 128), dev) for nm in names}
        qn = {nm: L.QuantizedWeight.empty(L.make_desc("nf4", *shapes[nm], double_quant=True), dev) for nm in names}
        for nm in names:
            L.lbq_quantize(W[nm], "minmax", 4, 128, out=q4[nm])
            L.lbq_quantize(W[nm], "nf4", double_quant=True, out=qn[nm])
        if not need("quant_int4", "quant_nf4dq"):
            W = None
        copies = [q4] + ([{nm: clone_qw(L, q) for nm, q in q4.items()} for _ in range(R - 1)]
                         if need("gemv_m1", "gemv_m1_per_linear", "gemv_m4", "gemv_m16") else [])
        wbf = {nm: torch.empty(shapes[nm], dtype=torch.bfloat16, device=dev) for nm in names} if need("dequant") else {}

        def xs(cfg, slot, off, m, dim_of, on):
            if not on:
                return {}
            return {nm: SI.dev_bf16_normal(SI.seed_of(cfg, i, slot) + off, (m, dim_of[nm]), dev) for i, nm in enumerate(names)}

        def ys(m, dim_of, on):
            return {nm: torch.empty((m, dim_of[nm]), dtype=torch.bfloat16, device=dev) for nm in names} if on else {}

        X1, Y1 = xs(2, SI.SLOT_X, 0, 1, K_of, need("gemv_m1", "gemv_m1_per_linear")), ys(1, N_of, need("gemv_m1", "gemv_m1_per_linear"))
        X4, Y4 = xs(2, SI.SLOT_X, 50, 4, K_of, need("gemv_m4")), ys(4, N_of, need("gemv_m4"))
        X16, Y16 = xs(2, SI.SLOT_X, 100, 16, K_of, need("gemv_m16")), ys(16, N_of, need("gemv_m16"))
        ws16 = {}
        if need("gemv_m4", "gemv_m16"):
            for g in GROUPS:
                for m in (4, 16):
                    nb = L.lbq_linear_fwd_grouped_workspace_bytes([q4[nm] for nm in g], m)
                    ws16[(g, m)] = torch.empty(max(16, nb), dtype=torch.uint8, device=dev) if nb else None
        X2k, Y2k = xs(2, SI.SLOT_X, 200, 2048, K_of, need("gemm_m2048")), ys(2048, N_of, need("gemm_m2048"))
        X4k = xs(3, SI.SLOT_X, 0, 4096, K_of, need("fwd_m4096", "fwd_m4096_per_linear", "lora_m4096", "lora_bwd_m4096"))
        Y4k = ys(4096, N_of, need("fwd_m4096", "fwd_m4096_per_linear"))
        dY = xs(3, SI.SLOT_DY, 0, 4096, N_of, need("bwd_m4096", "bwd_m4096_grouped", "lora_bwd_m4096"))
        dX = ys(4096, K_of, need("bwd_m4096", "bwd_m4096_grouped", "lora_bwd_m4096"))
        lora, lora_bwd = {}, {}
        if need("lora_m4096", "lora_bwd_m4096"):
            for nm in ("q", "v"):
                i = names.index(nm)
                A = SI.dev_bf16_normal(SI.seed_of(3, i, SI.SLOT_A), (16, K_of[nm]), dev, std=0.01)
                B = SI.dev_bf16_normal(SI.seed_of(3, i, SI.SLOT_B), (N_of[nm], 16), dev, std=0.01)
                ws = torch.empty(L.lbq_lora_workspace_bytes(qn[nm], 4096, 16), dtype=torch.uint8, device=dev)
                lora[nm] = (A, B, ws, torch.empty((4096, N_of[nm]), dtype=torch.bfloat16, device=dev))
                wsb = torch.empty(L.lbq_lora_bwd_workspace_bytes(qn[nm], 4096, 16), dtype=torch.uint8, device=dev)
                lora_bwd[nm] = (A, B, wsb, torch.empty((16, K_of[nm]), dtype=torch.float32, device=dev),
                                torch.empty((N_of[nm], 16), dtype=torch.float32, device=dev))

        def call(qs, X, Y, g, ws=None):
            if len(g) == 1:
                L.lbq_linear_fwd(X[g[0]], qs[g[0]], out=Y[g[0]], workspace=ws)
            else:
                L.lbq_linear_fwd_grouped(X[g[0]], [qs[nm] for nm in g], outs=[Y[nm] for nm in g], workspace=ws)

        def p_gemv_grouped(X, Y, m):
            def f():
                for c in copies:
                    for g in GROUPS:
                        call(c, X, Y, g, ws16.get((g, m)))
            return f

        def p_gemv_per_linear():
            for c in copies:
                for nm in names:
                    L.lbq_linear_fwd(X1[nm], c[nm], out=Y1[nm])

        def units(qs, X, Y, per_linear=False):
            if per_linear:
                return [(nm, (lambda nm=nm: L.lbq_linear_fwd(X[nm], qs[nm], out=Y[nm]))) for nm in names]
            return [("+".join(g), (lambda g=g: call(qs, X, Y, g))) for g in GROUPS]

        def p_quant(qs, fmt):
            def f():
                for nm in names:
                    if fmt == "int4":
                        L.lbq_quantize(W[nm], "minmax", 4, 128, out=qs[nm])
                    else:
                        L.lbq_quantize(W[nm], "nf4", double_quant=True, out=qs[nm])
            return f

        def p_dequant():
            for nm in names:
                L.lbq_dequant(qn[nm], out=wbf[nm])

        def p_lora():
            for nm, (A, B, ws, Y) in lora.items():
                L.lbq_lora_fwd(X4k[nm], qn[nm], A, B, 1.0, out=Y, workspace=ws)

        def p_bwd():
            for nm in names:
                L.lbq_linear_bwd_dx(dY[nm], qn[nm], out=dX[nm])

        def p_bwd_grouped():
            for g in GROUPS:
                if len(g) == 1:
                    L.lbq_linear_bwd_dx(dY[g[0]], qn[g[0]], out=dX[g[0]])
                else:
                    L.lbq_linear_bwd_dx_grouped([dY[nm] for nm in g], [qn[nm] for nm in g], out=dX[g[0]])

        def p_lora_bwd():
            for nm, (A, B, ws, dA, dB) in lora_bwd.items():
                L.lbq_lora_bwd(X4k[nm], dY[nm], qn[nm], A, B, 1.0, dX=dX[nm], dA=dA, dB=dB, workspace=ws)

        flop = lambda m: sum(2 * m * n * k for n, k in shapes.values())
        wbytes = lambda c: sum(c[nm].nbytes() for nm in names)
        gemv_bytes = lambda m: sum(wbytes(c) + sum(2 * m * N_of[nm] + 2 * m * K_of[nm] for nm in names) for c in copies)
        gemv_bytes_grouped = lambda m: sum(wbytes(c) + sum(2 * m * N_of[nm] for nm in names) +
                                           sum(2 * m * K_of[g[0]] for g in GROUPS) for c in copies)
        per_layer_launches = lambda qs, m: sum(grouped_launches(L, [qs[nm] for nm in g], m) if len(g) > 1
                                               else single_launches(L, qs[g[0]], m) for g in GROUPS)
        quant_bytes = lambda qs: sum(4 * N_of[nm] * K_of[nm] + qs[nm].nbytes() for nm in names)
        lora_launches = 2 * 3  # per adapted linear: adapter product, its finalize, the GEMM with the LoRA slab
        phases += [
            ("gemv_m1", p_gemv_grouped(X1, Y1, 1), {"bound": "hbm", "bytes": gemv_bytes_grouped(1),
                                                    "launches": per_layer_launches(q4, 1) * len(copies)}),
            ("gemv_m1_per_linear", p_gemv_per_linear, {"bound": "hbm", "bytes": gemv_bytes(1), "launches": 7 * len(copies)}),
            ("gemv_m4", p_gemv_grouped(X4, Y4, 4), {"bound": "hbm", "bytes": gemv_bytes_grouped(4),
                                                    "launches": per_layer_launches(q4, 4) * len(copies)}),
            ("gemv_m16", p_gemv_grouped(X16, Y16, 16), {"bound": "hbm", "bytes": gemv_bytes_grouped(16),
                                                        "launches": per_layer_launches(q4, 16) * len(copies)}),
            ("quant_int4", p_quant(q4, "int4"), {"bound": "hbm", "bytes": quant_bytes(q4), "launches": 7}),
            ("quant_nf4dq", p_quant(qn, "nf4dq"), {"bound": "hbm", "bytes": quant_bytes(qn), "launches": 7}),
            ("dequant", p_dequant, {"bound": "hbm", "bytes": sum(qn[nm].nbytes() + 2 * N_of[nm] * K_of[nm] for nm in names),
                                    "launches": 7}),
            ("gemm_m2048", None, {"bound": "mfma", "flop": flop(2048), "launches": per_layer_launches(q4, 2048),
                                  "units": units(q4, X2k, Y2k)}),
            ("fwd_m4096", None, {"bound": "mfma", "flop": flop(4096), "launches": per_layer_launches(qn, 4096),
                                 "units": units(qn, X4k, Y4k),
                                 "unit_flop": {"+".join(g): sum(2 * 4096 * N_of[nm] * K_of[nm] for nm in g) for g in GROUPS},
                                 # q's launch inside the q+k+v call (256 x 256 tiles), timed alone for the roofline
                                 "roofline_units": [("q", lambda: L.lbq_linear_fwd_grouped(X4k["q"], [qn["q"]], outs=[Y4k["q"]]))],
                                 "roofline_unit_flop": {"q": 2 * 4096 * N_of["q"] * K_of["q"]}}),
            ("fwd_m4096_per_linear", None, {"bound": "mfma", "flop": flop(4096), "launches": 7,
                                            "units": units(qn, X4k, Y4k, per_linear=True)}),
            ("lora_m4096", p_lora, {"bound": "mfma", "flop": sum(2 * 4096 * N_of[nm] * K_of[nm] + 2 * 4096 * 16 * (K_of[nm] + N_of[nm])
                                                                 for nm in lora), "launches": lora_launches}),
            # down's input gradient (k = 14336: 3.5 rounds of 256x256 tiles) runs as two launches
            ("bwd_m4096", p_bwd, {"bound": "mfma", "flop": flop(4096), "launches": 8}),
            ("bwd_m4096_grouped", p_bwd_grouped, {"bound": "mfma", "flop": flop(4096), "launches": len(GROUPS) + 1}),
            # dX = dY W + G A, G = dY B, T = X A^T, dA = G^T X, dB = (T^T dY)^T: 6 launches per adapted linear
            ("lora_bwd_m4096", p_lora_bwd, {"bound": "mfma", "flop": sum(2 * 4096 * N_of[nm] * K_of[nm] +
                                                                         2 * 4096 * 16 * (2 * N_of[nm] + 3 * K_of[nm])
                                                                         for nm in lora_bwd), "launches": 12}),
        ]
        decode_units = {"copies": copies, "X": X1, "Y": Y1}
    else:
        decode_units = None

    # ---- LLaMA-3-70B-shaped layer: channel mix and layer mix ----------------
    s70 = SI.LLAMA3_70B
    n70 = list(s70)
    p70 = ("chmix_70b_m1", "chmix_70b_m3", "chmix_70b_m16", "chmix_70b_m40", "chmix_70b_m1024", "lmix70_i4_m1", "lmix70_i2_m1", "lmix70_i2c_m1", "lmix70_i4_m1024",
           "lmix70_i2_m1024")
    if need(*p70):
        cm, lm = {}, {"i4": {}, "i2": {}, "i2c": {}}
        X70 = {nm: SI.dev_bf16_normal(SI.seed_of(4, i, SI.SLOT_X), (1, s70[nm][1]), dev) for i, nm in enumerate(n70)}
        Xs70 = {mm: {nm: SI.dev_bf16_normal(SI.seed_of(4, i, SI.SLOT_X) + 300 + mm, (mm, s70[nm][1]), dev)
                     for i, nm in enumerate(n70)} for mm in (3, 16, 40) if need(f"chmix_70b_m{mm}")}
        Ys70 = {mm: {nm: torch.empty((mm, s70[nm][0]), dtype=torch.bfloat16, device=dev) for nm in n70} for mm in Xs70}
        X70k = {nm: SI.dev_bf16_normal(SI.seed_of(4, i, SI.SLOT_X) + 100, (1024, s70[nm][1]), dev) for i, nm in enumerate(n70)}
        Y70 = {nm: torch.empty((1, s70[nm][0]), dtype=torch.bfloat16, device=dev) for nm in n70}
        Y70k = {nm: torch.empty((1024, s70[nm][0]), dtype=torch.bfloat16, device=dev) for nm in n70}
        for i, nm in enumerate(n70):
            n, k = s70[nm]
            w = SI.dev_gaussian_weights(SI.seed_of(4, i, SI.SLOT_W), n, k, dev)
            if need("chmix_70b_m1", "chmix_70b_m3", "chmix_70b_m16", "chmix_70b_m40", "chmix_70b_m1024"):
                rows4 = SI.dev_channel_mask(SI.seed_of(4, i, SI.SLOT_CHMASK), n, dev)
                mask = torch.zeros(n, dtype=torch.bool, device=dev)
                mask[rows4.long()] = True
                rows2 = torch.nonzero(~mask).flatten().to(torch.int32)
                a = L.lbq_quantize(w[rows4.long()].contiguous(), "minmax", 4, 128)
                b = L.lbq_quantize(w[rows2.long()].contiguous(), "minmax", 2, 64)
                a.out_rows, b.out_rows = rows4, rows2
                cm[nm] = (a, b)
            if need("lmix70_i4_m1", "lmix70_i4_m1024"):
                lm["i4"][nm] = L.lbq_quantize(w, "minmax", 4, 128)
            if need("lmix70_i2_m1", "lmix70_i2_m1024"):
                lm["i2"][nm] = L.lbq_quantize(w, "minmax", 2, 64)
            if need("lmix70_i2c_m1"):
                lm["i2c"][nm] = L.lbq_quantize(w, "minmax", 2, 64, compact=True)
            del w

        def rotation(layer_qs):
            one = sum(q.nbytes() for q in layer_qs.values())
            return [layer_qs] + [{nm: clone_qw(L, q) for nm, q in layer_qs.items()} for _ in range(copies_for(one) - 1)]

        def chmix_call(cmap, X, Y, ws=None):
            for g in GROUPS:
                qs = [q for nm in g for q in cmap[nm]]
                L.lbq_linear_fwd_grouped(X[g[0]], qs, outs=[Y[nm] for nm in g for _ in range(2)],
                                         workspace=None if ws is None else ws[g])

        def lmix_call(qs, X, Y):
            for g in GROUPS:
                if len(g) == 1:
                    L.lbq_linear_fwd(X[g[0]], qs[g[0]], out=Y[g[0]])
                else:
                    L.lbq_linear_fwd_grouped(X[g[0]], [qs[nm] for nm in g], outs=[Y[nm] for nm in g])

        def dec_bytes(layer_list, m):
            return sum(sum(q.nbytes() for v in lay.values() for q in (v if isinstance(v, tuple) else (v,)))
                       + sum(2 * m * s70[nm][0] for nm in n70) + sum(2 * m * s70[g[0]][1] for g in GROUPS)
                       for lay in layer_list)

        flop70 = lambda m: sum(2 * m * n * k for n, k in s70.values())
        if cm:
            cmr = [cm] + ([{nm: (clone_qw(L, a), clone_qw(L, b)) for nm, (a, b) in cm.items()}
                           for _ in range(copies_for(sum(a.nbytes() + b.nbytes() for a, b in cm.values())) - 1)]
                          if need("chmix_70b_m1", "chmix_70b_m3", "chmix_70b_m16", "chmix_70b_m40") else [])
            cm_launch = lambda m: sum(grouped_launches(L, [q for nm in g for q in cm[nm]], m) for g in GROUPS)
            if need("chmix_70b_m1"):
                phases.append(("chmix_70b_m1", lambda: [chmix_call(c, X70, Y70) for c in cmr],
                               {"bound": "hbm", "bytes": dec_bytes(cmr, 1), "launches": cm_launch(1) * len(cmr)}))
            for mm in Xs70:
                wsm = {}
                for g in GROUPS:
                    nbw = L.lbq_linear_fwd_grouped_workspace_bytes([q for nm in g for q in cm[nm]], mm)
                    wsm[g] = torch.empty(max(16, nbw), dtype=torch.uint8, device=dev) if nbw else None
                phases.append((f"chmix_70b_m{mm}",
                               lambda mm=mm, wsm=wsm: [chmix_call(c, Xs70[mm], Ys70[mm], wsm) for c in cmr],
                               {"bound": "hbm", "bytes": dec_bytes(cmr, mm), "launches": cm_launch(mm) * len(cmr)}))
            if need("chmix_70b_m1024"):
                phases.append(("chmix_70b_m1024", lambda: chmix_call(cm, X70k, Y70k),
                               {"bound": "mfma", "flop": flop70(1024), "launches": cm_launch(1024)}))
        for tag in ("i4", "i2", "i2c"):
            if not lm[tag]:
                continue
            lay = lm[tag]
            launches = lambda m, lay=lay: sum(grouped_launches(L, [lay[nm] for nm in g], m) if len(g) > 1
                                              else single_launches(L, lay[g[0]], m) for g in GROUPS)
            if need(f"lmix70_{tag}_m1"):
                rot = rotation(lay)
                phases.append((f"lmix70_{tag}_m1", lambda rot=rot: [lmix_call(c, X70, Y70) for c in rot],
                               {"bound": "hbm", "bytes": dec_bytes(rot, 1), "launches": launches(1) * len(rot)}))
            if need(f"lmix70_{tag}_m1024"):
                phases.append((f"lmix70_{tag}_m1024", lambda lay=lay: lmix_call(lay, X70k, Y70k),
                               {"bound": "mfma", "flop": flop70(1024), "launches": launches(1024)}))

    # ---- Qwen1.5-110B-shaped layer, INT2 g64 --------------------------------
    sq = SI.QWEN15_110B
    nq = list(sq)
    if need("qwen_quant_int2", "qwen_gemv_m1", "qwen_gemm_m512"):
        Wq = {nm: SI.dev_student_t_weights(SI.seed_of(5, i, SI.SLOT_W), *sq[nm], dev) for i, nm in enumerate(nq)}
        qq = {nm: L.lbq_quantize(Wq[nm], "minmax", 2, 64) for nm in nq}
        if not need("qwen_quant_int2"):
            Wq = None
        Xq1 = {nm: SI.dev_bf16_normal(SI.seed_of(5, i, SI.SLOT_X), (1, sq[nm][1]), dev) for i, nm in enumerate(nq)}
        Xq5 = {nm: SI.dev_bf16_normal(SI.seed_of(5, i, SI.SLOT_X) + 100, (512, sq[nm][1]), dev) for i, nm in enumerate(nq)}
        Yq1 = {nm: torch.empty((1, sq[nm][0]), dtype=torch.bfloat16, device=dev) for nm in nq}
        Yq5 = {nm: torch.empty((512, sq[nm][0]), dtype=torch.bfloat16, device=dev) for nm in nq}

        def q_call(qs, X, Y):
            for g in GROUPS:
                if len(g) == 1:
                    L.lbq_linear_fwd(X[g[0]], qs[g[0]], out=Y[g[0]])
                else:
                    L.lbq_linear_fwd_grouped(X[g[0]], [qs[nm] for nm in g], outs=[Y[nm] for nm in g])

        q_launch = lambda m: sum(grouped_launches(L, [qq[nm] for nm in g], m) if len(g) > 1
                                 else single_launches(L, qq[g[0]], m) for g in GROUPS)
        if need("qwen_quant_int2"):
            def p_qq():
                for nm in nq:
                    L.lbq_quantize(Wq[nm], "minmax", 2, 64, out=qq[nm])
            phases.append(("qwen_quant_int2", p_qq, {"bound": "hbm", "launches": 7,
                                                     "bytes": sum(4 * n * k + qq[nm].nbytes() for nm, (n, k) in sq.items())}))
        if need("qwen_gemv_m1"):
            one = sum(q.nbytes() for q in qq.values())
            rot = [qq] + [{nm: clone_qw(L, q) for nm, q in qq.items()} for _ in range(copies_for(one) - 1)]
            qbytes = sum(one + sum(2 * sq[nm][0] for nm in nq) + sum(2 * sq[g[0]][1] for g in GROUPS) for _ in rot)
            phases.append(("qwen_gemv_m1", lambda: [q_call(c, Xq1, Yq1) for c in rot],
                           {"bound": "hbm", "bytes": qbytes, "launches": q_launch(1) * len(rot)}))
        if need("qwen_gemm_m512"):
            phases.append(("qwen_gemm_m512", lambda: q_call(qq, Xq5, Yq5),
                           {"bound": "mfma", "flop": sum(2 * 512 * n * k for n, k in sq.values()), "launches": q_launch(512)}))

    if need("copy_1g"):
        cp_src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        cp_dst = torch.empty_like(cp_src)
        phases.append(("copy_1g", lambda: cp_dst.copy_(cp_src), {"bound": "hbm", "bytes": 2 << 30, "launches": 1}))
    torch.cuda.synchronize()
    order = {p: i for i, p in enumerate(ALL_PHASES + EXTRA_PHASES)}
    phases = sorted((ph for ph in phases if ph[0] in want), key=lambda ph: order[ph[0]])
    return phases, decode_units


# ---------------------------------------------------------------------------
# Same-run ceilings and the per-shape decode table
# ---------------------------------------------------------------------------

class Stream:
    """The streaming-read probe (bench_stream.hip), loaded with ctypes."""

    def __init__(self, torch, dev):
        self.torch = torch
        path = os.path.join(ROOT, "libbench_stream.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built; run `python -m group_wise_minmax_amd.build`")
        self.lib = ctypes.CDLL(path)
        self.lib.bench_stream_read.restype = ctypes.c_int
        self.lib.bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_void_p, ctypes.c_void_p]
        self.sink = torch.empty(1 << 16, dtype=torch.int32, device=dev)

    def read(self, buf, grid, unroll):
        s = self.torch.cuda.current_stream(buf.device).cuda_stream
        rc = self.lib.bench_stream_read(buf.data_ptr(), buf.numel(), grid, unroll, self.sink.data_ptr(), s)
        if rc != 0:
            raise RuntimeError(f"bench_stream_read: hip error {rc}")


def time_graph(torch, fn, reps, warm=3):
    """Capture fn once, replay it `reps` times, one event pair per replay;
    returns the list of replay times in microseconds."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warm):
        g.replay()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in evs]


def pctl(v):
    import numpy as np
    a = np.array(v)
    return {"median": round(float(np.median(a)), 3), "p10": round(float(np.percentile(a, 10)), 3),
            "p90": round(float(np.percentile(a, 90)), 3)}


def best_stream(torch, st, bufs, reps=20):
    """The best (grid, unroll) of a small sweep for buffers of this size, and
    its per-launch replay times over the rotation of `bufs`."""
    nb = bufs[0].numel()
    best = None
    for grid in (1024, 2048, 4096, 8192):
        if grid * 256 * 16 > nb * 4 and grid > 1024:
            continue
        for unroll in (2, 4, 8):
            t = time_graph(torch, lambda: [st.read(b, grid, unroll) for b in bufs], reps)
            med = sorted(t)[len(t) // 2] / len(bufs)
            if best is None or med < best[0]:
                best = (med, grid, unroll)
    return best


def ceilings(L, torch, dev, st, decode_units, reps):
    """Streaming read over 1 GiB; hipBLASLt bf16 GEMMs; the per-shape decode
    table with the streaming read of the same bytes."""
    out = {}
    big = [torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(3)]
    med, grid, unroll = best_stream(torch, st, big, reps=10)
    out["stream_read_1GiB"] = {"GBps": round((1 << 30) / (med * 1e-6) / 1e9, 1), "grid": grid, "unroll": unroll}
    del big
    for (mm, nn, kk) in ((4096, 4096, 4096), (4096, 14336, 4096)):
        a = torch.randn((mm, kk), device=dev, dtype=torch.bfloat16)
        b = torch.randn((kk, nn), device=dev, dtype=torch.bfloat16)
        c = torch.empty((mm, nn), device=dev, dtype=torch.bfloat16)
        t = time_graph(torch, lambda: [torch.matmul(a, b, out=c) for _ in range(10)], 20)
        med = sorted(t)[len(t) // 2] / 10
        out[f"hipblaslt_bf16_{mm}x{nn}x{kk}"] = {"TFLOPs": round(2 * mm * nn * kk / (med * 1e-6) / 1e12, 1)}
        del a, b, c
    table = {}
    if decode_units is not None:
        q4, X, Y = decode_units["copies"][0], decode_units["X"], decode_units["Y"]
        for g in GROUPS:
            name = "+".join(g)
            one = sum(q4[nm].nbytes() for nm in g) + sum(2 * Y[nm].shape[1] for nm in g) + 2 * X[g[0]].shape[1]
            R = copies_for(one)
            pool = [{nm: q4[nm] for nm in g}] + [{nm: clone_qw(L, q4[nm]) for nm in g} for _ in range(R - 1)]

            def run(pool=pool, g=g):
                for c in pool:
                    if len(g) == 1:
                        L.lbq_linear_fwd(X[g[0]], c[g[0]], out=Y[g[0]])
                    else:
                        L.lbq_linear_fwd_grouped(X[g[0]], [c[nm] for nm in g], outs=[Y[nm] for nm in g])
            t = [v / R for v in time_graph(torch, run, reps)]
            bufs = [torch.empty((one + 15) // 16 * 16, dtype=torch.uint8, device=dev).fill_(5) for _ in range(R)]
            smed, sgrid, sunroll = best_stream(torch, st, bufs)
            sgrid_t = [v / R for v in time_graph(torch, lambda: [st.read(b, sgrid, sunroll) for b in bufs], reps)]
            p, ps = pctl(t), pctl(sgrid_t)
            table[name] = {"bytes": one, "copies": R, "launches_timed": R * reps, "us": p,
                           "GBps_median": round(one / (p["median"] * 1e-6) / 1e9, 1),
                           "stream_us": ps, "stream_GBps_median": round(one / (ps["median"] * 1e-6) / 1e9, 1),
                           "frac_of_stream": round(ps["median"] / p["median"], 3)}
            del pool, bufs
            torch.cuda.empty_cache()
    return out, table


# ---------------------------------------------------------------------------
# CPU baseline: the oracle
# ---------------------------------------------------------------------------

def cpu_info():
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = os.cpu_count()
    return model, avail


def cpu_baseline():
    """The oracle, as it stands, on a bounded sample of the headline workload
    (all 7 linears of the LLaMA-3-8B layer):
      * NF4 + double quantization and INT4 g128 quantization (numpy
        elementwise, one thread), reported apart in GB/s of fp32 read;
      * the fp64 forward Y = X W^T and input gradient dX = dY W at m = 4096
        with every BLAS thread -- ``value``, TFLOP/s of 2*m*n*k per product;
      * the fp64 m = 1 GEMV, one BLAS thread and every thread, GB/s of the
        packed INT4 layer it stands for."""
    import numpy as np
    import synth_inputs as SI
    from oracle import lbq_oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    model, avail = cpu_info()
    m = 4096
    flop = t_mm = t_q = t_q4 = qbytes = 0.0
    gemv1 = {"1": 0.0, "all": 0.0}
    int4_bytes = 0
    for i, (nm, (n, k)) in enumerate(SI.LLAMA3_8B.items()):
        W = SI.gaussian_weights(SI.seed_of(3, i, SI.SLOT_W), n, k, outlier_seed=SI.seed_of(3, i, SI.SLOT_OUTLIER))
        X = SI.bf16_normal(SI.seed_of(3, i, SI.SLOT_X), (m, k))
        dY = SI.bf16_normal(SI.seed_of(3, i, SI.SLOT_DY), (m, n))
        t0 = time.perf_counter()
        ref = O.quantize(W, "nf4", double_quant_on=True)
        t1 = time.perf_counter()
        ref4 = O.quantize(W, "minmax", 4, 128)
        t2 = time.perf_counter()
        t_q += t1 - t0
        t_q4 += t2 - t1
        qbytes += 4.0 * n * k
        int4_bytes += ref4["packed"].nbytes + ref4["scales"].nbytes + ref4["zeros"].nbytes
        x1 = X[:1]
        for key, nthr in (("1", 1), ("all", threads)):
            with threadpool_limits(limits=nthr, user_api="blas"):
                t3 = time.perf_counter()
                O.linear_fwd(x1, ref4["w_exact"])
                gemv1[key] += time.perf_counter() - t3
        t3 = time.perf_counter()
        Y = O.linear_fwd(X, ref["w_exact"])
        dX = O.linear_bwd_dx(dY, ref["w_exact"])
        t_mm += time.perf_counter() - t3
        assert Y.shape == (m, n) and dX.shape == (m, k)
        flop += 4.0 * m * n * k
        del W, X, dY, ref, ref4, Y, dX
    return {"value": round(flop / t_mm / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": model, "cpus_available": int(avail), "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "blas_threads": int(threads),
            "matmul_seconds": round(t_mm, 2),
            "quantize_nf4dq": {"seconds": round(t_q, 2), "GBps_fp32_read": round(qbytes / t_q / 1e9, 3), "threads": 1},
            "quantize_int4": {"seconds": round(t_q4, 2), "GBps_fp32_read": round(qbytes / t_q4 / 1e9, 3), "threads": 1},
            "gemv_m1_fp64": {"seconds_1_thread": round(gemv1["1"], 3), "seconds_all_threads": round(gemv1["all"], 3),
                             "GBps_packed_int4_1_thread": round(int4_bytes / gemv1["1"] / 1e9, 3),
                             "GBps_packed_int4_all_threads": round(int4_bytes / gemv1["all"] / 1e9, 3)},
            "sample": "the 7 LLaMA-3-8B linears: NF4+DQ and INT4 g128 quantize (1 thread, numpy elementwise), "
                      "fp64 forward + input gradient at m=4096 (value; all BLAS threads), fp64 m=1 GEMV (1 and all threads)"}


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--copies", type=int, default=6, help="distinct INT4 8B-layer copies for the decode phases")
    ap.add_argument("--phases", default="", help="comma-separated subset of phases (profiling)")
    ap.add_argument("--eager", action="store_true", help="launch phases directly instead of replaying graphs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the same-run ceilings and per-shape table")
    ap.add_argument("--shape-reps", type=int, default=100, help="graph replays per decode shape")
    ap.add_argument("--mark-phases", metavar="FILE",
                    help="launch a one-element fill before each phase's timed launches (trace separators) and "
                         "write the phase order to FILE")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc counter CSVs and exit")
    ap.add_argument("--trace-summary", nargs=3, metavar=("TRACE_CSV", "PHASES_JSON", "OUT_MD"),
                    help="summarize a rocprofv3 kernel trace per phase and launch shape and exit")
    ap.add_argument("--trace-command", default="", help="command line recorded in the trace summary")
    ap.add_argument("--stats-summary", nargs=2, metavar=("STATS_CSV", "OUT_MD"),
                    help="summarize a rocprofv3 --stats kernel CSV (library kernels) and exit")
    ap.add_argument("--counter-summary", nargs="+", metavar="CSV_OR_OUT",
                    help="summarize rocprofv3 --pmc CSVs (one per counter pass) into the markdown file given "
                         "last and exit; --trace-command may repeat the commands, separated by ' ;; '")
    args = ap.parse_args()
    if args.traffic_from:
        cmds = [c.strip() for c in args.trace_command.split(";;") if c.strip()]
        print(json.dumps(write_traffic(*args.traffic_from, commands=cmds)), flush=True)
        return
    if args.trace_summary:
        trace_summary(*args.trace_summary, command=args.trace_command)
        return
    if args.stats_summary:
        stats_summary(*args.stats_summary, command=args.trace_command)
        return
    if args.counter_summary:
        cmds = [c.strip() for c in args.trace_command.split(";;") if c.strip()]
        counter_summary(args.counter_summary[:-1], args.counter_summary[-1], cmds)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus_requested": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    import group_wise_minmax_amd as L
    import synth_inputs as SI

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_setup = time.perf_counter()
    want = set(args.phases.split(",")) if args.phases else set(ALL_PHASES)
    unknown = want - set(ALL_PHASES) - set(EXTRA_PHASES)
    if unknown:
        print(json.dumps({"error": f"unknown phases {sorted(unknown)}"}), flush=True)
        sys.exit(2)
    phases, decode_units = build_workload(L, SI, torch, dev, args.copies, want)
    print(f"# setup {time.perf_counter() - t_setup:.1f}s; phases: {[p[0] for p in phases]}", file=sys.stderr, flush=True)

    # A phase runs as one graph, or (phases with "units") as one graph per
    # launch unit so that each unit is timed on its own.
    def capture(fn):
        fn()  # eager warm call (first-launch costs stay out of the graph)
        torch.cuda.synchronize()
        if args.eager:
            return fn
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g.replay

    runners = []
    for name, fn, info in phases:
        units = info.get("units") or [(name, fn)]
        runners.append((name, [(u, capture(f)) for u, f in units], info))
    torch.cuda.synchronize()
    print("# captured", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        for _, units, _ in runners:
            for _, run in units:
                run()
    torch.cuda.synchronize()

    marker = torch.empty(1, device=dev, dtype=torch.float64) if args.mark_phases else None
    if args.mark_phases:
        with open(args.mark_phases, "w") as fh:
            json.dump({"phases": [name for name, _, _ in runners]}, fh)

    # The K steps run unit by unit: each unit's graph is replayed K times back
    # to back between two events, so a unit's time is that of K consecutive
    # launches and no unit inherits another phase's cache write-back.  The work
    # timed is exactly K steps.
    K = args.steps
    ev = lambda: torch.cuda.Event(enable_timing=True)
    evs = {name: [(ev(), ev()) for _ in units] for name, units, _ in runners}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, (name, units, _) in enumerate(runners):
        if marker is not None:
            marker.fill_(float(i))
        for j, (_, run) in enumerate(units):
            a, b = evs[name][j]
            a.record()
            for _ in range(K):
                run()
            b.record()
    if marker is not None:
        marker.fill_(-1.0)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / K * 1e3

    # Launches that run inside a unit together with others, timed alone (after
    # the K steps) so that the roofline can describe them.
    roof_us = {}
    for name, fn, info in phases:
        for u, f in (info.get("roofline_units", []) if not args.eager else []):
            run = capture(f)
            for _ in range(args.warmup):
                run()
            a, b = ev(), ev()
            torch.cuda.synchronize()
            a.record()
            for _ in range(K):
                run()
            b.record()
            torch.cuda.synchronize()
            roof_us[u] = a.elapsed_time(b) / K * 1e3

    report = {}
    unit_us = {}
    for name, units, info in runners:
        per_unit = [a.elapsed_time(b) / K for a, b in evs[name]]
        ms = sum(per_unit)
        if len(units) > 1:
            unit_us[name] = {u: per_unit[j] * 1e3 for j, (u, _) in enumerate(units)}
        ent = {"ms": round(ms, 4), "launches": info["launches"], "avg_launch_us": round(ms * 1e3 / info["launches"], 3)}
        if info["bound"] == "hbm":
            gbps = info["bytes"] / (ms * 1e-3) / 1e9
            ent.update(GBps=round(gbps, 1), bytes=info["bytes"], hbm_frac=round(gbps / HBM_PEAK_GBPS, 4))
        else:
            tf = info["flop"] / (ms * 1e-3) / 1e12
            ent.update(TFLOPs=round(tf, 1), flop=info["flop"], mfma_frac=round(tf / BF16_PEAK_TFLOPS, 4))
        if name in unit_us:
            ent["unit_us"] = {u: round(v, 2) for u, v in unit_us[name].items()}
        report[name] = ent
        print(f"# {name:20s} {json.dumps(ent)}", file=sys.stderr, flush=True)

    head = report.get("fwd_m4096")
    value = head["TFLOPs"] if head else None
    gemv = report.get("gemv_m1")
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "LLaMA-3-8B decoder layer (q,k,v,o 4096/1024 x 4096; gate,up 14336x4096; down 4096x14336): "
                        "NF4+DQ forward at m=4096 (headline), INT4 g128 GEMV m=1/4/16, GEMM m=2048, quantize, dequant, "
                        "LoRA r=16 on q,v, input gradient; 70B-shaped layer: channel mix 25% INT4 g128 / 75% INT2 g64 and "
                        "layer mix (INT4 g128, INT2 g64, compact INT2) at m=1 and 1024; Qwen1.5-110B-shaped INT2 g64 "
                        "layer: quantize, GEMV m=1, GEMM m=512",
            "gemm_m": 4096, "gemv_m": 1, "headline_format": "nf4+dq (fwd m=4096); int4 g128 (gemv m=1)",
            "graph_replay": not args.eager,
        },
        "gemv_m1_hbm_GBps": gemv["GBps"] if gemv else None,
        "phases": report,
    }
    if head:
        # Dominant kernel: the 256 x 256-tile NF4+DQ GEMM launches at m = 4096:
        # q (the first of the q+k+v call's two launches; k+v takes 256 x 128
        # tiles), o, gate+up side by side, down.
        info = next(info for name, _, info in runners if name == "fwd_m4096")
        uf = dict(info["unit_flop"], **info["roofline_unit_flop"])
        us = dict(unit_us["fwd_m4096"], **roof_us)
        big = [u for u in ("q", "o", "gate+up", "down") if u in us]
        t_big = sum(us[u] for u in big)
        ach = sum(uf[u] for u in big) / (t_big * 1e-6) / 1e12
        out["roofline"] = {"kernel": "k_gemm_fwd / k_gemm_fwd_set <NF4+DQ, 256x256 tiles> (q, o, gate+up, down at m=4096)",
                           "bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(ach / BF16_PEAK_TFLOPS, 4),
                           "traffic": load_traffic("fwd_m4096_big"),
                           "avg_launch_us": round(t_big / len(big), 2),
                           "per_call_us": {u: round(v, 2) for u, v in us.items()}}
    if gemv:
        per_launch = gemv["bytes"] / gemv["launches"]
        ach = per_launch / (gemv["avg_launch_us"] * 1e-6) / 1e9
        out["roofline_gemv_m1"] = {"kernel": "k_gemv1 / k_gemv1_set <INT4 g128> (m=1: q/k/v, o, gate/up, down launches x copies)",
                                   "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                   "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": load_traffic("gemv_m1")}
    if not args.no_ceilings and not args.eager:
        print("# ceilings and per-shape decode table ...", file=sys.stderr, flush=True)
        st = Stream(torch, dev)
        ceil, table = ceilings(L, torch, dev, st, decode_units, args.shape_reps)
        out["ceilings"] = ceil
        if table:
            out["gemv_m1_shapes"] = table
    if not args.no_cpu_baseline:
        print("# cpu_baseline: timing the oracle on a bounded sample ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

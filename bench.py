#!/usr/bin/env python3
"""Benchmark of the lbq hot path on one MI355X.

One step is one pass of the whole hot path over a LLaMA-3-8B decoder layer
(q, k, v, o, gate, up, down) plus the 70B-shaped mixed-precision dispatch, in
this order:

  gemv_m1      Y = X W^T at m = 1, INT4 g128, over R distinct weight copies
               (R * 118 MB > 2 x 256 MB Infinity Cache, so weights stream from HBM);
               q/k/v and gate/up share X and run as one launch each
               (lbq_linear_fwd_grouped), o and down alone: 4 launches per layer
  gemv_m1_per_linear  the same with one launch per linear (7 per layer)
  gemv_m4      m = 4, launched like gemv_m1 (the rows of X staged together;
               down, k = 14336, takes the small-batch MFMA kernel)
  gemv_m16     m = 16, launched like gemv_m1 (the small-batch MFMA kernel; its
               split-K partials are summed by a second launch per group)
  chmix_70b_m1     70B-shaped layer, per-channel 25% INT4 g128 / 75% INT2 g64
                   (each format's rows scatter into Y), m = 1: the linears that
                   share X in one call, both formats in one launch (4 per layer)
  quant_int4   quantize + pack the 7 fp32 weights, MinMax INT4 g128
  quant_nf4dq  quantize + pack the 7 weights, NF4 block 64 + double quant
  dequant      dequantize the 7 NF4-DQ weights to bf16
  gemm_m2048   INT4 g128 forward at m = 2048, launched like fwd_m4096 (grouped
               calls for q/k/v and gate/up)
  fwd_m4096    NF4-DQ forward at m = 4096 (2 x 2048 tokens)       <- headline;
               q/k/v and gate/up share X and run as one grouped call each
               (their column tiles side by side; q/k/v as two launches, q
               with 256x256 tiles and k+v with 256x128), o and down alone
  fwd_m4096_per_linear  the same with one launch per linear
  lora_m4096   NF4-DQ forward + rank-16 LoRA on q and v at m = 4096
  bwd_m4096    NF4-DQ input gradient dX = dY deq(W) at m = 4096, one call per
               linear
  bwd_m4096_grouped  the layer's input gradients: q/k/v and gate/up each summed
               into their shared input's gradient in one grouped call
               (lbq_linear_bwd_dx_grouped), o and down alone
  lora_bwd_m4096  NF4-DQ LoRA backward (dX with the adapter term, dA, dB),
               rank 16 on q and v, at m = 4096
  chmix_70b_m1024  the 70B-shaped channel-mix layer at m = 1024, grouped like
                   chmix_70b_m1 (one GEMM launch per format and call: 8 per layer)
  copy_1g      (only with --phases) a plain 1 GiB device-to-device copy, the
               reference kernel for scaling hardware byte counters

Each phase (or each launch of the headline phases) is captured once as a HIP
graph (torch.cuda.CUDAGraph) and replayed K times back to back between two HIP
events on the launch stream, so the timed region holds device work only.  The JSON line's ``value`` is the dequant-
GEMM TFLOP/s of fwd_m4096 (2*m*n*k summed over the 7 linears / phase time);
``gemv_m1_hbm_GBps`` is the other half of the headline metric.  Both count
the same 7 linears as the per-linear phases; only the launches differ.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
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

METRIC = "dequant-GEMM TFLOP/s at M=4096; GEMV HBM GB/s at M=1 (LLaMA-3-8B shapes)"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "group_wise_minmax_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, units_per_launch=None):
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


ALL_PHASES = ("quant_int4", "quant_nf4dq", "dequant", "gemv_m1", "gemv_m1_per_linear", "gemv_m4", "gemv_m16", "gemm_m2048",
              "fwd_m4096", "fwd_m4096_per_linear", "lora_m4096", "bwd_m4096", "bwd_m4096_grouped", "lora_bwd_m4096",
              "chmix_70b_m1",
              "chmix_70b_m1024")
EXTRA_PHASES = ("copy_1g",)  # opt-in: plain 1 GiB device copy (counter calibration)


# Kernel-name patterns (rocprofv3 demangled names) of the kernels whose HBM
# traffic the JSON line reports.
TRAFFIC_KERNELS = {
    "fwd_m4096_big": ("k_gemm_fwd<5, 256, 256, 4, 2, false>", "k_gemm_fwd_set<5, 256, 256, 4, 2>"),
    "gemv_m1": ("k_gemv1<0,", "k_gemv1_set<0,"),
}


def write_traffic(fetch_csv: str, write_csv: str) -> dict:
    """profiles/traffic.json from two rocprofv3 --pmc runs (FETCH_SIZE, then
    WRITE_SIZE, KiB per dispatch) of `--phases fwd_m4096,gemv_m1,copy_1g
    --eager`.  Each counter is scaled by what it reads for the plain 1 GiB
    device copy (2^30 bytes read and 2^30 written)."""
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


def build_workload(L, SI, torch, dev, R, want):
    """Allocate the inputs/outputs of the phases in `want` once; return the phase list."""
    shapes = SI.LLAMA3_8B
    names = list(shapes)
    K_of = {nm: shapes[nm][1] for nm in names}
    N_of = {nm: shapes[nm][0] for nm in names}
    need = lambda *ph: any(p in want for p in ph)
    W = {nm: SI.dev_gaussian_weights(SI.seed_of(2, i, SI.SLOT_W), *shapes[nm], dev)
         for i, nm in enumerate(names)}
    q4 = {nm: L.QuantizedWeight.empty(L.make_desc("minmax", *shapes[nm], 4, 128), dev) for nm in names}
    qn = {nm: L.QuantizedWeight.empty(L.make_desc("nf4", *shapes[nm], double_quant=True), dev) for nm in names}
    for nm in names:
        L.lbq_quantize(W[nm], "minmax", 4, 128, out=q4[nm])
        L.lbq_quantize(W[nm], "nf4", double_quant=True, out=qn[nm])
    if not need("quant_int4", "quant_nf4dq"):
        W = None
    # R independent copies of the INT4 layer for the decode phases
    copies = [q4]
    if need("gemv_m1", "gemv_m16"):
        for _ in range(R - 1):
            copies.append({nm: L.QuantizedWeight(q.desc, q.packed.clone(), q.scales.clone(), q.zeros.clone())
                           for nm, q in q4.items()})
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
    X2k, Y2k = xs(2, SI.SLOT_X, 200, 2048, K_of, need("gemm_m2048")), ys(2048, N_of, need("gemm_m2048"))
    X4k = xs(3, SI.SLOT_X, 0, 4096, K_of, need("fwd_m4096", "fwd_m4096_per_linear", "lora_m4096", "lora_bwd_m4096"))
    Y4k = ys(4096, N_of, need("fwd_m4096", "fwd_m4096_per_linear"))
    dY = xs(3, SI.SLOT_DY, 0, 4096, N_of, need("bwd_m4096", "bwd_m4096_grouped", "lora_bwd_m4096"))
    dX = ys(4096, K_of, need("bwd_m4096", "bwd_m4096_grouped", "lora_bwd_m4096"))
    lora = {}
    if need("lora_m4096", "lora_bwd_m4096"):
        for nm in ("q", "v"):
            i = names.index(nm)
            A = SI.dev_bf16_normal(SI.seed_of(3, i, SI.SLOT_A), (16, K_of[nm]), dev, std=0.01)
            B = SI.dev_bf16_normal(SI.seed_of(3, i, SI.SLOT_B), (N_of[nm], 16), dev, std=0.01)
            ws = torch.empty(L.lbq_lora_workspace_bytes(qn[nm], 4096, 16), dtype=torch.uint8, device=dev)
            lora[nm] = (A, B, ws, torch.empty((4096, N_of[nm]), dtype=torch.bfloat16, device=dev))
    lora_bwd = {}
    if need("lora_bwd_m4096"):
        for nm, (A, B, _, _) in lora.items():
            ws = torch.empty(L.lbq_lora_bwd_workspace_bytes(qn[nm], 4096, 16), dtype=torch.uint8, device=dev)
            lora_bwd[nm] = (A, B, ws, torch.empty((16, K_of[nm]), dtype=torch.float32, device=dev),
                            torch.empty((N_of[nm], 16), dtype=torch.float32, device=dev))

    # 70B-shaped channel-mix layer (quantized once at setup)
    s70 = SI.LLAMA3_70B
    cm = []
    if need("chmix_70b_m1", "chmix_70b_m1024"):
        for i, nm in enumerate(s70):
            n, k = s70[nm]
            w = SI.dev_gaussian_weights(SI.seed_of(4, i, SI.SLOT_W), n, k, dev)
            rows4 = SI.dev_channel_mask(SI.seed_of(4, i, SI.SLOT_CHMASK), n, dev)
            mask = torch.zeros(n, dtype=torch.bool, device=dev)
            mask[rows4.long()] = True
            rows2 = torch.nonzero(~mask).flatten().to(torch.int32)
            a = L.lbq_quantize(w[rows4.long()].contiguous(), "minmax", 4, 128)
            b = L.lbq_quantize(w[rows2.long()].contiguous(), "minmax", 2, 64)
            a.out_rows, b.out_rows = rows4, rows2
            del w
            x1 = SI.dev_bf16_normal(SI.seed_of(4, i, SI.SLOT_X), (1, k), dev)
            x1k = SI.dev_bf16_normal(SI.seed_of(4, i, SI.SLOT_X) + 100, (1024, k), dev)
            cm.append((nm, a, b, x1, x1k, torch.empty((1, n), dtype=torch.bfloat16, device=dev),
                       torch.empty((1024, n), dtype=torch.bfloat16, device=dev)))
    cp_src = cp_dst = None
    if need("copy_1g"):
        cp_src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        cp_dst = torch.empty_like(cp_src)
    torch.cuda.synchronize()

    def p_quant_int4():
        for nm in names:
            L.lbq_quantize(W[nm], "minmax", 4, 128, out=q4[nm])

    def p_quant_nf4dq():
        for nm in names:
            L.lbq_quantize(W[nm], "nf4", double_quant=True, out=qn[nm])

    def p_dequant():
        for nm in names:
            L.lbq_dequant(qn[nm], out=wbf[nm])

    def p_gemv(X, Y):
        def f():
            for c in copies:
                for nm in names:
                    L.lbq_linear_fwd(X[nm], c[nm], out=Y[nm])
        return f

    # Linears that read the same activation in a decoder layer: one launch each.
    GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))

    def p_gemv_grouped(X, Y):
        def f():
            for c in copies:
                for g in GROUPS:
                    if len(g) == 1:
                        L.lbq_linear_fwd(X[g[0]], c[g[0]], out=Y[g[0]])
                    else:
                        L.lbq_linear_fwd_grouped(X[g[0]], [c[nm] for nm in g], outs=[Y[nm] for nm in g])
        return f

    def p_gemm(qs, X, Y):
        def f():
            for nm in names:
                L.lbq_linear_fwd(X[nm], qs[nm], out=Y[nm])
        return f

    def p_gemm_grouped(qs, X, Y):
        def f():
            for g in GROUPS:
                if len(g) == 1:
                    L.lbq_linear_fwd(X[g[0]], qs[g[0]], out=Y[g[0]])
                else:
                    L.lbq_linear_fwd_grouped(X[g[0]], [qs[nm] for nm in g], outs=[Y[nm] for nm in g])
        return f

    def gemm_group_units(qs, X, Y):
        def unit(g):
            if len(g) == 1:
                return lambda: L.lbq_linear_fwd(X[g[0]], qs[g[0]], out=Y[g[0]])
            return lambda: L.lbq_linear_fwd_grouped(X[g[0]], [qs[nm] for nm in g], outs=[Y[nm] for nm in g])
        return [("+".join(g), unit(g)) for g in GROUPS]

    def gemm_units(qs, X, Y):
        return [(nm, (lambda nm=nm: L.lbq_linear_fwd(X[nm], qs[nm], out=Y[nm]))) for nm in names]

    def p_lora():
        for nm, (A, B, ws, Y) in lora.items():
            L.lbq_lora_fwd(X4k[nm], qn[nm], A, B, 1.0, out=Y, workspace=ws)

    def p_bwd():
        for nm in names:
            L.lbq_linear_bwd_dx(dY[nm], qn[nm], out=dX[nm])

    def p_bwd_grouped():
        # the layer's input gradients: the linears that read one X (q/k/v,
        # gate/up) summed into that X's gradient in one grouped call
        for g in GROUPS:
            if len(g) == 1:
                L.lbq_linear_bwd_dx(dY[g[0]], qn[g[0]], out=dX[g[0]])
            else:
                L.lbq_linear_bwd_dx_grouped([dY[nm] for nm in g], [qn[nm] for nm in g], out=dX[g[0]])

    def p_lora_bwd():
        for nm, (A, B, ws, dA, dB) in lora_bwd.items():
            L.lbq_lora_bwd(X4k[nm], dY[nm], qn[nm], A, B, 1.0, dX=dX[nm], dA=dA, dB=dB, workspace=ws)

    def p_chmix_m1():
        # per activation group, both row sets of every linear in one call
        # (one launch per format: INT4 g128 and INT2 g64)
        by = {e[0]: e for e in cm}
        for g in GROUPS:
            x1 = by[g[0]][3]
            qs = [q for nm in g for q in by[nm][1:3]]
            ys = [by[nm][5] for nm in g for _ in range(2)]
            L.lbq_linear_fwd_grouped(x1, qs, outs=ys)

    def p_chmix_m1024():
        # as at m = 1: per activation group, both row sets of every linear in
        # one call (one GEMM launch per format)
        by = {e[0]: e for e in cm}
        for g in GROUPS:
            x = by[g[0]][4]
            qs = [q for nm in g for q in by[nm][1:3]]
            ys = [by[nm][6] for nm in g for _ in range(2)]
            L.lbq_linear_fwd_grouped(x, qs, outs=ys)

    def p_copy():
        cp_dst.copy_(cp_src)

    def bytes_fwd(q, m, n, k):
        return q.nbytes() + 2 * m * k + 2 * m * n

    flop = lambda m: sum(2 * m * n * k for n, k in shapes.values())
    gemv_bytes = lambda m: sum(bytes_fwd(c[nm], m, N_of[nm], K_of[nm]) for c in copies for nm in names)
    # grouped: X is read once per launch
    gemv_bytes_grouped = lambda m: sum(c[nm].nbytes() + 2 * m * N_of[nm] for c in copies for nm in names) + \
        len(copies) * sum(2 * m * K_of[g[0]] for g in GROUPS)
    quant_bytes = lambda qs: sum(4 * N_of[nm] * K_of[nm] + qs[nm].nbytes() for nm in names)
    phases = [
        ("gemv_m1", p_gemv_grouped(X1, Y1), lambda: {"bound": "hbm", "bytes": gemv_bytes_grouped(1), "launches": len(GROUPS) * R}),
        ("gemv_m1_per_linear", p_gemv(X1, Y1), lambda: {"bound": "hbm", "bytes": gemv_bytes(1), "launches": 7 * R}),
        ("gemv_m4", p_gemv_grouped(X4, Y4), lambda: {"bound": "hbm", "bytes": gemv_bytes_grouped(4), "launches": len(GROUPS) * R}),
        ("gemv_m16", p_gemv_grouped(X16, Y16), lambda: {"bound": "hbm", "bytes": gemv_bytes_grouped(16), "launches": len(GROUPS) * R}),
        ("chmix_70b_m1", p_chmix_m1, lambda: {"bound": "hbm", "bytes": sum(a.nbytes() + b.nbytes() + 2 * (a.n + b.n) for _, a, b, *_ in cm) + sum(2 * next(a.k for nm, a, *_ in cm if nm == g[0]) for g in GROUPS), "launches": len(GROUPS)}),
        ("quant_int4", p_quant_int4, lambda: {"bound": "hbm", "bytes": quant_bytes(q4), "launches": 7}),
        ("quant_nf4dq", p_quant_nf4dq, lambda: {"bound": "hbm", "bytes": quant_bytes(qn), "launches": 7}),
        ("dequant", p_dequant, lambda: {"bound": "hbm", "bytes": sum(qn[nm].nbytes() + 2 * N_of[nm] * K_of[nm] for nm in names), "launches": 7}),
        ("gemm_m2048", p_gemm_grouped(q4, X2k, Y2k), lambda: {"bound": "mfma", "flop": flop(2048), "launches": len(GROUPS)}),
        ("fwd_m4096", None, lambda: {"bound": "mfma", "flop": flop(4096), "launches": len(GROUPS) + 1,
                                     "units": gemm_group_units(qn, X4k, Y4k),
                                     "unit_flop": {"+".join(g): sum(2 * 4096 * N_of[nm] * K_of[nm] for nm in g) for g in GROUPS},
                                     # q's launch inside the q+k+v call (256 x 256 tiles), timed alone for the roofline
                                     "roofline_units": [("q", lambda: L.lbq_linear_fwd_grouped(X4k["q"], [qn["q"]], outs=[Y4k["q"]]))],
                                     "roofline_unit_flop": {"q": 2 * 4096 * N_of["q"] * K_of["q"]}}),
        ("fwd_m4096_per_linear", None, lambda: {"bound": "mfma", "flop": flop(4096), "launches": 7,
                                                "units": gemm_units(qn, X4k, Y4k),
                                                "unit_flop": {nm: 2 * 4096 * n * k for nm, (n, k) in shapes.items()}}),
        ("lora_m4096", p_lora, lambda: {"bound": "mfma", "flop": sum(2 * 4096 * N_of[nm] * K_of[nm] + 2 * 4096 * 16 * (K_of[nm] + N_of[nm]) for nm in lora), "launches": 4}),
        ("bwd_m4096", p_bwd, lambda: {"bound": "mfma", "flop": flop(4096), "launches": 7}),
        ("bwd_m4096_grouped", p_bwd_grouped, lambda: {"bound": "mfma", "flop": flop(4096), "launches": len(GROUPS)}),
        # dX = dY W + G A, G = dY B, T = X A^T, dA = G^T X, dB = (T^T dY)^T
        ("lora_bwd_m4096", p_lora_bwd, lambda: {"bound": "mfma", "flop": sum(2 * 4096 * N_of[nm] * K_of[nm] + 2 * 4096 * 16 * (2 * N_of[nm] + 3 * K_of[nm]) for nm in lora_bwd), "launches": 12}),
        ("chmix_70b_m1024", p_chmix_m1024, lambda: {"bound": "mfma", "flop": sum(2 * 1024 * (a.n + b.n) * a.k for _, a, b, *_ in cm), "launches": 2 * len(GROUPS)}),
        ("copy_1g", p_copy, lambda: {"bound": "hbm", "bytes": 2 << 30, "launches": 1}),
    ]
    # Decode phases (HBM-bound reads) run first in each step, after the
    # compute-bound GEMMs of the previous step, so that they do not inherit the
    # write-back of the hundreds of MB the quantize/dequant phases leave dirty
    # in the caches.
    return [(nm, fn, info()) for nm, fn, info in phases if nm in want]


def cpu_baseline():
    """The oracle, as it stands, on a bounded sample of the headline workload:
    NF4 + double quantization of all 7 linears of the 8B layer, then the fp64
    forward Y = X W^T and input gradient dX = dY W at m = 4096 for the 7
    linears.  Reported in TFLOP/s of the matmuls' 2*m*n*k (forward and input
    gradient) over the whole oracle time, quantization included."""
    import numpy as np
    import synth_inputs as SI
    from oracle import lbq_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    m = 4096
    flop = 0.0
    dt = 0.0
    for i, (nm, (n, k)) in enumerate(SI.LLAMA3_8B.items()):
        W = SI.gaussian_weights(SI.seed_of(3, i, SI.SLOT_W), n, k, outlier_seed=SI.seed_of(3, i, SI.SLOT_OUTLIER))
        X = SI.bf16_normal(SI.seed_of(3, i, SI.SLOT_X), (m, k))
        dY = SI.bf16_normal(SI.seed_of(3, i, SI.SLOT_DY), (m, n))
        t0 = time.perf_counter()
        ref = O.quantize(W, "nf4", double_quant_on=True)
        Y = O.linear_fwd(X, ref["w_exact"])
        dX = O.linear_bwd_dx(dY, ref["w_exact"])
        dt += time.perf_counter() - t0
        assert Y.shape == (m, n) and dX.shape == (m, k)
        flop += 4.0 * m * n * k
        del W, X, dY, ref, Y, dX
    return {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": "NF4+DQ quantize of the 7 LLaMA-3-8B linears + fp64 forward and input gradient at m=4096"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--copies", type=int, default=6, help="distinct INT4 layer copies for the decode phases")
    ap.add_argument("--phases", default="", help="comma-separated subset of phases (profiling)")
    ap.add_argument("--eager", action="store_true", help="launch phases directly instead of replaying graphs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc counter CSVs and exit")
    args = ap.parse_args()
    if args.traffic_from:
        print(json.dumps(write_traffic(*args.traffic_from)), flush=True)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
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
    phases = build_workload(L, SI, torch, dev, args.copies, want)
    print(f"# setup {time.perf_counter() - t_setup:.1f}s; phases: {[p[0] for p in phases]}", file=sys.stderr, flush=True)

    # A phase runs as one graph, or (phases with "units", the headline) as one
    # graph per launch so that each launch is timed on its own.
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

    for _ in range(args.warmup):
        for _, units, _ in runners:
            for _, run in units:
                run()
    torch.cuda.synchronize()

    # The K steps run unit by unit: each unit's graph is replayed K times back
    # to back between two events, so a unit's time is that of K consecutive
    # launches (the next replay is queued while one runs) and no unit inherits
    # another phase's cache write-back.  The work timed is exactly K steps.
    K = args.steps
    ev = lambda: torch.cuda.Event(enable_timing=True)
    evs = {name: [(ev(), ev()) for _ in units] for name, units, _ in runners}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for name, units, _ in runners:
        for j, (_, run) in enumerate(units):
            a, b = evs[name][j]
            a.record()
            for _ in range(K):
                run()
            b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / K * 1e3

    # Launches that run inside a unit together with others, timed alone
    # (after the K steps) so that the roofline can describe them.  Not in
    # --eager runs (the counter passes): there every launch runs exactly as
    # often as in the phases.
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
        report[name] = ent
        print(f"# {name:12s} {json.dumps(ent)}", file=sys.stderr, flush=True)

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
                        "INT4 g128 + NF4-DQ quantize, dequant, GEMV m=1/16 (INT4 g128, 6 weight copies), "
                        "GEMM m=2048 (INT4), fwd m=4096 (NF4-DQ, headline), LoRA r=16 on q,v, bwd dX m=4096; "
                        "plus 70B-shaped channel-mix (25% INT4 g128 / 75% INT2 g64) at m=1 and 1024",
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
                           "traffic": load_traffic("fwd_m4096_big", None),
                           "avg_launch_us": round(t_big / len(big), 2),
                           "per_call_us": {u: round(v, 2) for u, v in us.items()}}
    if gemv:
        per_launch = gemv["bytes"] / gemv["launches"]
        ach = per_launch / (gemv["avg_launch_us"] * 1e-6) / 1e9
        out["roofline_gemv_m1"] = {"kernel": "k_gemv1 / k_gemv1_set <INT4 g128> (m=1: q/k/v, o, gate/up, down launches x copies)", "bound": "hbm",
                                   "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                   "frac": round(ach / HBM_PEAK_GBPS, 4),
                                   "traffic": load_traffic("gemv_m1", per_launch)}
    if not args.no_cpu_baseline:
        print("# cpu_baseline: timing the oracle on a bounded sample ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the BaKron per-layer hot path on one MI355X.

One step = the whole path for one layer on synthetic inputs already resident
in HBM: H_I = X^T X / T and H_O = G^T G / T (fp32 products formed from two
fp16 pieces per operand of power-of-two-scaled columns on the fp16 matrix
cores), damping + LDL of
both (fp64), fp32 per-row scales, and the BaKron rounding solve with its proxy
loss. Default workload: the attention-projection shape, W* 4096 x 4096,
T = 32768 tokens, 2-bit nearest rounding.

Prints ONE JSON line. `value` is layer throughput in weights/s (m*n per step
time); per-phase times, the solve-only rate, the roofline of the dominant
kernel (the solve's k_solve_run, timed with HIP events on the stream it runs
on), the rooflines of the Hessian calls and the LDL pair, and the CPU oracle
baseline with its replay of the device's codes ride along.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_F16_MFMA_TFLOPS = 2500.0
PIECE_PRODUCTS = 3  # fp16 piece products per fp32 product (Hessian, solve far field)
PEAK_FP64_MFMA_TFLOPS = 78.6
CAL_BYTES = 256 << 20

# HBM traffic per launch of the kernels the roofline objects price, from two
# rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE; KiB per
# dispatch). The counters are scaled by what they read for the calibration copy
# above (CAL_* below: KiB read by FETCH_SIZE and WRITE_SIZE for 262144 KiB moved
# each way). A reading is valid only for the kernel source it was taken on: the
# key is a hash of the listed source files with comments and blank space
# removed, so edits to comments keep it and any code change drops it (null).
CAL_FETCH_KIB, CAL_WRITE_KIB = 131089.0, 262144.0
COUNTERS = {
    # one solve at attn, 2-bit nearest: k_solve_run
    ("solve", "attn", "dbf2c268b3a81d14"): {"fetch_kib": 2688065.3, "write_kib": 822587.6,
                                            "mfma_busy": 0.066, "clock_ghz": 2.35},
    # one hessian_accum call at attn (mean of H_I and H_O): k_colmax + k_colexp + k_split2
    # + k_syrk2_full + k_syrk2_split + k_syrk_reduce
    ("hessian", "attn", "23d9959685c68706"): {"fetch_kib": 2026493.2, "write_kib": 630644.3,
                                              "mfma_busy": 0.565, "clock_ghz": 1.87},
    # one LDL pair at attn (both 4096 factors in one launch): k_ldl_sched
    ("ldl", "attn", "d61a493cfa1a054e"): {"fetch_kib": 1864342.7, "write_kib": 757905.0,
                                          "mfma_busy": 0.304, "clock_ghz": 2.20},
}
# "mfma_busy" and "clock_ghz" come from a third rocprofv3 --pmc run of this script
# (GRBM_GUI_ACTIVE, SQ_VALU_MFMA_BUSY_CYCLES and the SQ_INSTS_VALU_MFMA_MOPS_* counters):
# the share of SIMD cycles in which a matrix instruction issued, and the clock the
# kernel ran at (GRBM_GUI_ACTIVE per XCD over its duration), for the main kernel of
# each kind (k_syrk2_full, the mean of the two calls; k_ldl_sched; k_solve_run).
COUNTER_SOURCES = {
    "hessian": ("bk_accum.hip", "bk_common.hpp"),
    "solve": ("bk_solve.hip", "bk_common.hpp"),
    "ldl": ("bk_ldl.hip", "bk_common.hpp"),
}


def source_key(kind):
    """Hash of the kernel sources behind `kind`, comments and blank space removed, and
    of the compiler flags they are built with."""
    import hashlib
    import re

    from kronecker_hessian_rounding_amd import build as hip_build

    csrc = os.path.join(ROOT, "kronecker_hessian_rounding_amd", "csrc")
    h = hashlib.sha256()
    for f in COUNTER_SOURCES[kind]:
        text = open(os.path.join(csrc, f)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
        h.update(" ".join(hip_build.CFLAGS[:-2] + hip_build.FILE_FLAGS.get(f, [])).encode())
    return h.hexdigest()[:16]


def mfma_counters(kind, workload):
    """MFMA-busy share and clock of the kind's main kernel from the counters, or None."""
    c = COUNTERS.get((kind, workload, source_key(kind)))
    if c is None or "mfma_busy" not in c:
        return None
    return {"mfma_busy": c["mfma_busy"], "clock_ghz": c["clock_ghz"]}


def traffic_bytes(kind, workload):
    """Calibrated HBM bytes per launch (call), or None if not measured for this source."""
    c = COUNTERS.get((kind, workload, source_key(kind)))
    if c is None:
        return None
    cal_kib = CAL_BYTES / 1024.0
    return 1024.0 * (c["fetch_kib"] * cal_kib / CAL_FETCH_KIB + c["write_kib"] * cal_kib / CAL_WRITE_KIB)


WORKLOAD_LABEL = {
    "tiny": "tiny 64x64, T=1024",
    "small": "small 512x512, T=8192",
    "attn": "attn-proj 4096x4096, T=32768",
    "mlp_down": "mlp-down 4096x14336, T=32768",
    "up70b": "70B up-proj 28672x8192, T=16384",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="attn", choices=sorted(WORKLOAD_LABEL))
    ap.add_argument("--bits", type=int, default=2)
    ap.add_argument("--rounding", default="nearest", choices=["nearest", "stochastic"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=1024, help="rows of the CPU sweep sample")
    ap.add_argument("--cpu-full", action="store_true",
                    help="time the whole oracle chain on the whole layer (the default where its work, "
                         "m n (m + n), is at most the attention shape's: about 26 s on 16 cores there)")
    ap.add_argument("--cpu-sample", action="store_true",
                    help="time a bounded sample of the oracle and extrapolate, whatever the shape")
    ap.add_argument("--hessian", default="tokens", choices=["tokens", "sketch_a", "sketch_b"],
                    help="factor estimate: X^T X / T and G^T G / T over tokens, Sketch A (alternating, "
                         "per-token weights) on the same X and G, or Sketch B from per-sequence weight "
                         "gradients")
    ap.add_argument("--iters", type=int, default=3, help="Sketch A iterations")
    ap.add_argument("--sequences", type=int, default=8, help="gradients per step for Sketch B")
    ap.add_argument("--rotate", action="store_true",
                    help="two-sided incoherence rotation of W, H_I and H_O before the LDL "
                         "(W is rotated in place every step)")
    return ap.parse_args()


def _replay(dev, LO, LI, bits, rounding, seed, rows):
    """The oracle's replay of the device's codes (all rows, or the first `rows`)."""
    if dev is None:
        return None
    import numpy as np

    import oracle

    t0 = time.perf_counter()
    w = dev["W"]
    m, n = w.shape
    if rows is None:
        rp = oracle.replay(w, LO, LI, dev["scales"], bits, dev["codes"], rounding, seed,
                           DO=dev["DO"], DI=dev["DI"])
        loss_rel = abs(dev["loss"] - rp["loss"]) / abs(rp["loss"]) if rp["loss"] else None
        what = "every entry"
    else:
        rp = oracle.replay_rows(w, LO, LI, dev["scales"], bits, dev["codes"], np.arange(rows),
                                rounding, seed)
        loss_rel = None
        what = "rows 0..%d" % (rows - 1)
    return {"entries": int(rp["y"].size), "rows": what, "mismatches": rp["mismatches"],
            "flips": rp["flips"], "max_flip_margin": rp["max_flip_margin"], "bad": rp["bad"],
            "band": 1e-4, "loss_rel": loss_rel, "seconds": time.perf_counter() - t0,
            "factors": "the device's L_O, L_I, D_O, D_I and scales"}


def cpu_baseline(w, LO, LI, x, bits, rounding, seed, rows, g=None, full=False, dev=None):
    """The oracle as it stands, timed on the host cores.

    Default: a bounded sample of the same layer, extrapolated. Phases: fp64 X^T X
    on 8192 tokens (scaled by T/8192, for H_I (T n^2) and H_O (T m^2)), the plain
    O(d^3) LDL at d=2048 (scaled by (d/2048)^3 per factor) and the row-major
    accumulator sweep on the first `rows` rows with the device's factors (scaled
    by the sweep's cost model (m^2 n + m n^2) / (r^2 n + r n^2)).

    full=True: the whole oracle chain on the whole layer, every phase measured
    (fp64 X^T X / T and G^T G / T, damping, the LDL of both factors as the oracle's
    pipeline takes it, the fp32 scales and the whole accumulator sweep).

    dev (untimed): the device's last step (W as solved, its codes, scales, D_O, D_I
    and proxy loss; LO / LI are its factors). The oracle replays the device's codes
    on the device's own factors -- every entry with full=True, the sampled rows
    otherwise -- and the counts land in the result's "replay" entry: mismatches,
    boundary flips (within 1e-4 of a grid step of the boundary between adjacent
    codes), their largest margin, bad entries, and the proxy loss agreement.
    """
    import numpy as np

    import oracle

    m, n = w.shape
    T = x.shape[0]
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    if full:
        t = {}
        t0 = time.perf_counter()
        HI = oracle.damp(oracle.hessian(x))
        HO = oracle.damp(oracle.hessian(g))
        t["hessians"] = time.perf_counter() - t0
        t0 = time.perf_counter()
        li, di = oracle.udu(HI) if n <= 2048 else oracle.udu_lapack(HI)
        lo, do = oracle.udu(HO) if m <= 2048 else oracle.udu_lapack(HO)
        t["ldl"] = time.perf_counter() - t0
        del HI, HO
        t0 = time.perf_counter()
        s = oracle.row_scales(w, bits)
        oracle.sweep(w, lo, li, s, bits, rounding, seed)
        t["sweep"] = time.perf_counter() - t0
        total = sum(t.values())
        return {
            "replay": _replay(dev, LO, LI, bits, rounding, seed, None),
            "value": m * n / total,
            "unit": "weights/s",
            "cores": cores,
            "kind": "oracle",
            "sample": ("fp64 oracle, the whole %dx%d layer measured: Hessians %.1fs, LDL of both %.1fs, "
                       "scales and accumulator sweep %.1fs; %.1fs in all" % (m, n, t["hessians"], t["ldl"],
                                                                              t["sweep"], total)),
            "solve_only_value": m * n / t["sweep"],
            "phases_s": t,
        }
    ts = min(T, 8192)
    t0 = time.perf_counter()
    oracle.hessian(x[:ts])
    t_h = (time.perf_counter() - t0) * (T / ts)
    ds = min(2048, n)
    Hs = oracle.damp(oracle.hessian(x[: 4 * ds, :ds]))
    t0 = time.perf_counter()
    oracle.udu(Hs)
    t_udu = time.perf_counter() - t0
    t_ldl = t_udu * ((n / ds) ** 3 + (m / ds) ** 3)
    r = min(rows, m)
    s = oracle.row_scales(w[:r], bits)
    lo = None if LO is None else LO[:r, :r].astype(np.float64)
    t0 = time.perf_counter()
    oracle.sweep(w[:r], lo, LI, s, bits, rounding, seed)
    t_s = time.perf_counter() - t0
    t_sweep = t_s * (m * m * n + m * n * n) / (r * r * n + r * n * n)
    t_layer = t_h * (1.0 + (m / n) ** 2) + t_ldl + t_sweep  # H_I (T n^2) and H_O (T m^2)
    return {
        "replay": _replay(dev, LO, LI, bits, rounding, seed, r),
        "value": m * n / t_layer,
        "unit": "weights/s",
        "cores": cores,
        "kind": "oracle",
        "sample": ("fp64 oracle, extrapolated to the whole %dx%d layer: X^T X on %d of %d tokens "
                   "(%.2fs measured), plain LDL at d=%d (%.2fs), accumulator sweep on the first %d "
                   "rows (%.2fs); layer estimate %.1fs (solve phase alone %.1fs = %.3g weights/s)"
                   % (m, n, ts, T, t_h * ts / T, ds, t_udu, r, t_s, t_layer, t_sweep,
                      m * n / t_sweep)),
        "solve_only_value": m * n / t_sweep,
    }


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs the BaKron path on one GPU only; --gpus %d is not "
              "supported (a layer's solve is one dependency chain; layers shard across GPUs "
              "with no communication)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import kronecker_hessian_rounding_amd as bk
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workloads.get(args.workload)
    m, n, T = wl.m, wl.n, wl.T
    # the whole oracle where it finishes in about half a minute on the host, else a sample
    args.cpu_full = not args.cpu_sample and (args.cpu_full or m * n * (m + n) <= 4096 * 4096 * 8192)
    w, x, g = workloads.make_inputs(args.workload)
    W = torch.from_numpy(w).to(dev)
    X = torch.from_numpy(x).to(dev)
    G = torch.from_numpy(g).to(dev)
    if not args.cpu_full:
        del g
    HI = torch.empty((n, n), dtype=torch.float32, device=dev)
    HO = torch.empty((m, m), dtype=torch.float32, device=dev)
    DI = torch.empty(n, dtype=torch.float32, device=dev)
    DO = torch.empty(m, dtype=torch.float32, device=dev)
    out = bk.SolveResult(codes=torch.empty((m, n), dtype=torch.uint8, device=dev),
                         scales=torch.empty(m, dtype=torch.float32, device=dev), delta=None,
                         loss=torch.empty(1, dtype=torch.float64, device=dev),
                         clamped=torch.empty(1, dtype=torch.int64, device=dev),
                         info=torch.empty(1, dtype=torch.int32, device=dev))
    seed = wl.seed_round
    # A plain device copy of known size (256 MiB read + 256 MiB written) runs once
    # before the warm-up: under a counter profiler its FETCH_SIZE / WRITE_SIZE
    # readings calibrate the counters that price the Hessian kernel's traffic.
    cal = torch.empty(CAL_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    cal_out = torch.empty_like(cal)
    cal_out.copy_(cal)
    torch.cuda.synchronize()
    del cal, cal_out
    sketch = args.hessian == "sketch_b"
    if sketch:
        grads = torch.from_numpy(workloads.make_grads(args.sequences, m, n, 5000 + wl.key)).to(dev)
    hess_phases = {"tokens": ("hess_I", "hess_O"), "sketch_b": ("hess_sketch_b",),
                   "sketch_a": ("hess_sketch_a",)}[args.hessian]
    phases = hess_phases + (("rotate",) if args.rotate else ()) + ("ldl", "solve")
    ev = {k: [] for k in phases}
    ldl_status = torch.empty(2, dtype=torch.int64, device=dev)

    def step(timed=False):
        marks = []
        if timed:
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            marks.append(e)

        def mark():
            if timed:
                e = torch.cuda.Event(enable_timing=True)
                e.record()
                marks.append(e)

        if sketch:
            bk.sketch_b(grads, HI, HO)
            mark()
        elif args.hessian == "sketch_a":
            hi, ho = bk.sketch_a(X, G, args.iters)
            HI.copy_(hi)
            HO.copy_(ho)
            mark()
        else:
            bk.hessian_accum(X, HI)
            mark()
            bk.hessian_accum(G, HO)
            mark()
        if args.rotate:
            bk.rotate_layer(W, HI, HO, seed + 1, seed + 2)
            mark()
        # the two factorisations are independent: one persistent launch serves both
        # (orders up to 8192), else two chains of launches run side by side; their
        # pivot statuses are checked once the steps have run, so the solve is queued
        # right behind them
        bk.ldl_pair(HI, HO, 0.01, DI, DO, status=ldl_status)
        mark()
        bk.solve(W, HO, HI, args.bits, args.rounding, seed, D_O=DO, D_I=DI, want_loss=True,
                 out=out)
        mark()
        return marks

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.warmup:
        bk.check_ldl_pair(ldl_status)
    all_marks = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        all_marks.append(step(timed=True))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    bk.check_ldl_pair(ldl_status)  # every step factors the same matrices
    ms_step = (t1 - t0) * 1e3 / args.steps
    for marks in all_marks:
        for k, a, b in zip(phases, marks[:-1], marks[1:]):
            ev[k].append(a.elapsed_time(b))
    ph = {k: float(np.median(v)) for k, v in ev.items()}
    info = int(out.info.item())
    loss = float(out.loss.item())
    clamped = int(out.clamped.item())

    # The Hessian calls (two per step), priced per hessian_accum call (events on the
    # stream the kernels run on); one call is the k_colmax / k_colexp / k_split2
    # pre-pass, k_syrk2_full and, when the tile count is not a whole number of
    # rounds, the split-K pair k_syrk2_split + k_syrk_reduce for the leftover tiles.
    if sketch:
        # one "call" is the whole Sketch B phase: S sequences, each an m n^2 (H_I)
        # and an n m^2 (H_O) accumulation
        syrk_ms = float(np.mean(ev["hess_sketch_b"]))
        syrk_flops = float(args.sequences) * (m * n * n + n * m * m)
    elif args.hessian == "sketch_a":
        # the whole phase in fp32-equivalent flops: the SYRKs (the initial X^T X,
        # then two per iteration, T d^2 each) and the token weights' quadratic
        # forms (T d^2 each with the symmetry of H, fp32 MFMA): one over H_I per
        # iteration, one over H_O from the second on (the first weights the
        # gradients with H_O = I)
        syrk_ms = float(np.mean(ev["hess_sketch_a"]))
        syrk_flops = float(T) * (n * n * (1 + args.iters) + m * m * args.iters
                                 + args.iters * n * n + (args.iters - 1) * m * m)
    else:
        syrk_ms = float(np.mean(ev["hess_I"] + ev["hess_O"]))
        # algorithmic fp32 flops per call, averaged over the two calls: T d^2 per
        # factor (the upper half, T d^2 / 2 FMAs at 2 flops each); the matrix cores
        # run three fp16 piece products for each
        syrk_flops = float(T) * (n * n + m * m) / 2.0
    solve_flops = float(m) * n * (m + n)            # far-field feedback, minimal
    dominant = max(ph, key=ph.get)
    fp32_equiv = syrk_flops / (syrk_ms * 1e-3) / 1e12
    roof_hess = {
        "kernel": "hessian_accum: k_colmax + k_colexp + k_split2 + k_syrk2_full (+ k_syrk2_split, "
                  "k_syrk_reduce), fp16 MFMA, three piece products per fp32 product",
        "bound": "mfma",
        "achieved": PIECE_PRODUCTS * fp32_equiv,
        "peak": PEAK_F16_MFMA_TFLOPS,
        "unit": "TFLOP/s",
        "traffic": None if args.hessian != "tokens" else traffic_bytes("hessian", args.workload),
        "flops_per_call": PIECE_PRODUCTS * syrk_flops,
        "fp32_equiv_tflops": fp32_equiv,
        "fp32_equiv_frac_of_fp32_peak": fp32_equiv / PEAK_FP32_MFMA_TFLOPS,
        "counters": None if args.hessian != "tokens" else mfma_counters("hessian", args.workload),
    }
    if args.hessian == "sketch_a":
        roof_hess.update(kernel="sketch_a phase: token-weight tile GEMMs (fp32 MFMA) and weighted SYRKs "
                                "(fp16 pieces), in fp32-equivalent flops",
                         achieved=fp32_equiv, peak=PEAK_FP32_MFMA_TFLOPS, flops_per_call=syrk_flops)
    roof_hess["frac"] = roof_hess["achieved"] / roof_hess["peak"]

    # The solve, the kernel with the most time per step at the attention shape: one
    # persistent launch, k_solve_run, behind the row scales and the factors' piece
    # pre-pass, timed per solve call. It runs the far-field GEMMs and the base case
    # together; its roofline is the one whose ideal time is longer. The far field's
    # minimum is mn(m+n) fp32 flops (two triangular long-K products), each done as
    # three fp16 piece products, against the fp16 MFMA peak. The base case's
    # algorithmic traffic is the accumulator form's 33 B per weight (W* 4, the two
    # far-field offsets 8, D 4, C 4, the pieces of D and C 8, the code 1, the
    # diagonal factor blocks about 4), against HBM. The floor of both is the chain
    # of dependent steps the schedule runs (64 x 64 leaves, a leaf-diagonal lag of 96
    # steps: (M + N - 2) 96 + 127 steps), reported beside the rule's own chain
    # (m + n - 1 anti-diagonals).
    solve_s = float(np.mean(ev["solve"])) * 1e-3  # average per call
    M, N = (m + 63) // 64, (n + 63) // 64
    chain = (M + N - 2) * 96 + 127
    base_bytes = 33.0 * m * n
    ff_flops = PIECE_PRODUCTS * solve_flops
    t_ff = ff_flops / (PEAK_F16_MFMA_TFLOPS * 1e12)
    t_base = base_bytes / (PEAK_HBM_GBS * 1e9)
    far_field = {"bound": "mfma", "flops": ff_flops, "achieved": ff_flops / solve_s / 1e12,
                 "peak": PEAK_F16_MFMA_TFLOPS, "unit": "TFLOP/s",
                 "frac": ff_flops / solve_s / 1e12 / PEAK_F16_MFMA_TFLOPS,
                 "fp32_equiv_tflops": solve_flops / solve_s / 1e12, "ideal_ms": t_ff * 1e3}
    base_case = {"bound": "hbm", "bytes": base_bytes, "achieved": base_bytes / solve_s / 1e9,
                 "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": base_bytes / solve_s / 1e9 / PEAK_HBM_GBS,
                 "ideal_ms": t_base * 1e3}
    main = far_field if t_ff >= t_base else base_case
    roof = {
        "kernel": "k_solve_run (timed as the solve call: + k_scales, k_lstats / k_lexp / k_lsplit, "
                  "k_solve_init, k_solve_finish)",
        "bound": main["bound"], "achieved": main["achieved"], "peak": main["peak"], "unit": main["unit"],
        "frac": main["frac"], "traffic": traffic_bytes("solve", args.workload),
        "time_ms": solve_s * 1e3,
        "far_field": far_field,
        "base_case": base_case,
        "chain": {"steps": chain, "ns_per_step": solve_s * 1e9 / chain, "rule_steps": m + n - 1,
                  "ns_per_rule_step": solve_s * 1e9 / (m + n - 1)},
        "counters": mfma_counters("solve", args.workload),
    }
    if roof["traffic"] is not None:
        roof["traffic_gbs"] = roof["traffic"] / solve_s / 1e9

    # The LDL pair: d^3/3 fp64 flops per factor against the fp64 MFMA peak, and its
    # chain of 64-wide diagonal blocks (the longer factor's) priced per block
    ldl_s = ph["ldl"] * 1e-3
    ldl_flops = (float(m) ** 3 + float(n) ** 3) / 3.0
    nblk = (max(m, n) + 63) // 64
    roof_ldl = {
        "kernel": ("k_ldl_sched (both factors in one persistent launch)" if max(m, n) <= 8192 else
                   "chains of launches (k_ldl_panel, k_ldl_diag_update, k_ldl_outer) on two streams"),
        "bound": "mfma", "flops": ldl_flops, "achieved": ldl_flops / ldl_s / 1e12,
        "peak": PEAK_FP64_MFMA_TFLOPS, "unit": "TFLOP/s",
        "frac": ldl_flops / ldl_s / 1e12 / PEAK_FP64_MFMA_TFLOPS,
        "traffic": traffic_bytes("ldl", args.workload),
        "chain": {"blocks": nblk, "us_per_block": ldl_s * 1e6 / nblk},
        "counters": mfma_counters("ldl", args.workload),
    }

    res = {
        "metric": "BaKron ms/layer + weights/s at 4096x4096 2-bit; % of MFMA / HBM roofline",
        "value": m * n / (ms_step * 1e-3),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "dtype_detail": "Hessian: fp32 products as three fp16 piece products of power-of-two-scaled "
                        "columns, fp32 accumulate; LDL: fp64; solve: fp32 (far field: three fp16 piece products "
                        "per fp32 product, fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": "%s, %d-bit %s" % (WORKLOAD_LABEL[args.workload], args.bits,
                                                  args.rounding),
                   "m": m, "n": n, "tokens": T, "bits": args.bits, "rounding": args.rounding,
                   "damp_rel": 0.01, "leaf": 64, "rotate": bool(args.rotate),
                   "hessian": args.hessian + (" x %d sequences" % args.sequences if sketch else "")
                   + (" x %d iterations" % args.iters if args.hessian == "sketch_a" else "")},
        "phases_ms": ph,
        "dominant_phase": dominant,
        "solve_ms": ph["solve"],
        "solve_weights_per_s": m * n / (ph["solve"] * 1e-3),
        "solve_gemm_tflops": solve_flops / (ph["solve"] * 1e-3) / 1e12,
        "ldl_fp64_tflops": (m ** 3 + n ** 3) / 3.0 / (ph["ldl"] * 1e-3) / 1e12,
        "roofline": roof,
        "roofline_hessian": roof_hess,
        "roofline_ldl": roof_ldl,
        "proxy_loss": loss,
        "clamped": clamped,
        "info": info,
    }
    if args.rotate:
        # algorithmic HBM bytes of the rotation: every pass reads and writes its
        # matrix once; a column rotation of order d takes ceil(k / 6) passes
        # (k = the power of two in d), a row rotation one
        def col_passes(dim):
            k = (dim & -dim).bit_length() - 1
            return max(1, (k + 5) // 6)
        rot_bytes = 8.0 * (m * n * (col_passes(m) + 1) + n * n * (col_passes(n) + 1)
                           + m * m * (col_passes(m) + 1))
        res["rotate_ms"] = ph["rotate"]
        res["rotate_hbm_gbs"] = rot_bytes / (ph["rotate"] * 1e-3) / 1e9
        res["rotate_bytes"] = rot_bytes
    # the layer's bound terms from the last step's factors and scales (untimed;
    # the traces of H are not kept past the LDL, so they are left out)
    rep = bk.layer_report(DO, DI, out.scales)
    res["bound"] = {k: rep[k] for k in ("tr_DO", "tr_DI", "bound_sharp", "bound_page")}
    if not args.no_cpu_baseline:
        LI = np.triu(HI.cpu().numpy(), 1).astype(np.float64)
        LO = HO.cpu().numpy()
        dev_out = {"W": W.cpu().numpy(), "codes": out.codes.cpu().numpy(),
                   "scales": out.scales.cpu().numpy(), "DO": DO.cpu().numpy().astype(np.float64),
                   "DI": DI.cpu().numpy().astype(np.float64), "loss": loss}
        res["cpu_baseline"] = cpu_baseline(w, LO, LI, x, args.bits, args.rounding, seed,
                                           args.cpu_rows, g if args.cpu_full else None, args.cpu_full,
                                           dev_out)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

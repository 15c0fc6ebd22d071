"""Benchmark of the BaKron per-layer hot path on one MI355X.

One step = the whole path for one layer on synthetic inputs already resident
in HBM: H_I = X^T X / T and H_O = G^T G / T (fp32 products formed from three
bf16 pieces per operand on the bf16 matrix cores), damping + LDL of
both (fp64), fp32 per-row scales, and the BaKron rounding solve with its proxy
loss. Default workload: the attention-projection shape, W* 4096 x 4096,
T = 32768 tokens, 2-bit nearest rounding.

Prints ONE JSON line. `value` is layer throughput in weights/s (m*n per step
time); per-phase times, the solve-only rate, the roofline of the dominant
kernel (timed with HIP events on the stream it runs on) and the CPU oracle
baseline (on a bounded sample, extrapolated to the whole layer) ride along.
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
PEAK_BF16_MFMA_TFLOPS = 2500.0
PIECE_PRODUCTS = 6  # bf16 piece products per fp32 product in the Hessian
PEAK_FP64_MFMA_TFLOPS = 78.6
CAL_BYTES = 256 << 20

# HBM traffic of one hessian_accum call at the attn workload, from two
# rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE; KiB per
# dispatch, summed over the call's k_split3, k_syrk3_full, k_syrk3_split and
# k_syrk_reduce). The counters are scaled by what they read for the
# calibration copy above: FETCH_SIZE 131089.0 KiB and WRITE_SIZE 262144.0 KiB
# for 262144 KiB moved each way. Valid only for the kernel source it was
# measured on (hash of bk_accum.hip, which holds the SYRK kernels); otherwise
# reported null.
SYRK_COUNTERS = {
    ("attn", "7e36cee6be0cd9f7"): {"fetch_kib": 2270509.1, "write_kib": 887728.2},
}
CAL_FETCH_KIB, CAL_WRITE_KIB = 131089.0, 262144.0


def syrk_traffic_bytes(workload):
    """Calibrated HBM bytes per hessian_accum call, or None if not measured for this source."""
    import hashlib
    csrc = os.path.join(ROOT, "kronecker_hessian_rounding_amd", "csrc")
    key = (workload, hashlib.sha256(open(os.path.join(csrc, "bk_accum.hip"), "rb").read()).hexdigest()[:16])
    c = SYRK_COUNTERS.get(key)
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


def cpu_baseline(w, LO, LI, x, bits, rounding, seed, rows):
    """The oracle as it stands, on a bounded sample of the same layer, extrapolated.

    Phases: fp64 X^T X on 8192 tokens (scaled by T/8192, twice: H_I and H_O of
    the same size class), the plain O(d^3) LDL at d=2048 (scaled by (d/2048)^3
    per factor) and the row-major accumulator sweep on the first `rows` rows
    with the device's factors (scaled by the sweep's cost model
    (m^2 n + m n^2) / (r^2 n + r n^2)).
    """
    import numpy as np

    import oracle

    m, n = w.shape
    T = x.shape[0]
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
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
    w, x, g = workloads.make_inputs(args.workload)
    W = torch.from_numpy(w).to(dev)
    X = torch.from_numpy(x).to(dev)
    G = torch.from_numpy(g).to(dev)
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
        # the two factorisations are independent and each a chain of small launches:
        # they run side by side on two streams
        bk.ldl_pair(HI, HO, 0.01, DI, DO)
        mark()
        bk.solve(W, HO, HI, args.bits, args.rounding, seed, D_O=DO, D_I=DI, want_loss=True,
                 out=out)
        mark()
        return marks

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    all_marks = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        all_marks.append(step(timed=True))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    for marks in all_marks:
        for k, a, b in zip(phases, marks[:-1], marks[1:]):
            ev[k].append(a.elapsed_time(b))
    ph = {k: float(np.median(v)) for k, v in ev.items()}
    info = int(out.info.item())
    loss = float(out.loss.item())
    clamped = int(out.clamped.item())

    # Roofline of the kernel with the most time per step, the Hessian SYRK (two
    # calls per step). Timed per hessian_accum call (events on the stream the
    # kernels run on); one call is the k_split3 pre-pass, k_syrk3_full and, when
    # the tile count is not a whole number of rounds, the split-K pair
    # k_syrk3_split + k_syrk_reduce for the leftover tiles.
    if sketch:
        # one "call" is the whole Sketch B phase: S sequences, each an m n^2 (H_I)
        # and an n m^2 (H_O) accumulation
        syrk_ms = float(np.mean(ev["hess_sketch_b"]))
        syrk_flops = float(args.sequences) * (m * n * n + n * m * m)
    elif args.hessian == "sketch_a":
        # the whole phase in fp32-equivalent flops: the SYRKs (the initial X^T X,
        # then two per iteration, T d^2 each) and the token weights' quadratic
        # forms (2 T d^2 per factor and iteration, fp32 MFMA)
        syrk_ms = float(np.mean(ev["hess_sketch_a"]))
        syrk_flops = float(T) * (n * n * (1 + args.iters) + m * m * args.iters
                                 + 2.0 * args.iters * (n * n + m * m))
    else:
        syrk_ms = float(np.mean(ev["hess_I"] + ev["hess_O"]))
        # algorithmic fp32 flops per call, averaged over the two calls: T d^2 per
        # factor (the upper half, T d^2 / 2 FMAs at 2 flops each); the matrix cores
        # run six bf16 piece products for each
        syrk_flops = float(T) * (n * n + m * m) / 2.0
    solve_flops = float(m) * n * (m + n)            # far-field feedback, minimal
    dominant = max(ph, key=ph.get)
    fp32_equiv = syrk_flops / (syrk_ms * 1e-3) / 1e12
    roof = {
        "kernel": "hessian_accum: k_split3 + k_syrk3_full (+ k_syrk3_split, k_syrk_reduce), "
                  "bf16 MFMA, six piece products per fp32 product",
        "bound": "mfma",
        "achieved": PIECE_PRODUCTS * fp32_equiv,
        "peak": PEAK_BF16_MFMA_TFLOPS,
        "unit": "TFLOP/s",
        "traffic": None if args.hessian != "tokens" else syrk_traffic_bytes(args.workload),
        "flops_per_call": PIECE_PRODUCTS * syrk_flops,
        "fp32_equiv_tflops": fp32_equiv,
        "fp32_equiv_frac_of_fp32_peak": fp32_equiv / PEAK_FP32_MFMA_TFLOPS,
    }
    if args.hessian == "sketch_a":
        roof.update(kernel="sketch_a phase: token-weight tile GEMMs (fp32 MFMA) and weighted SYRKs "
                           "(bf16 pieces), in fp32-equivalent flops",
                    achieved=fp32_equiv, peak=PEAK_FP32_MFMA_TFLOPS, flops_per_call=syrk_flops)
    roof["frac"] = roof["achieved"] / roof["peak"]

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
        "dtype_detail": "Hessian: fp32 products as six bf16 piece products, fp32 accumulate; "
                        "LDL: fp64; solve: fp32",
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
        res["cpu_baseline"] = cpu_baseline(w, LO, LI, x, args.bits, args.rounding, seed,
                                           args.cpu_rows)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

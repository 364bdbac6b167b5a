#!/usr/bin/env python3
"""Benchmark: one MXFP4 linear-layer training step on MI355X (gfx950).

A step is the whole hot path once, on the Flux-12B MLP fc2 shape
(tokens 18432, in 12288, out 3072):
  dual-quantize X (1D, RNE)  dual-quantize W (32x32 2D blocks, RNE)
  GEMM fwd    Y  = X_row  . W_row^T        (18432 x 3072,  K 12288)
  dual-quantize dY (stochastic rounding, seed 7, tensor id 2)
  GEMM dgrad  dX = dY_row . W_col^T        (18432 x 12288, K 3072)
  GEMM wgrad  dW = dY_col . X_col^T        (3072 x 12288,  K 18432)
All blobs in the tiled layout, bf16 outputs, fp32 accumulation.  Inputs are
seeded synthetic tensors already resident in HBM when timing starts.

Prints one JSON line: value = GEMM TFLOP/s of the whole step (3 GEMMs' flops
over the step's wall time), per-kernel timings from HIP events on the launch
stream, a roofline object for the dominant kernel (the GEMM, dense MXFP4 MFMA
peak) and one for the dual quantizer (HBM), and the CPU oracle timed on a
bounded sample of the same step.  "extras" times, on the same tensors, the
library's options the step does not use: the random Hadamard transform on
the column-wise blobs (the recipe's wgrad operands), the bias epilogue of the
forward GEMM, the device layout conversion, and the hybrid backward's
tensorwise FP8 quantize and FP8 dgrad/wgrad GEMMs.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "a4w4 GEMM TFLOP/s + dual-quantize GB/s (% roofline), Flux-12B-shaped linears"
PEAK_FP4_TFLOPS = 10100.0      # MI355X dense MXFP4 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
VALU_ISSUE_PEAK_G = 1024 * 2.4 / 4   # G wave64 VALU instructions/s: 256 CUs x 4 SIMDs, 16 lanes/clock, 2.4 GHz


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    # the GPU's clocks settle over the first ~20 ms of back-to-back steps (the first
    # timed steps after 3 warmups ran ~7% slower than the steady state)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--tokens", type=int, default=18432)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the timings of the options outside the step (RHT, bias epilogue, layout conversion)")
    p.add_argument("--cpu-tokens", type=int, default=96,
                   help="token slice of the step the CPU oracle is timed on")
    p.add_argument("--profile-copy-mib", type=int, default=0,
                   help="run one plain device copy of this many MiB first (a known-size kernel "
                        "that calibrates rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    p.add_argument("--workload", default="fc2_step", choices=["fc2_step"] + sorted(WORKLOADS),
                   help="fc2_step (default): the bench line.  Any other: only that workload's kernels, "
                        "--steps passes of them after --warmup, per-kernel event timings in one JSON line "
                        "(for rocprofv3 runs of one configuration)")
    return p.parse_args()


# Workloads other than the fc2 step, by name: what each pass runs.  Small
# inputs cycle through buffer sets larger than twice the 256 MB Infinity Cache
# so that every pass reads from HBM.
WORKLOADS = {
    "dual_4600x3072": "dual quantize 4600x3072 (N(0,1), 0.1% outliers x100, a zero 32x32 tile per 1024 rows)",
    "qkv": "QKV forward: A 4608x3072 and W 9216x3072 row-wise quantize, GEMM 4608 x 9216 x 3072",
    "fc1_step": "MLP fc1 step: X 9216x3072, W 12288x3072, dY 9216x12288 dual quantize; fwd, dgrad, wgrad",
    "fc2_w2d": "fc2 weight 3072x12288 dual quantize with 32x32 blocks",
}


def run_workload(args):
    """--workload NAME: that workload's kernels only, each timed over `steps`
    batches of back-to-back launches with HIP events on the launch stream."""
    import torch
    import mxfp4_precision_amd as mx
    from mxfp4_precision_amd import synth

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    mx.lib()
    dev = torch.device("cuda:0")
    T = mx.MX_LAYOUT_TILED
    plain = mx.quant_opts()
    stream = torch.cuda.current_stream()
    MALL = 256 << 20

    def dev_bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev)

    def dual_bytes(M, N):
        d1, s1 = mx.mx_blob_bytes(M, N, T)
        d2, s2 = mx.mx_blob_bytes(N, M, T)
        return 2.0 * M * N + d1 + s1 + d2 + s2

    def row_bytes(M, N):
        return 2.0 * M * N + sum(mx.mx_blob_bytes(M, N, T))

    def sets_for(nbytes):
        return max(2, -(-2 * MALL // int(nbytes)) + 1)

    if args.profile_copy_mib:
        n = args.profile_copy_mib << 20
        src = torch.ones(n // 2, dtype=torch.int16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    kernels = []   # (name, fn(i), nsets, bytes or None, flops or None)
    if args.workload in ("dual_4600x3072", "fc2_w2d"):
        if args.workload == "dual_4600x3072":
            x0, opts = dev_bf16(synth.dual()["X"]), plain
        else:
            x0, opts = dev_bf16(synth.fc2()["W"]), mx.quant_opts(use_2d_block=True, tensor_id=1)
        M, N = x0.shape
        n = sets_for(dual_bytes(M, N))
        xs = [x0] + [x0.clone() for _ in range(n - 1)]
        outs = [mx.empty_blob(M, N, T, dev) + mx.empty_blob(N, M, T, dev) for _ in range(n)]
        kernels.append(("quant_dual", lambda i: mx.mx_quantize_dual(xs[i], M, N, N, opts, opts, T, *outs[i], stream),
                        n, dual_bytes(M, N), None))
    elif args.workload == "qkv":
        d = synth.qkv()
        a0, w0 = dev_bf16(d["A"]), dev_bf16(d["W"])
        (M, K), N = a0.shape, w0.shape[0]
        na, nw = sets_for(row_bytes(M, K)), sets_for(row_bytes(N, K))
        a_s = [a0] + [a0.clone() for _ in range(na - 1)]
        w_s = [w0] + [w0.clone() for _ in range(nw - 1)]
        ab = [mx.empty_blob(M, K, T, dev) for _ in range(na)]
        wb = [mx.empty_blob(N, K, T, dev) for _ in range(nw)]
        kernels.append(("quant_A", lambda i: mx.mx_quantize_rowwise(a_s[i], M, K, K, plain, T, *ab[i], stream),
                        na, row_bytes(M, K), None))
        kernels.append(("quant_W", lambda i: mx.mx_quantize_rowwise(w_s[i], N, K, K, plain, T, *wb[i], stream),
                        nw, row_bytes(N, K), None))
        for i in range(na):
            mx.mx_quantize_rowwise(a_s[i], M, K, K, plain, T, *ab[i], stream)
        for i in range(nw):
            mx.mx_quantize_rowwise(w_s[i], N, K, K, plain, T, *wb[i], stream)
        ng = sets_for(sum(t.numel() for t in ab[0] + wb[0]) + 2.0 * M * N)
        Cs = [torch.empty((M, N), dtype=torch.int16, device=dev) for _ in range(ng)]
        kernels.append(("gemm_fwd", lambda i: mx.mx_gemm_a4w4(0, 1, M, N, K, *ab[i % na], *wb[i % nw], T, mx.MX_BF16,
                                                              Cs[i], N, stream), ng, None, 2.0 * M * N * K))
    elif args.workload == "fc1_step":
        d = synth.fc1()
        X, W, G = dev_bf16(d["X"]), dev_bf16(d["W"]), dev_bf16(d["dY"])
        (Tk, din), dout = X.shape, W.shape[0]
        bl = {}
        for name, t in (("X", X), ("W", W), ("dY", G)):
            M, N = t.shape
            bl[name] = mx.empty_blob(M, N, T, dev) + mx.empty_blob(N, M, T, dev)
            kernels.append(("quant_" + name, (lambda t, M, N, b: lambda i: mx.mx_quantize_dual(
                t, M, N, N, plain, plain, T, *b, stream))(t, M, N, bl[name]), 1, dual_bytes(M, N), None))
        Y = torch.empty((Tk, dout), dtype=torch.int16, device=dev)
        dX = torch.empty((Tk, din), dtype=torch.int16, device=dev)
        dW = torch.empty((dout, din), dtype=torch.int16, device=dev)
        xb, wb, gb = bl["X"], bl["W"], bl["dY"]
        for name, (M, N, K, A_, As_, B_, Bs_, C_, ldc) in (
                ("fwd", (Tk, dout, din, xb[0], xb[1], wb[0], wb[1], Y, dout)),
                ("dgrad", (Tk, din, dout, gb[0], gb[1], wb[2], wb[3], dX, din)),
                ("wgrad", (dout, din, Tk, gb[2], gb[3], xb[2], xb[3], dW, din))):
            kernels.append(("gemm_" + name, (lambda M, N, K, A_, As_, B_, Bs_, C_, ldc: lambda i: mx.mx_gemm_a4w4(
                0, 1, M, N, K, A_, As_, B_, Bs_, T, mx.MX_BF16, C_, ldc, stream))(M, N, K, A_, As_, B_, Bs_, C_, ldc),
                1, None, 2.0 * M * N * K))

    # Each kernel timed on its own: batches of 20 back-to-back launches (rotating
    # buffer sets) between two events on the launch stream, so that host
    # enqueue time never shows between launches; median, mean and minimum
    # over `steps` batches after `warmup` untimed launches.
    per = 20
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    res = {}
    for name, fn, nsets, nbytes, fl in kernels:
        for i in range(max(args.warmup, 2 * nsets)):
            fn(i % nsets)
        torch.cuda.synchronize()
        t = []
        for b in range(args.steps):
            ev[0].record(stream)
            for j in range(per):
                fn((b * per + j) % nsets)
            ev[1].record(stream)
            ev[1].synchronize()
            t.append(ev[0].elapsed_time(ev[1]) / per)
        ms = float(np.median(t))
        entry = {"ms": round(ms, 5), "ms_mean": round(float(np.mean(t)), 5), "ms_min": round(float(np.min(t)), 5),
                 "buffer_sets": nsets}
        if nbytes:
            entry["GB/s"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
            entry["frac_hbm_peak"] = round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        if fl:
            entry["TFLOP/s"] = round(fl / (ms * 1e-3) / 1e12, 1)
            entry["frac_fp4_peak"] = round(fl / (ms * 1e-3) / 1e12 / PEAK_FP4_TFLOPS, 4)
        res[name] = entry
    print(json.dumps({"workload": args.workload, "what": WORKLOADS[args.workload], "batches": args.steps,
                      "launches_per_batch": per, "warmup": args.warmup, "kernels": res}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: libmxfp4 has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.workload != "fc2_step":
        run_workload(args)
        return

    import torch
    import mxfp4_precision_amd as mx
    from mxfp4_precision_amd import synth

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    mx.lib()   # raises if libmxfp4.so is missing: there is no fallback
    dev = torch.device("cuda:0")
    T = mx.MX_LAYOUT_TILED

    tokens, din, dout = args.tokens, 12288, 3072
    t0 = time.time()
    data = synth.fc2(tokens=tokens)
    gen_s = time.time() - t0
    X = torch.from_numpy(data["X"].view(np.int16)).to(dev)
    W = torch.from_numpy(data["W"].view(np.int16)).to(dev)
    dY = torch.from_numpy(data["dY"].view(np.int16)).to(dev)

    def blob(rows, length):
        return mx.empty_blob(rows, length, T, dev)

    Xr, Xrs = blob(tokens, din); Xc, Xcs = blob(din, tokens)
    Wr, Wrs = blob(dout, din); Wc, Wcs = blob(din, dout)
    Gr, Grs = blob(tokens, dout); Gc, Gcs = blob(dout, tokens)
    Y = torch.empty((tokens, dout), dtype=torch.int16, device=dev)
    dX = torch.empty((tokens, din), dtype=torch.int16, device=dev)
    dW = torch.empty((dout, din), dtype=torch.int16, device=dev)

    if args.profile_copy_mib:
        n = args.profile_copy_mib << 20
        src = torch.ones(n // 2, dtype=torch.int16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    o_plain = mx.quant_opts()
    o_w = mx.quant_opts(use_2d_block=True, tensor_id=1)
    o_g = mx.quant_opts(use_sr=True, seed=7, tensor_id=2)
    stream = torch.cuda.current_stream()

    names = ["quant_X", "quant_W", "gemm_fwd", "quant_dY", "gemm_dgrad", "gemm_wgrad"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        mx.mx_quantize_dual(X, tokens, din, din, o_plain, o_plain, T, Xr, Xrs, Xc, Xcs, stream)
        mark(1)
        mx.mx_quantize_dual(W, dout, din, din, o_w, o_w, T, Wr, Wrs, Wc, Wcs, stream)
        mark(2)
        mx.mx_gemm_a4w4(0, 1, tokens, dout, din, Xr, Xrs, Wr, Wrs, T, mx.MX_BF16, Y, dout, stream)
        mark(3)
        mx.mx_quantize_dual(dY, tokens, dout, dout, o_g, o_g, T, Gr, Grs, Gc, Gcs, stream)
        mark(4)
        mx.mx_gemm_a4w4(0, 1, tokens, din, dout, Gr, Grs, Wc, Wcs, T, mx.MX_BF16, dX, din, stream)
        mark(5)
        mx.mx_gemm_a4w4(0, 1, dout, din, tokens, Gc, Gcs, Xc, Xcs, T, mx.MX_BF16, dW, din, stream)
        mark(6)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: exactly K steps, wall clock between synchronizations.
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = 1e3 * wall / args.steps

    # Per-kernel durations: events recorded between launches on the launch stream.
    evsets = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    for k in range(args.steps):
        step(evsets[k])
    torch.cuda.synchronize()
    samples = {n: [evs[i].elapsed_time(evs[i + 1]) for evs in evsets] for i, n in enumerate(names)}
    per = {n: float(np.mean(v)) for n, v in samples.items()}

    gemm_shapes = {"gemm_fwd": (tokens, dout, din), "gemm_dgrad": (tokens, din, dout),
                   "gemm_wgrad": (dout, din, tokens)}
    flops = {n: 2.0 * m * n_ * k for n, (m, n_, k) in gemm_shapes.items()}
    step_flops = sum(flops.values())
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    def qbytes(M, N):
        d1, s1 = mx.mx_blob_bytes(M, N, T)
        d2, s2 = mx.mx_blob_bytes(N, M, T)
        return 2.0 * M * N + d1 + s1 + d2 + s2
    qb = {"quant_X": qbytes(tokens, din), "quant_W": qbytes(dout, din), "quant_dY": qbytes(tokens, dout)}

    kernels = {}
    for n in names:
        entry = {"ms": round(per[n], 5), "ms_median": round(float(np.median(samples[n])), 5),
                 "ms_min": round(float(np.min(samples[n])), 5)}
        if n in flops:
            entry["TFLOP/s"] = round(flops[n] / (per[n] * 1e-3) / 1e12, 1)
            entry["frac_fp4_peak"] = round(flops[n] / (per[n] * 1e-3) / 1e12 / PEAK_FP4_TFLOPS, 4)
        else:
            entry["GB/s"] = round(qb[n] / (per[n] * 1e-3) / 1e9, 1)
            entry["frac_hbm_peak"] = round(qb[n] / (per[n] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        kernels[n] = entry

    traffic = load_traffic()
    # Dominant kernel: the GEMM (one kernel, three launches of equal flops per launch).
    gemm_ms = float(np.mean([per[n] for n in gemm_shapes]))
    gemm_achieved = (step_flops / 3) / (gemm_ms * 1e-3) / 1e12
    # Dual quantizer roofline on the largest launch (X: 18432 x 12288).
    qx_gbs = qb["quant_X"] / (per["quant_X"] * 1e-3) / 1e9

    def enqueue_us(fn, n=200):
        """Host time per call (Python binding + C-ABI validation + launch), no sync per call."""
        torch.cuda.synchronize()
        t = []
        for i in range(n):
            t0 = time.perf_counter()
            fn()
            t.append(time.perf_counter() - t0)
            if i % 20 == 19:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        return round(float(np.median(t)) * 1e6, 2)

    def measured_ceilings():
        """What this chip sustains with no algorithm around it: the FP4 matrix
        instruction's rate on the step's own X codes and on uniform random codes
        (mx_measure_mfma, E2M1 x E2M1), and a plain 1 GiB device copy."""
        gen = torch.Generator(device="cpu").manual_seed(11)
        uniform = torch.randint(0, 256, (16384,), generator=gen, dtype=torch.uint8).to(dev)
        res = {"mfma_fp4_x_codes_TFLOP/s": mfma_rate(mx, torch, dev, stream, 4, 4, Xr),
               "mfma_fp4_uniform_codes_TFLOP/s": mfma_rate(mx, torch, dev, stream, 4, 4, uniform)}
        src = torch.empty((1 << 30,), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        reps = 5
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(reps):
            dst.copy_(src)
        ev[1].record(stream)
        torch.cuda.synchronize()
        res["copy_1GiB_GB/s"] = round(2.0 * (1 << 30) / (ev[0].elapsed_time(ev[1]) / reps * 1e-3) / 1e9, 1)
        del src, dst
        res["what"] = ("MFMA-only loop (8 waves per CU, 4 accumulator chains, operands switching every instruction) "
                       "on the fc2 X blob's first 16 KB of E2M1 codes and on uniform random codes; torch device copy "
                       "of 1 GiB (read + write bytes)")
        return res

    def telemetry(nsteps=60):
        """Power cap, memory clock, the clock table with its current level, and the
        power drawn (hwmon power1_input sampled every ~2 ms by a host thread) while
        the step runs back to back and while the MFMA-only loop runs, from the
        card's sysfs files; empty if they are not readable."""
        import glob
        import threading
        cards = [d for d in sorted(glob.glob("/sys/class/drm/card*/device")) if os.path.exists(d + "/pp_dpm_sclk")]
        if len(cards) != 1:
            return {"note": "%d cards with clock tables visible; not sampled" % len(cards)}
        dev_dir = cards[0]
        hw = sorted(glob.glob(dev_dir + "/hwmon/hwmon*"))

        def read(path):
            try:
                return open(path).read().strip()
            except OSError:
                return None

        res = {}
        cap = read(hw[0] + "/power1_cap") if hw else None
        if cap:
            res["power_cap_W"] = round(int(cap) / 1e6, 1)
        mclk = [l for l in (read(dev_dir + "/pp_dpm_mclk") or "").splitlines() if l.endswith("*")]
        if mclk:
            res["mclk"] = mclk[0].split(":", 1)[1].strip(" *")
        res["sclk_levels"] = ", ".join(l.strip() for l in (read(dev_dir + "/pp_dpm_sclk") or "").splitlines())
        if not hw or read(hw[0] + "/power1_input") is None:
            return res
        def sampled(run):
            samples, sclk, stop = [], [], threading.Event()

            def sampler():
                while not stop.is_set():
                    v = read(hw[0] + "/power1_input")
                    if v:
                        samples.append(int(v) / 1e6)
                    cur = [l for l in (read(dev_dir + "/pp_dpm_sclk") or "").splitlines() if l.endswith("*")]
                    if cur:
                        try:
                            sclk.append(int(cur[0].split(":", 1)[1].strip(" *").lower().replace("mhz", "")))
                        except ValueError:
                            pass
                    time.sleep(0.002)
            run()
            torch.cuda.synchronize()
            th = threading.Thread(target=sampler)
            th.start()
            run()
            torch.cuda.synchronize()
            stop.set()
            th.join()
            if not samples:
                return None
            return {"power_W_mean": round(float(np.mean(samples)), 1), "power_W_max": round(float(np.max(samples)), 1),
                    "sclk_MHz_min_max": [min(sclk), max(sclk)] if sclk else None, "samples": len(samples)}

        def steps():
            for _ in range(nsteps):
                step()
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        ops = torch.randint(0, 256, (16384,), generator=torch.Generator(device="cpu").manual_seed(11),
                            dtype=torch.uint8).to(dev)
        obuf = torch.empty((cus * 512,), dtype=torch.float32, device=dev)

        def mfma_loop():
            for _ in range(10):
                mx.mx_measure_mfma(4, 4, ops, cus, 40000, obuf, stream)
        res["during_steps"] = sampled(steps)
        res["during_mfma_only_loop"] = sampled(mfma_loop)
        return res

    ceilings = None if args.no_extras else measured_ceilings()
    if ceilings is not None:
        ceilings["telemetry"] = telemetry()
    host_enqueue = None if args.no_extras else {
        "mx_quantize_dual_us": enqueue_us(lambda: mx.mx_quantize_dual(X, tokens, din, din, o_plain, o_plain, T, Xr,
                                                                      Xrs, Xc, Xcs, stream)),
        "mx_gemm_a4w4_us": enqueue_us(lambda: mx.mx_gemm_a4w4(0, 1, tokens, dout, din, Xr, Xrs, Wr, Wrs, T,
                                                              mx.MX_BF16, Y, dout, stream)),
        "what": "median host time per call through the Python binding (ctypes) and the C ABI, no "
                "synchronization per call"}
    extras = None if args.no_extras else time_extras(mx, torch, dev, stream, X, W, dY, tokens, din, dout,
                                                      Xr, Xrs, Wr, Wrs, qb, flops["gemm_fwd"])
    if extras is not None:
        extras["other_workloads"] = time_other_workloads(mx, torch, dev, stream, synth)
        extras["host_enqueue"] = host_enqueue

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4 (e2m1 x e2m1, e8m0 scales, fp32 accumulate, bf16 out)",
        "data": "synthetic (seeded numpy PCG64, Flux-12B MLP fc2 shapes; random values, no weights)",
        "config": {"workload": "MLP fc2 train step: X %dx%d GELU(N(0,1)), W %dx%d N(0,0.02) 2D-block, "
                               "dY %dx%d N(0,1e-3) SR; dual quantize x3 + fwd/dgrad/wgrad a4w4 GEMMs"
                               % (tokens, din, dout, din, tokens, dout),
                   "tokens": tokens, "in_features": din, "out_features": dout,
                   "layout": "tiled", "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": "mx_gemm_a4w4", "bound": "mfma",
                     "achieved": round(gemm_achieved, 1), "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_achieved / PEAK_FP4_TFLOPS, 4),
                     "traffic": traffic.get("gemm") if traffic else None},
        "roofline_quantize": {"kernel": "mx_quantize_dual (X %dx%d)" % (tokens, din), "bound": "hbm",
                              "achieved": round(qx_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                              "frac": round(qx_gbs / PEAK_HBM_GBS, 4),
                              "traffic": traffic.get("quant_X") if traffic else None},
        "kernels": kernels,
        "input_gen_s": round(gen_s, 1),
    }
    # The stochastic-rounding dual quantize is bound by its VALU work (Philox
    # rounds and the encode), not by HBM: its wave-level VALU instructions per
    # launch (SQ_INSTS_VALU from the committed counter profile, valid while
    # the sources match) over the live event-timed duration, against the
    # chip's VALU issue ceiling: 1024 SIMDs x one wave64 instruction per 4
    # cycles (16 lanes per clock) at 2.4 GHz.
    if traffic and traffic.get("quant_dY_valu_insts"):
        insts = traffic["quant_dY_valu_insts"]
        rate = insts / (per["quant_dY"] * 1e-3) / 1e9
        out["roofline_quantize_sr"] = {
            "kernel": "mx_quantize_dual (dY %dx%d, stochastic rounding both blobs)" % (tokens, dout),
            "bound": "alu", "achieved": round(rate, 1), "peak": VALU_ISSUE_PEAK_G, "unit": "G VALU wave-instructions/s",
            "frac": round(rate / VALU_ISSUE_PEAK_G, 4),
            "valu_insts_per_element": round(insts / (tokens * dout), 4),
            "hbm_frac": kernels["quant_dY"]["frac_hbm_peak"]}
    if extras is not None:
        out["extras"] = extras

    if ceilings is not None:
        ceilings["gemm_frac_of_x_codes_rate"] = round(gemm_achieved / ceilings["mfma_fp4_x_codes_TFLOP/s"], 4)
        ceilings["quant_X_frac_of_copy"] = round(qx_gbs / ceilings["copy_1GiB_GB/s"], 4)
        out["measured_ceilings"] = ceilings
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(data, args.cpu_tokens, din, dout)
    print(json.dumps(out), flush=True)


def time_extras(mx, torch, dev, stream, X, W, dY, tokens, din, dout, Xr, Xrs, Wr, Wrs, qb, fwd_flops, reps=10):
    """Event-timed launches (mean of `reps` after 2 warmups) of the options outside the step."""
    T = mx.MX_LAYOUT_TILED

    def timed(fn):
        for _ in range(2):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(reps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    plain = mx.quant_opts()
    rht = mx.quant_opts(rht=0x5248)
    sr = mx.quant_opts(use_sr=True, seed=7, tensor_id=2)
    sr_rht = mx.quant_opts(use_sr=True, seed=7, tensor_id=2, rht=0x5248)
    qr, qrs = mx.empty_blob(tokens, din, T, dev); qc, qcs = mx.empty_blob(din, tokens, T, dev)
    gr, grs = mx.empty_blob(tokens, dout, T, dev); gc, gcs = mx.empty_blob(dout, tokens, T, dev)
    out = {}
    ms = timed(lambda: mx.mx_quantize_dual(X, tokens, din, din, plain, rht, T, qr, qrs, qc, qcs, stream))
    out["quant_X_col_rht"] = {"ms": round(ms, 5), "GB/s": round(qb["quant_X"] / (ms * 1e-3) / 1e9, 1),
                              "what": "X dual, column-wise blob with the random Hadamard transform"}
    ms = timed(lambda: mx.mx_quantize_dual(dY, tokens, dout, dout, sr, sr_rht, T, gr, grs, gc, gcs, stream))
    out["quant_dY_sr_col_rht"] = {"ms": round(ms, 5), "GB/s": round(qb["quant_dY"] / (ms * 1e-3) / 1e9, 1),
                                  "what": "dY dual, stochastic rounding, column-wise blob transformed"}
    bias = torch.zeros((dout,), dtype=torch.int16, device=dev)
    Yb = torch.empty((tokens, dout), dtype=torch.int16, device=dev)
    ms = timed(lambda: mx.mx_gemm_a4w4_bias(0, 1, tokens, dout, din, Xr, Xrs, Wr, Wrs, T, mx.MX_BF16, bias, Yb,
                                            dout, stream))
    out["gemm_fwd_bias"] = {"ms": round(ms, 5), "TFLOP/s": round(fwd_flops / (ms * 1e-3) / 1e12, 1),
                            "what": "fwd GEMM with the bias added in the epilogue"}
    # hybrid backward: tensorwise E5M2 of dY (both blobs), W and X (column blobs), FP8 dgrad and wgrad
    f8 = lambda r, l: torch.empty((mx.mx_fp8_blob_bytes(r, l, T),), dtype=torch.uint8, device=dev)
    gr8, gc8, wc8, xc8 = f8(tokens, dout), f8(dout, tokens), f8(din, dout), f8(din, tokens)
    info = torch.empty((3, 4), dtype=torch.float32, device=dev)
    ms_q = timed(lambda: mx.mx_quantize_fp8_tw(dY, tokens, dout, dout, T, gr8, gc8, info[0], stream))
    out["fp8_quant_dY_tw"] = {"ms": round(ms_q, 5),
                              "GB/s": round((2.0 * tokens * dout + 2.0 * tokens * dout) / (ms_q * 1e-3) / 1e9, 1),
                              "what": "dY tensorwise E5M2, row and column blobs (amax + quantize launches)"}
    mx.mx_quantize_fp8_tw(X, tokens, din, din, T, None, xc8, info[1], stream)
    mx.mx_quantize_fp8_tw(W, dout, din, din, T, None, wc8, info[2], stream)
    dXf = torch.empty((tokens, din), dtype=torch.int16, device=dev)
    dWf = torch.empty((dout, din), dtype=torch.int16, device=dev)
    fl = 2.0 * tokens * din * dout
    ms = timed(lambda: mx.mx_gemm_f8_tw(0, 1, tokens, din, dout, gr8, info[0, 1:], wc8, info[2, 1:], T, mx.MX_BF16,
                                        dXf, din, stream))
    out["fp8_gemm_dgrad"] = {"ms": round(ms, 5), "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 1),
                             "frac_fp8_peak": round(fl / (ms * 1e-3) / 1e12 / 5000.0, 4),
                             "what": "hybrid backward dgrad dY . W, tensorwise E5M2 (dense FP8 peak 5.0 PF/s)"}
    ms = timed(lambda: mx.mx_gemm_f8_tw(0, 1, dout, din, tokens, gc8, info[0, 1:], xc8, info[1, 1:], T, mx.MX_BF16,
                                        dWf, din, stream))
    out["fp8_gemm_wgrad"] = {"ms": round(ms, 5), "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 1),
                             "frac_fp8_peak": round(fl / (ms * 1e-3) / 1e12 / 5000.0, 4),
                             "what": "hybrid backward wgrad dY^T . X, tensorwise E5M2"}
    c8 = mfma_rate(mx, torch, dev, stream, 1, 1, gr8)
    out["fp8_mfma_ceiling"] = {"TFLOP/s": c8, "gemm_dgrad_frac": round(out["fp8_gemm_dgrad"]["TFLOP/s"] / c8, 4),
                               "gemm_wgrad_frac": round(out["fp8_gemm_wgrad"]["TFLOP/s"] / c8, 4),
                               "what": "MFMA-only loop, E5M2 x E5M2, on the dY FP8 blob's codes"}
    # quantizer prologue: dual quantize of bf16(dY * g) with the product formed in the staging read,
    # against the unfused pair (torch's bf16 multiply writing the product, then the quantizer)
    gfac = torch.empty_like(dY)
    gfac.copy_((torch.rand(dY.shape, device=dev) + 0.5).to(torch.bfloat16).view(torch.int16))
    prod = torch.empty_like(dY)
    ms_f = timed(lambda: mx.mx_quantize_dual_mul(dY, gfac, tokens, dout, dout, dout, sr, sr, T, gr, grs, gc, gcs,
                                                 stream))

    def unfused():
        torch.mul(dY.view(torch.bfloat16), gfac.view(torch.bfloat16), out=prod.view(torch.bfloat16))
        mx.mx_quantize_dual(prod, tokens, dout, dout, sr, sr, T, gr, grs, gc, gcs, stream)
    ms_u = timed(unfused)
    out["quant_dY_mul_prologue"] = {"ms": round(ms_f, 5), "unfused_ms": round(ms_u, 5),
                                    "GB/s": round((qb["quant_dY"] + 2.0 * tokens * dout) / (ms_f * 1e-3) / 1e9, 1),
                                    "what": "dY dual SR of bf16(dY * g), product in the staging read, vs torch "
                                            "multiply + quantize"}
    # MXFP6: X and W in E2M3 (both blobs), dY in E3M2 with stochastic rounding; the step's three GEMMs
    E2M3, E3M2 = mx.MX_FP6_E2M3, mx.MX_FP6_E3M2

    def f6(r, l):
        d, s_ = mx.mx_fp6_blob_bytes(r, l, T)
        return (torch.empty((d,), dtype=torch.uint8, device=dev), torch.empty((s_,), dtype=torch.uint8, device=dev))
    x6r, x6c, w6r, w6c, g6r, g6c = f6(tokens, din), f6(din, tokens), f6(dout, din), f6(din, dout), \
        f6(tokens, dout), f6(dout, tokens)
    x_bytes = 2.0 * tokens * din + sum(t.numel() for t in x6r + x6c)
    ms = timed(lambda: mx.mx_quantize_fp6(X, tokens, din, din, E2M3, plain, E2M3, plain, T, *x6r, *x6c, stream))
    out["fp6_quant_X"] = {"ms": round(ms, 5), "GB/s": round(x_bytes / (ms * 1e-3) / 1e9, 1),
                          "what": "X dual MXFP6 E2M3 (row and column blobs)"}
    g_bytes = 2.0 * tokens * dout + sum(t.numel() for t in g6r + g6c)
    ms = timed(lambda: mx.mx_quantize_fp6(dY, tokens, dout, dout, E3M2, sr, E3M2, sr, T, *g6r, *g6c, stream))
    out["fp6_quant_dY_sr"] = {"ms": round(ms, 5), "GB/s": round(g_bytes / (ms * 1e-3) / 1e9, 1),
                              "what": "dY dual MXFP6 E3M2, stochastic rounding"}
    mx.mx_quantize_fp6(W, dout, din, din, E2M3, mx.quant_opts(use_2d_block=True), E2M3,
                       mx.quant_opts(use_2d_block=True), T, *w6r, *w6c, stream)
    Y6 = torch.empty((tokens, dout), dtype=torch.int16, device=dev)
    for name, args6, what in [
            ("fp6_gemm_fwd", (tokens, dout, din, E2M3, *x6r, E2M3, *w6r, Y6, dout), "fwd X . W^T, E2M3 x E2M3"),
            ("fp6_gemm_dgrad", (tokens, din, dout, E3M2, *g6r, E2M3, *w6c, dXf, din), "dgrad dY . W, E3M2 x E2M3"),
            ("fp6_gemm_wgrad", (dout, din, tokens, E3M2, *g6c, E2M3, *x6c, dWf, din), "wgrad dY^T . X, E3M2 x E2M3")]:
        M6, N6, K6, fa6, qa6, sa6, fb6, qb6, sb6, C6, ldc6 = args6
        ms = timed(lambda: mx.mx_gemm_fp6(0, 1, M6, N6, K6, fa6, qa6, sa6, fb6, qb6, sb6, T, mx.MX_BF16, C6, ldc6,
                                          stream))
        out[name] = {"ms": round(ms, 5), "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 1),
                     "frac_fp6_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_FP4_TFLOPS, 4), "what": what}
    c22 = mfma_rate(mx, torch, dev, stream, E2M3, E2M3, x6r[0])
    c32 = mfma_rate(mx, torch, dev, stream, E3M2, E2M3, g6r[0])
    out["fp6_mfma_ceiling"] = {"E2M3xE2M3_TFLOP/s": c22, "E3M2xE2M3_TFLOP/s": c32,
                               "gemm_fwd_frac": round(out["fp6_gemm_fwd"]["TFLOP/s"] / c22, 4),
                               "gemm_dgrad_frac": round(out["fp6_gemm_dgrad"]["TFLOP/s"] / c32, 4),
                               "gemm_wgrad_frac": round(out["fp6_gemm_wgrad"]["TFLOP/s"] / c32, 4),
                               "what": "MFMA-only loop on the X (E2M3) and dY (E3M2) FP6 blobs' codes"}
    d_bytes, s_bytes = mx.mx_blob_bytes(tokens, din, mx.MX_LAYOUT_CANONICAL)
    cq = torch.empty((d_bytes,), dtype=torch.uint8, device=dev)
    cs = torch.empty((s_bytes,), dtype=torch.uint8, device=dev)
    ms = timed(lambda: mx.mx_layout_convert(0, tokens, din, Xr, Xrs, cq, cs, stream))
    out["layout_convert_to_canonical"] = {"ms": round(ms, 5),
                                          "GB/s": round(2.0 * (d_bytes + s_bytes) / (ms * 1e-3) / 1e9, 1),
                                          "what": "X row-wise blob %dx%d, tiled -> canonical" % (tokens, din)}
    return out


def mfma_rate(mx, torch, dev, stream, fmt_a, fmt_b, ops, iters=40000, reps=5):
    """TFLOP/s of the MFMA-only loop (mx_measure_mfma) on the first 16 KB of
    `ops` (uint8 device tensor of element codes), one workgroup of 8 waves per CU."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty((cus * 512,), dtype=torch.float32, device=dev)
    ops = ops[:16384]
    mx.mx_measure_mfma(fmt_a, fmt_b, ops, cus, iters, out, stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        mx.mx_measure_mfma(fmt_a, fmt_b, ops, cus, iters, out, stream)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    return round(cus * 32.0 * iters * 131072 / (ms * 1e-3) / 1e12, 1)


def time_other_workloads(mx, torch, dev, stream, synth, reps=20):
    """The other seeded workloads of the suite: the 4600x3072 dual quantize (M
    not a multiple of 128, outliers, zero blocks) and the QKV forward (4608 x
    9216 x 3072, its two row-wise quantizes and the GEMM), each over rotating
    buffer sets larger than twice the Infinity Cache, median and minimum of 30
    batches of 20 launches; the MLP fc1 step (9216 tokens, 3072 -> 12288: three
    dual quantizes, fwd, dgrad, wgrad; tensors of 56-226 MB), timed like the
    extras (event pair around `reps` back-to-back launches, inputs resident)."""
    T = mx.MX_LAYOUT_TILED
    plain = mx.quant_opts()

    def timed(fn):
        for _ in range(2):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(reps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    def dev_bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev)

    def dual_bytes(M, N):
        d1, s1 = mx.mx_blob_bytes(M, N, T)
        d2, s2 = mx.mx_blob_bytes(N, M, T)
        return 2.0 * M * N + d1 + s1 + d2 + s2

    def quant_entry(ms, nbytes, what):
        gbs = nbytes / (ms * 1e-3) / 1e9
        return {"ms": round(ms, 5), "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "what": what}

    def gemm_entry(ms, M, N, K, what):
        tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        return {"ms": round(ms, 5), "TFLOP/s": round(tf, 1), "frac_fp4_peak": round(tf / PEAK_FP4_TFLOPS, 4),
                "what": what}

    out = {}
    # The two small workloads move 43 MB and ~110 MB per call, less than the
    # 256 MB Infinity Cache, so they cycle through enough buffer sets (inputs
    # and outputs) to exceed twice its size and report the median and the
    # minimum over batches of launches.
    MALL = 256 << 20

    def batch_stats(fn_i, nsets, batches, per):
        for i in range(2 * nsets):
            fn_i(i % nsets)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        t = []
        for b in range(batches):
            ev[0].record(stream)
            for j in range(per):
                fn_i((b * per + j) % nsets)
            ev[1].record(stream)
            ev[1].synchronize()
            t.append(ev[0].elapsed_time(ev[1]) / per)
        return float(np.median(t)), float(np.min(t))

    def with_stats(entry, med, mn, nsets):
        entry["min_ms"] = round(mn, 5)
        entry["buffer_sets"] = nsets
        entry["timing"] = "median of 30 batches of 20 launches, rotating buffer sets"
        return entry

    # dual quantize only, 4600 x 3072
    x0 = dev_bf16(synth.dual()["X"])
    M, N = x0.shape
    set_bytes = dual_bytes(M, N)
    nsets = max(2, -(-2 * MALL // int(set_bytes)) + 1)
    xs = [x0] + [x0.clone() for _ in range(nsets - 1)]
    outs = [mx.empty_blob(M, N, T, dev) + mx.empty_blob(N, M, T, dev) for _ in range(nsets)]
    med, mn = batch_stats(lambda i: mx.mx_quantize_dual(xs[i], M, N, N, plain, plain, T, *outs[i], stream),
                          nsets, 30, 20)
    out["dual_4600x3072"] = with_stats(quant_entry(med, set_bytes, "dual quantize 4600x3072 (outliers, zero blocks)"),
                                       med, mn, nsets)
    del x0, xs, outs
    # QKV forward: both row-wise quantizes and the GEMM, each over rotating sets
    d = synth.qkv()
    a0, w0 = dev_bf16(d["A"]), dev_bf16(d["W"])
    (M, K), N = a0.shape, w0.shape[0]
    rb = lambda r, k: 2.0 * r * k + sum(mx.mx_blob_bytes(r, k, T))
    na = max(2, -(-2 * MALL // int(rb(M, K))) + 1)
    nw = max(2, -(-2 * MALL // int(rb(N, K))) + 1)
    a_s = [a0] + [a0.clone() for _ in range(na - 1)]
    w_s = [w0] + [w0.clone() for _ in range(nw - 1)]
    ab = [mx.empty_blob(M, K, T, dev) for _ in range(na)]
    wb = [mx.empty_blob(N, K, T, dev) for _ in range(nw)]
    med, mn = batch_stats(lambda i: mx.mx_quantize_rowwise(a_s[i], M, K, K, plain, T, *ab[i], stream), na, 30, 20)
    out["qkv_quant_A_rowwise"] = with_stats(quant_entry(med, rb(M, K), "A 4608x3072 row-wise"), med, mn, na)
    med, mn = batch_stats(lambda i: mx.mx_quantize_rowwise(w_s[i], N, K, K, plain, T, *wb[i], stream), nw, 30, 20)
    out["qkv_quant_W_rowwise"] = with_stats(quant_entry(med, rb(N, K), "W 9216x3072 row-wise"), med, mn, nw)
    # GEMM sets: operand blobs + C; the blobs are copies of the quantized ones
    g_set = sum(t.numel() for t in ab[0] + wb[0]) + 2.0 * M * N
    ng = max(2, -(-2 * MALL // int(g_set)) + 1)
    ga = [ab[0]] + [tuple(t.clone() for t in ab[0]) for _ in range(ng - 1)]
    gw = [wb[0]] + [tuple(t.clone() for t in wb[0]) for _ in range(ng - 1)]
    Cs = [torch.empty((M, N), dtype=torch.int16, device=dev) for _ in range(ng)]
    med, mn = batch_stats(lambda i: mx.mx_gemm_a4w4(0, 1, M, N, K, ga[i][0], ga[i][1], gw[i][0], gw[i][1], T,
                                                    mx.MX_BF16, Cs[i], N, stream), ng, 30, 20)
    out["qkv_gemm_fwd"] = with_stats(gemm_entry(med, M, N, K, "QKV forward 4608 x 9216 x 3072"), med, mn, ng)
    del a0, w0, a_s, w_s, ab, wb, ga, gw, Cs, d
    # MLP fc1 training step
    d = synth.fc1()
    X, W, G = dev_bf16(d["X"]), dev_bf16(d["W"]), dev_bf16(d["dY"])
    del d
    (Tk, din), dout = X.shape, W.shape[0]
    blobs = {}
    tot = 0.0
    for name, t in (("X", X), ("W", W), ("dY", G)):
        M, N = t.shape
        b = mx.empty_blob(M, N, T, dev) + mx.empty_blob(N, M, T, dev)
        ms = timed(lambda: mx.mx_quantize_dual(t, M, N, N, plain, plain, T, *b, stream))
        out["fc1_quant_" + name] = quant_entry(ms, dual_bytes(M, N), "%s %dx%d dual" % (name, M, N))
        blobs[name] = b
        tot += ms
    Y = torch.empty((Tk, dout), dtype=torch.int16, device=dev)
    dX = torch.empty((Tk, din), dtype=torch.int16, device=dev)
    dW = torch.empty((dout, din), dtype=torch.int16, device=dev)
    xb, wb, gb = blobs["X"], blobs["W"], blobs["dY"]
    for name, (M, N, K, A_, As_, B_, Bs_, C_, ldc) in (
            ("fwd", (Tk, dout, din, xb[0], xb[1], wb[0], wb[1], Y, dout)),
            ("dgrad", (Tk, din, dout, gb[0], gb[1], wb[2], wb[3], dX, din)),
            ("wgrad", (dout, din, Tk, gb[2], gb[3], xb[2], xb[3], dW, din))):
        ms = timed(lambda: mx.mx_gemm_a4w4(0, 1, M, N, K, A_, As_, B_, Bs_, T, mx.MX_BF16, C_, ldc, stream))
        out["fc1_gemm_" + name] = gemm_entry(ms, M, N, K, "fc1 %s %d x %d x %d" % (name, M, N, K))
        tot += ms
    out["fc1_step_sum_ms"] = round(tot, 5)
    return out


def load_traffic():
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary
    (profiles/hbm_traffic_fc2_step.json, calibrated against a plain 1 GiB copy), used only
    while the kernel sources are the ones the counters were taken on."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic_fc2_step.json")
    try:
        rec = json.load(open(path))
        for name, digest in rec["source_sha256"].items():
            src = os.path.join(ROOT, "mxfp4_precision_amd", "csrc", name)
            if hashlib.sha256(open(src, "rb").read()).hexdigest() != digest:
                return None
        L = rec["launches"]
        gemm = sum(L[n]["hbm_bytes"] for n in ("gemm_fwd", "gemm_dgrad", "gemm_wgrad")) / 3.0
        out = {"gemm": int(gemm), "quant_X": int(L["quant_X"]["hbm_bytes"])}
        valu = rec.get("valu", {}).get("quant_dY", {})
        if "SQ_INSTS_VALU_per_launch" in valu:
            out["quant_dY_valu_insts"] = float(valu["SQ_INSTS_VALU_per_launch"])
        return out
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(data, ct, din, dout):
    """The CPU oracle, as it stands, on the first `ct` tokens of the same step:
    dual-quantize X[:ct], W (2D) and dY[:ct] (SR), then the three GEMMs of that
    slice (fwd and dgrad rows of the slice, wgrad over the slice's tokens)."""
    import oracle
    oracle.build()
    x = np.ascontiguousarray(data["X"][:ct])
    w = data["W"]
    g = np.ascontiguousarray(data["dY"][:ct])
    t0 = time.perf_counter()
    xr = oracle.quantize(x, 0)
    xc = oracle.quantize(x, 1)
    wr = oracle.quantize(w, 0, use_2d=True, tensor_id=1)
    wc = oracle.quantize(w, 1, use_2d=True, tensor_id=1)
    gr = oracle.quantize(g, 0, use_sr=True, seed=7, tensor_id=2)
    gc = oracle.quantize(g, 1, use_sr=True, seed=7, tensor_id=2)
    oracle.gemm_rows(xr[0], xr[1], wr[0], wr[1], ct, dout, din, 0, ct)
    oracle.gemm_rows(gr[0], gr[1], wc[0], wc[1], ct, din, dout, 0, ct)
    oracle.gemm_rows(gc[0], gc[1], xc[0], xc[1], dout, din, ct, 0, dout)
    dt = time.perf_counter() - t0
    fl = 2.0 * ct * din * dout * 3
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count()
    out = {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "seconds": round(dt, 2),
           "sample": "fc2 step on a %d-token slice (X %dx%d, W %dx%d, dY %dx%d): oracle dual "
                     "quantize of all three + the slice's fwd, dgrad and wgrad GEMMs in fp64"
                     % (ct, ct, din, dout, din, ct, dout)}
    out.update(host_description())
    out["components"] = cpu_components(data, ct, 16)
    return out


def host_description():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return {"cpu_model": model, "cpus_available": avail}


def oracle_components(x, w, rows):
    """Oracle rates on two pieces of the step, comparable across thread counts:
    the dual quantize of x (bytes read + both blobs written) and the forward
    GEMM over its first `rows` token rows (against all of W)."""
    import oracle
    M, N = x.shape
    t0 = time.perf_counter()
    xr = oracle.quantize(x, 0)
    xc = oracle.quantize(x, 1)
    dq = time.perf_counter() - t0
    qbytes = 2.0 * M * N + sum(a.nbytes for a in xr + xc)
    wr = oracle.quantize(w, 0, use_2d=True, tensor_id=1)
    t0 = time.perf_counter()
    oracle.gemm_rows(xr[0], xr[1], wr[0], wr[1], M, w.shape[0], N, 0, rows)
    dg = time.perf_counter() - t0
    return {"quantize_GB/s": round(qbytes / dq / 1e9, 4),
            "gemm_GFLOP/s": round(2.0 * rows * w.shape[0] * N / dg / 1e9, 4)}


# oracle_components in a child process with one OpenMP thread (an OpenMP
# runtime fixes its thread count when it starts)
_ONE_CORE = r"""
import json, sys
import numpy as np
sys.path.insert(0, sys.argv[1])
import bench
d = np.load(sys.argv[2])
print(json.dumps(bench.oracle_components(d["x"], d["w"], int(sys.argv[3]))))
"""


def cpu_components(data, ct, rows):
    """oracle_components on all cores (this process) and on one core (a child)."""
    import subprocess
    import tempfile
    x = np.ascontiguousarray(data["X"][:ct])
    w = data["W"]
    out = {"all_cores": oracle_components(x, w, rows)}
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "slice.npz")
        np.savez(path, x=x, w=w)
        env = dict(os.environ, OMP_NUM_THREADS="1")
        r = subprocess.run([sys.executable, "-c", _ONE_CORE, ROOT, path, str(rows)], env=env, capture_output=True,
                           text=True, timeout=600)
    if r.returncode == 0:
        out["one_core"] = json.loads(r.stdout.strip().splitlines()[-1])
    else:
        out["one_core_error"] = r.stderr.strip().splitlines()[-1] if r.stderr.strip() else "exit %d" % r.returncode
    out["what"] = ("oracle dual quantize of X[:%d] (GB/s of bytes read and written) and its forward GEMM over "
                   "%d token rows (GFLOP/s), on all cores and with OMP_NUM_THREADS=1" % (ct, rows))
    return out


if __name__ == "__main__":
    main()

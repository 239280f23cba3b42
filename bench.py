#!/usr/bin/env python3
"""Benchmark: one W4A4G4 training step of the spectral-domain FP4 linear layer
at LLaMA-3-8B FFN shapes (up 4096 -> 14336 and down 14336 -> 4096, 8192
tokens), on one MI355X.

A step is the whole hot path over one batch of synthetic, HBM-resident input:
  * split + MXFP4-quantize six tensors (W_up, W_down, X_up, X_down, dY_up,
    dY_down; k = 64, l = 80, Gaussian sketch; residual in both orientations);
  * six GEMMs with their low-rank corrections: Y = X W^T, dX = dY W,
    dW = dY^T X for both layers (6 x 962.07 GFLOP).
value = sum(2 M N K) / step time. Splits run on three streams and the GEMMs on
a fourth; a GEMM starts when the splits it reads are done.

Prints one JSON line. Usage: python bench.py [--steps K] [--warmup W]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP4_PEAK_TFLOPS = 10100.0  # MI355X dense MXFP4 MFMA
HBM_PEAK_GBS = 8000.0
CFG = 4


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_flops(cfg_shapes, gemms):
    total = 0
    for out, a, ao, b, bo in gemms:
        ra = cfg_shapes[a][1] if ao == "t" else cfg_shapes[a][0]
        T = cfg_shapes[a][0] if ao == "t" else cfg_shapes[a][1]
        rb = cfg_shapes[b][1] if bo == "t" else cfg_shapes[b][0]
        total += 2 * ra * rb * T
    return total


def cpu_baseline(tensors, gemm_total_flops):
    """The fp64 oracle on a bounded sample of the same workload: the split of
    X_up (8192 x 4096) and the forward GEMM Y_up on 256 sampled rows; the
    step time is extrapolated by element count (splits) and by rows (GEMMs)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import linear as OL
    from oracle import split as OS

    t = tensors["X_up"]
    w = tensors["W_up"]
    A = t.values.astype(np.float64)
    t0 = time.perf_counter()
    r = OS.spectral_split(A, t.l, t.k, omega=t.omega_values().astype(np.float64))
    rec_x = OS.quantize_record("mxfp4", r["R"], r["U"], r["S"], r["V"], orientations=("n", "t"))
    t_split = time.perf_counter() - t0
    Aw = w.values.astype(np.float64)
    rw = OS.spectral_split(Aw, w.l, w.k, omega=w.omega_values().astype(np.float64))
    rec_w = OS.quantize_record("mxfp4", rw["R"], rw["U"], rw["S"], rw["V"], orientations=("n",))
    rows = np.arange(0, 8192, 32)
    t0 = time.perf_counter()
    OL.linear_fwd(rec_x, rec_w, rows=rows)
    t_gemm = time.perf_counter() - t0
    elems = {n: x.shape[0] * x.shape[1] for n, x in tensors.items()}
    split_s = t_split * sum(elems.values()) / elems["X_up"]
    gemm_s = t_gemm * (gemm_total_flops / (2 * len(rows) * 4096 * 14336))
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": round(gemm_total_flops / (split_s + gemm_s) / 1e12, 6), "unit": "TFLOP/s",
            "cores": threads, "kind": "oracle",
            "sample": "fp64 oracle: split+quantize of X_up (8192x4096, both orientations) in %.1f s and Y_up "
                      "on 256 of 8192 rows in %.1f s; step time extrapolated by element count (6 splits) and "
                      "by rows (6 GEMMs of 962 GFLOP)" % (t_split, t_gemm)}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (see DESIGN.md for how it "
              "would shard); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp4_spectral_split_amd as M
    import synth

    dev = torch.device("cuda:0")
    names = synth.TENSOR_NAMES[CFG]
    gemms = synth.GEMMS[CFG]
    t0 = time.perf_counter()
    tensors = {}
    for n in names:
        tensors[n] = synth.make_tensor(CFG, n)
        log("generated %s %s (%.1fs)" % (n, tensors[n].shape, time.perf_counter() - t0))
    shapes = {n: t.shape for n, t in tensors.items()}
    total_flops = gemm_flops(shapes, gemms)

    A = {n: torch.from_numpy(t.bits.view(np.int16)).view(torch.bfloat16).to(dev) for n, t in tensors.items()}
    Om = {n: torch.from_numpy(t.omega.view(np.int16)).view(torch.bfloat16).to(dev).contiguous()
          for n, t in tensors.items()}
    recs = {n: M.empty_split(t.shape[0], t.shape[1], t.k, "mxfp4", ("n", "t"), dev) for n, t in tensors.items()}
    outs, gobj = {}, {}
    for out, a, ao, b, bo in gemms:
        g = M.GemmNT(recs[a], ao == "t", recs[b], bo == "t")
        gobj[out] = g
        outs[out] = torch.empty(g.rows, g.cols, dtype=torch.float32, device=dev)

    split_streams = [torch.cuda.Stream(dev) for _ in range(3)]
    gstream = torch.cuda.Stream(dev)
    lanes = [["X_up", "X_down"], ["W_up", "W_down"], ["dY_up", "dY_down"]]
    done = {n: torch.cuda.Event() for n in names}
    step_end = torch.cuda.Event()
    t = tensors
    ev = lambda: torch.cuda.Event(enable_timing=True)
    split_ev = [{n: (ev(), ev()) for n in names} for _ in range(args.steps)]
    main_ev = [{o: (ev(), ev()) for o in outs} for _ in range(args.steps)]

    def step(i):
        rec = i is not None
        for s, lane in zip(split_streams, lanes):
            s.wait_event(step_end)
            with torch.cuda.stream(s):
                for n in lane:
                    if rec:
                        split_ev[i][n][0].record(s)
                    M.metis_split(A[n], t[n].l, t[n].k, "mxfp4", omega=Om[n], out=recs[n])
                    if rec:
                        split_ev[i][n][1].record(s)
                    done[n].record(s)
        with torch.cuda.stream(gstream):
            for out, a, ao, b, bo in gemms:
                gstream.wait_event(done[a])
                gstream.wait_event(done[b])
                gobj[out].prepare()
                if rec:
                    main_ev[i][out][0].record(gstream)
                gobj[out].main(outs[out])
                if rec:
                    main_ev[i][out][1].record(gstream)
            step_end.record(gstream)

    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    log("warmup done (%d steps)" % args.warmup)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    value = total_flops / (ms_per_step / 1e3) / 1e12
    log("step %.3f ms -> %.1f TFLOP/s" % (ms_per_step, value))
    split_ms = {n: sum(e[n][0].elapsed_time(e[n][1]) for e in split_ev) for n in names}
    main_ms = {o: sum(e[o][0].elapsed_time(e[o][1]) for e in main_ev) for o in outs}

    per_gemm = total_flops / len(gemms)
    main_avg_ms = sum(main_ms.values()) / (len(gemms) * args.steps)
    achieved = per_gemm / (main_avg_ms / 1e3) / 1e12
    line = {
        "metric": "TFLOP/s of spectral-FP4 linear fwd+bwd at LLaMA-3-8B shapes; split ms",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4", "data": "synthetic",
        "config": {"workload": "llama3-8b-ffn-up+down-w4a4g4", "tokens": 8192, "hidden": 4096, "ffn": 14336,
                   "k": 64, "l": 80, "fmt": "mxfp4", "sketch": "gaussian", "gemm_gflop_per_step":
                   round(total_flops / 1e9, 2)},
        "split_ms": {n: round(v / args.steps, 4) for n, v in split_ms.items()},
        "gemm_main_ms": {o: round(v / args.steps, 4) for o, v in main_ms.items()},
        "roofline": {"bound": "mfma", "kernel": "gemm_kernel (main MXFP4 GEMM + low-rank correction)",
                     "achieved": round(achieved, 2), "peak": FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / FP4_PEAK_TFLOPS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline(tensors, total_flops)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

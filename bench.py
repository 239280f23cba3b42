#!/usr/bin/env python3
"""Benchmark: one W4A4G4 training step of the spectral-domain FP4 linear layer
at LLaMA-3-8B FFN shapes (up 4096 -> 14336 and down 14336 -> 4096, 8192
tokens), on one MI355X.

A step is the whole hot path over one batch of synthetic, HBM-resident input:
  * split + MXFP4-quantize six tensors (W_up, W_down, X_up, X_down, dY_up,
    dY_down; k = 64, l = 80, Gaussian sketch; residual in both orientations);
  * six GEMMs with their low-rank corrections: Y = X W^T, dX = dY W,
    dW = dY^T X for both layers (6 x 962.07 GFLOP).
value = sum(2 M N K) / step time. Each split runs on a stream (lane) of its
own, so the six splits' latency-bound l x l stages (Cholesky, Jacobi) run
side by side on six CUs; each GEMM follows one of its operands' splits in
that lane and waits for the other's, so the up-projection GEMMs overlap the
down-projection splits. Work is enqueued in dependency order, and a step
starts when every lane has finished the previous one. Seven streams (six
lanes and the default stream) each get a hardware queue of their own: the
HIP runtime is asked for 8 queues (GPU_MAX_HW_QUEUES) before it starts, as
two streams that share a queue run one after the other.

Prints one JSON line. Usage: python bench.py [--steps K] [--warmup W]

roofline.traffic is the main GEMM kernel's HBM bytes per launch, read from the
committed counter summary in profiles/ (FETCH_SIZE and WRITE_SIZE, scaled by
what the same counters read for a plain copy of known size); it is null when
that summary was taken on a different version of the GEMM source. The copy
that calibrates the counters runs with --calibrate-copy MIB, ahead of the
steps, in the same profiled process.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP4_PEAK_TFLOPS = 10100.0  # MI355X dense MXFP4 MFMA
HBM_PEAK_GBS = 8000.0
CFG = 4
HW_QUEUES = 8
GEMM_SOURCE = os.path.join(ROOT, "fp4_spectral_split_amd", "csrc", "linear.hip")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_mx_kernel_llama3-8b-ffn_traffic.md")


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


def gemm_traffic():
    """HBM bytes per main-GEMM launch from the committed counter summary, or
    None when it is missing or was taken on another version of linear.hip."""
    try:
        fields = dict(line.split(":", 1) for line in open(TRAFFIC_SUMMARY) if line.startswith("- ") and ":" in line)
    except OSError:
        return None
    fields = {k[2:].strip(): v.strip().strip("`") for k, v in fields.items()}
    src = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    if fields.get("linear.hip sha256") != src or "hbm bytes per launch" not in fields:
        return None
    return int(fields["hbm bytes per launch"])


def calibrate_copy(torch, dev, mib):
    """A plain elementwise copy of mib MiB (fp32 in, fp32 out), five times,
    so that the profiled process holds dispatches of known traffic."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log("calibration copy: 5 x %d MiB read + %d MiB written" % (mib, mib))


def mean_split_leg(torch, M, A, tensors, reps=10):
    """The mean-residual split (next to the spectral one) timed alone on the
    activation and gradient inputs, after the timed steps: milliseconds per
    call and HBM rate against its algorithmic bytes (A read twice, the
    residual codes and scales of both orientations written)."""
    out = {}
    for n in ("X_up", "dY_up"):
        m_, n_ = tensors[n].shape
        rec = M.empty_split(m_, n_, 1, "mxfp4", ("n", "t"), A[n].device)
        M.metis_mean_split(A[n], "mxfp4", out=rec)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            M.metis_mean_split(A[n], "mxfp4", out=rec)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        elems = m_ * n_
        nbytes = 2 * 2 * elems + 2 * (elems // 2 + elems // 32)
        out[n] = {"ms": round(ms, 4), "GB/s": round(nbytes / (ms / 1e3) / 1e9, 1), "algorithmic_bytes": nbytes}
    return out


def power_split_leg(torch, M, A, Om, recs, tensors, reps=5):
    """The spectral split with q = 1 power iteration (two more passes over A)
    timed alone on X_up, after the timed steps, next to q = 0."""
    t = tensors["X_up"]
    out = {}
    for q in (0, 1):
        M.metis_split(A["X_up"], t.l, t.k, "mxfp4", omega=Om["X_up"], out=recs["X_up"], q=q)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            M.metis_split(A["X_up"], t.l, t.k, "mxfp4", omega=Om["X_up"], out=recs["X_up"], q=q)
        e1.record()
        torch.cuda.synchronize()
        out["q%d_ms" % q] = round(e0.elapsed_time(e1) / reps, 4)
    return {"tensor": "X_up 8192x4096 bf16, k 64, l 80", **out}


def profile_splits(torch, M, A, Om, recs, tensors, reps):
    """For kernel profiles of the split and quantize kernels alone (their HBM
    rate is read from the profiler, not printed): each of the six spectral
    splits reps times back to back on one stream, then the standalone MXFP4
    quantizer on X_up in both orientations reps times. Replaces the steps."""
    for n, t in tensors.items():
        for _ in range(reps):
            M.metis_split(A[n], t.l, t.k, "mxfp4", omega=Om[n], out=recs[n])
        torch.cuda.synchronize()
        log("profiled split %s x %d" % (n, reps))
    x = A["X_up"]
    for _ in range(reps):
        M.fp4_block_quant(x, "mxfp4")
        M.fp4_block_quant(x, "mxfp4", transpose=True)
    torch.cuda.synchronize()
    log("profiled fp4_block_quant X_up (both orientations) x %d" % reps)


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
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="run a plain copy of MIB MiB ahead of the steps (counter calibration)")
    ap.add_argument("--two-call-splits", action="store_true",
                    help="enqueue the splits as metis_split_begin / _finish, the down-projection first phases after "
                         "the up-projection ones (measured slower than one call per split)")
    ap.add_argument("--profile-splits", type=int, default=0, metavar="REPS",
                    help="instead of the steps, run each split and the quantizer REPS times alone (for profiles)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (see DESIGN.md for how it "
              "would shard); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    # one hardware queue per lane (read by the HIP runtime when it starts)
    os.environ["GPU_MAX_HW_QUEUES"] = str(max(HW_QUEUES, int(os.environ.get("GPU_MAX_HW_QUEUES", "4"))))
    import numpy as np
    import torch

    import fp4_spectral_split_amd as M
    import synth

    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        calibrate_copy(torch, dev, args.calibrate_copy)
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
    if args.profile_splits:
        profile_splits(torch, M, A, Om, recs, tensors, args.profile_splits)
        return
    outs, gobj = {}, {}
    for out, a, ao, b, bo in gemms:
        g = M.GemmNT(recs[a], ao == "t", recs[b], bo == "t")
        gobj[out] = g
        outs[out] = torch.empty(g.rows, g.cols, dtype=torch.float32, device=dev)

    lanes = [torch.cuda.Stream(dev) for _ in range(6)]
    # (lane, kind, name) in an order where every GEMM follows the splits it reads
    order = [(0, "split", "W_up"), (1, "split", "X_up"), (2, "split", "dY_up"),
             (1, "gemm", "Y_up"), (2, "gemm", "dX_up"), (0, "gemm", "dW_up"),
             (3, "split", "W_down"), (4, "split", "X_down"), (5, "split", "dY_down"),
             (4, "gemm", "Y_down"), (5, "gemm", "dX_down"), (3, "gemm", "dW_down")]
    gemm_of = {g[0]: g for g in gemms}
    assert sorted(n for _, k, n in order if k == "split") == sorted(names)
    assert sorted(n for _, k, n in order if k == "gemm") == sorted(gemm_of)
    done = {n: torch.cuda.Event() for n in names}
    lane_end = [torch.cuda.Event() for _ in lanes]
    t = tensors
    ev = lambda: torch.cuda.Event(enable_timing=True)
    split_ev = [{n: (ev(), ev()) for n in names} for _ in range(args.steps)]
    main_ev = [{o: (ev(), ev()) for o in outs} for _ in range(args.steps)]

    # two-call splits (opt-in): the full-GPU first phase of the down-projection
    # splits runs while the up-projection splits are in their one-workgroup
    # small SVD; the down-projection first phases wait for the up ones
    two = {n: M.SplitInTwo(A[n], t[n].l, t[n].k, "mxfp4", omega=Om[n], out=recs[n])
           for n in names} if args.two_call_splits else {}
    lane_of = {n: li for li, kind, n in order if kind == "split"}
    up = [n for n in names if n.endswith("_up")]
    begun = {n: torch.cuda.Event() for n in names}

    def step_two(i):
        rec = i is not None
        for s in lanes:
            for e in lane_end:
                s.wait_event(e)
        seq = [("begin", n) for n in up] + [("begin", n) for n in names if n not in up]
        seq += [("finish", n) for n in up] + [("gemm", g) for _, k, g in order if k == "gemm" and g.endswith("_up")]
        seq += [("finish", n) for n in names if n not in up]
        seq += [("gemm", g) for _, k, g in order if k == "gemm" and not g.endswith("_up")]
        for kind, n in seq:
            li = lane_of[n] if kind != "gemm" else next(l for l, k, g in order if k == "gemm" and g == n)
            s = lanes[li]
            with torch.cuda.stream(s):
                if kind == "begin":
                    if n not in up:
                        for u in up:
                            s.wait_event(begun[u])
                    if rec:
                        split_ev[i][n][0].record(s)
                    two[n].begin()
                    begun[n].record(s)
                elif kind == "finish":
                    two[n].finish()
                    if rec:
                        split_ev[i][n][1].record(s)
                    done[n].record(s)
                else:
                    _, a, ao, b, bo = gemm_of[n]
                    s.wait_event(done[a])
                    s.wait_event(done[b])
                    gobj[n].prepare()
                    if rec:
                        main_ev[i][n][0].record(s)
                    gobj[n].main(outs[n])
                    if rec:
                        main_ev[i][n][1].record(s)
        for s, e in zip(lanes, lane_end):
            e.record(s)

    def step(i):
        if args.two_call_splits:
            return step_two(i)
        rec = i is not None
        for s in lanes:  # the previous step's GEMMs are done with every record
            for e in lane_end:
                s.wait_event(e)
        enqueued = set()
        for li, kind, n in order:
            s = lanes[li]
            with torch.cuda.stream(s):
                if kind == "split":
                    if rec:
                        split_ev[i][n][0].record(s)
                    M.metis_split(A[n], t[n].l, t[n].k, "mxfp4", omega=Om[n], out=recs[n])
                    if rec:
                        split_ev[i][n][1].record(s)
                    done[n].record(s)
                    enqueued.add(n)
                else:
                    _, a, ao, b, bo = gemm_of[n]
                    assert a in enqueued and b in enqueued
                    s.wait_event(done[a])
                    s.wait_event(done[b])
                    gobj[n].prepare()
                    if rec:
                        main_ev[i][n][0].record(s)
                    gobj[n].main(outs[n])
                    if rec:
                        main_ev[i][n][1].record(s)
        for s, e in zip(lanes, lane_end):
            e.record(s)

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
        "roofline": {"bound": "mfma", "kernel": "gemm_mx_kernel (main MXFP4 GEMM + low-rank correction)",
                     "achieved": round(achieved, 2), "peak": FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / FP4_PEAK_TFLOPS, 4), "traffic": gemm_traffic()},
    }
    # the same kernel alone on an idle GPU (context for the in-step figure,
    # which shares the CUs with the other lanes' kernels)
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    e0.record()
    for _ in range(5):
        gobj["Y_up"].main(outs["Y_up"])
    e1.record()
    torch.cuda.synchronize()
    iso = per_gemm / (e0.elapsed_time(e1) / 5 / 1e3) / 1e12
    line["roofline"]["isolated_achieved"] = round(iso, 2)
    line["roofline"]["isolated_frac"] = round(iso / FP4_PEAK_TFLOPS, 4)
    line["mean_split"] = mean_split_leg(torch, M, A, tensors)
    line["power_split"] = power_split_leg(torch, M, A, Om, recs, tensors)
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline(tensors, total_flops)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark: one W4A4G4 training step of the spectral-domain FP4 linear layer
at LLaMA-3-8B FFN shapes (up 4096 -> 14336 and down 14336 -> 4096, 8192
tokens), on one MI355X, plus legs for the other workloads.

The headline step is the whole hot path over one batch of synthetic,
HBM-resident input:
  * split + MXFP4-quantize six tensors (W_up, W_down, X_up, X_down, dY_up,
    dY_down; k = 64, l = 80, Gaussian sketch; residual in both orientations);
  * six GEMMs with their low-rank corrections: Y = X W^T, dX = dY W,
    dW = dY^T X for both layers (6 x 962.07 GFLOP).
value = sum(2 M N K) / step time. Each split runs on a stream (lane) of its
own, so the six splits' latency-bound l x l stages run side by side on six
CUs; each GEMM follows one of its operands' splits in that lane and waits for
the other's, so the up-projection GEMMs overlap the down-projection splits.
Work is enqueued in dependency order, and a step starts when every lane has
finished the previous one. Seven streams (six lanes and the default stream)
each get a hardware queue of their own: the HIP runtime is asked for 8 queues
(GPU_MAX_HW_QUEUES) before it starts, as two streams that share a queue run
one after the other.

After the timed steps (each leg in its own timed region, HIP events on the
stream the kernels run on):
  roofline       the main MXFP4 GEMM kernel (gemm_mx_kernel), the six GEMMs of
                 the step each REPS times back to back on one stream:
                 algorithmic 2MNK per launch / its average launch duration,
                 against the dense MXFP4 peak; the in-step figure (the kernel
                 sharing the GPU with the other lanes) beside it;
  split_hbm      each of the six splits alone, the 256 MB Infinity Cache
                 flushed (a 1 GiB write) before every rep: ms and GB/s of
                 algorithmic bytes against 8 TB/s, and the standalone MXFP4
                 quantizer the same way;
  configs        the other workloads as steps of their own on one stream
                 (splits / quantization, then their GEMMs): the 1.1B-class layer
                 (fwd), the 8B attention projection (fwd + dX), and the NVFP4
                 + 512-column-sampling down projection (fwd + bwd);
  mean_split, power_split   the two extra split variants on the FFN tensors;
  optim          the dual-range regularizer on W_up and the adaptive spectral
                 learning rate on the step's dW_up;
  cpu_baseline   the fp64 oracle on a bounded sample (one full split and one
                 full GEMM of the step), extrapolated to the step.

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
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP4_PEAK_TFLOPS = 10100.0   # MI355X dense MXFP4 / NVFP4-class MFMA
F16_PEAK_TFLOPS = 2500.0    # MI355X dense fp16 MFMA (the NVFP4 GEMM runs on it)
HBM_PEAK_GBS = 8000.0
CFG = 4
HW_QUEUES = 8
FLUSH_BYTES = 1 << 30       # > the 256 MB Infinity Cache
GEMM_SOURCE = os.path.join(ROOT, "fp4_spectral_split_amd", "csrc", "linear.hip")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_mx_kernel_llama3-8b-ffn_traffic.md")
CONFIG_LABEL = {2: "1.1b-layer-fwd", 3: "llama3-8b-attn-proj-fwd+dx", 5: "llama3-8b-ffn-down-nvfp4-sampled512"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_dims(shapes, g):
    _, a, ao, b, bo = g
    ra = shapes[a][1] if ao == "t" else shapes[a][0]
    T = shapes[a][0] if ao == "t" else shapes[a][1]
    rb = shapes[b][1] if bo == "t" else shapes[b][0]
    return ra, rb, T


def gemm_flops(shapes, gemms):
    return sum(2 * ra * rb * T for ra, rb, T in (gemm_dims(shapes, g) for g in gemms))


def split_bytes(t, orientations):
    """Algorithmic HBM bytes of one split (or of the quantization of an
    unsplit tensor): A read three times (sketch, projection, residual; once
    for a plain quantization), codes and scales of each residual orientation
    written (bf16 input; NVFP4 codes + E4M3 scales per 16)."""
    m, n = t.shape
    e = m * n
    elem = 2 if t.dtype == "bf16" else 4
    B = 16 if t.fmt == "nvfp4" else 32
    out = len(orientations) * (e // 2 + e // B)
    reads = 3 if t.k else 1
    if t.k and t.sketch == "columns":  # the gather reads l columns, not all of A
        reads = 2
        return reads * elem * e + elem * m * t.l + out
    return reads * elem * e + out


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


class Ops:
    """Device-side state of one workload: inputs, split records (or plain
    quantized operands), GEMM objects and outputs."""

    def __init__(self, torch, M, np, cfg, tensors, gemms, dev):
        self.torch, self.M, self.cfg = torch, M, cfg
        self.tensors, self.gemms = tensors, gemms
        self.A = {n: (torch.from_numpy(t.bits.view(np.int16)).view(torch.bfloat16) if t.dtype == "bf16"
                      else torch.from_numpy(np.ascontiguousarray(t.values))).to(dev)
                  for n, t in tensors.items()}
        self.sk = {}
        for n, t in tensors.items():
            if t.k and t.sketch == "gaussian":
                self.sk[n] = {"omega": torch.from_numpy(t.omega.view(np.int16)).view(torch.bfloat16).to(dev)
                              .contiguous()}
            elif t.k:
                self.sk[n] = {"columns": torch.from_numpy(t.columns.astype(np.int32)).to(dev)}
        self.recs = {}
        for n, t in tensors.items():
            if t.k:
                self.recs[n] = M.empty_split(t.shape[0], t.shape[1], t.k, t.fmt, t.orientations, dev)
            else:
                self.recs[n] = M.SplitRecord(t.shape[0], t.shape[1], 0, M._FMT[t.fmt])
                self.quantize(n)
        self.gobj, self.outs = {}, {}
        for out, a, ao, b, bo in gemms:
            g = M.GemmNT(self.recs[a], ao == "t", self.recs[b], bo == "t")
            self.gobj[out] = g
            self.outs[out] = torch.empty(g.rows, g.cols, dtype=torch.float32, device=dev)

    def quantize(self, n):
        """The unsplit operand n quantized in each orientation it is used in."""
        t, rec, M = self.tensors[n], self.recs[n], self.M
        if "n" in t.orientations:
            rec.R_q = M.fp4_block_quant(self.A[n], t.fmt, transpose=False, out=rec.R_q)
        if "t" in t.orientations:
            rec.Rt_q = M.fp4_block_quant(self.A[n], t.fmt, transpose=True, out=rec.Rt_q)

    def split(self, n):
        t = self.tensors[n]
        if t.k:
            self.M.metis_split(self.A[n], t.l, t.k, t.fmt, out=self.recs[n], **self.sk[n])
        else:
            self.quantize(n)

    def gemm(self, out):
        self.gobj[out].prepare()
        self.gobj[out].main(self.outs[out])


def timed_ms(torch, fn, reps, stream=None, flush=None):
    """Per-rep event times (ms) of fn() on the current stream, flush() run
    before each rep outside the events."""
    ev = lambda: torch.cuda.Event(enable_timing=True)
    pairs = []
    for _ in range(reps):
        if flush is not None:
            flush()
        e0, e1 = ev(), ev()
        e0.record()
        fn()
        e1.record()
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in pairs]


def roofline_leg(torch, ops, reps, in_step_ms):
    """gemm_mx_kernel timed alone: every GEMM of the step, reps launches back
    to back on one stream, each launch between HIP events."""
    per = {}
    for out in ops.gobj:
        ops.gobj[out].prepare()
        ts = timed_ms(torch, lambda: ops.gobj[out].main(ops.outs[out]), reps)
        per[out] = statistics.mean(ts)
    shapes = {n: t.shape for n, t in ops.tensors.items()}
    flops = {g[0]: 2 * (lambda d: d[0] * d[1] * d[2])(gemm_dims(shapes, g)) for g in ops.gemms}
    avg_ms = statistics.mean(per.values())
    per_launch = statistics.mean(flops.values())
    achieved = per_launch / (avg_ms / 1e3) / 1e12
    in_step = per_launch / (in_step_ms / 1e3) / 1e12
    return {"bound": "mfma", "kernel": "gemm_mx_kernel (main MXFP4 GEMM + low-rank correction)",
            "achieved": round(achieved, 2), "peak": FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / FP4_PEAK_TFLOPS, 4), "traffic": gemm_traffic(),
            "flop_per_launch": per_launch, "avg_launch_us": round(avg_ms * 1e3, 1),
            "launch_us": {o: round(v * 1e3, 1) for o, v in per.items()},
            "timing": "%d launches of each of the step's six GEMMs back to back on one stream, HIP events around "
                      "each launch" % reps,
            "in_step_achieved": round(in_step, 2), "in_step_frac": round(in_step / FP4_PEAK_TFLOPS, 4),
            "in_step_avg_launch_us": round(in_step_ms * 1e3, 1)}


def split_hbm_leg(torch, ops, dev, reps):
    """Each split alone with the Infinity Cache flushed before every rep:
    median ms and algorithmic GB/s; the standalone quantizer likewise."""
    junk = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    flush = lambda: junk.fill_(1.0)
    out = {}
    for n, t in ops.tensors.items():
        ms = statistics.median(timed_ms(torch, lambda: ops.split(n), reps, flush=flush))
        nb = split_bytes(t, t.orientations)
        out[n] = {"ms": round(ms, 4), "GB/s": round(nb / (ms / 1e3) / 1e9, 1),
                  "frac": round(nb / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4), "algorithmic_bytes": nb}
    x = ops.A["X_up"]
    e = x.numel()
    for tr in (False, True):
        ms = statistics.median(timed_ms(torch, lambda: ops.M.fp4_block_quant(x, "mxfp4", transpose=tr), reps,
                                        flush=flush))
        nb = 2 * e + e // 2 + e // 32
        out["quant_X_up_" + ("t" if tr else "n")] = {"ms": round(ms, 4), "GB/s": round(nb / (ms / 1e3) / 1e9, 1),
                                                      "frac": round(nb / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                                                      "algorithmic_bytes": nb}
    del junk
    return out


def config_leg(torch, np, M, synth, cfg, dev, steps, warmup):
    """One workload as a step of its own on the current stream: its splits
    (or quantization of unsplit operands), then its GEMMs."""
    t0 = time.perf_counter()
    tensors = {n: synth.make_tensor(cfg, n) for n in synth.TENSOR_NAMES[cfg]}
    log("config %d generated (%.1fs)" % (cfg, time.perf_counter() - t0))
    gemms = synth.GEMMS[cfg]
    ops = Ops(torch, M, np, cfg, tensors, gemms, dev)
    shapes = {n: t.shape for n, t in tensors.items()}
    flops = gemm_flops(shapes, gemms)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    marks = []

    def step(record):
        e = {}
        for n in tensors:
            e0, e1 = ev(), ev()
            e0.record()
            ops.split(n)
            e1.record()
            e[n] = (e0, e1)
        for g in gemms:
            e0, e1, e2 = ev(), ev(), ev()
            e0.record()
            ops.gobj[g[0]].prepare()
            e1.record()
            ops.gobj[g[0]].main(ops.outs[g[0]])
            e2.record()
            e[g[0]] = (e0, e1, e2)
        if record:
            marks.append(e)

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    s0, s1 = ev(), ev()
    s0.record()
    for _ in range(steps):
        step(True)
    s1.record()
    torch.cuda.synchronize()
    step_ms = s0.elapsed_time(s1) / steps
    split_ms = {n: statistics.mean(m[n][0].elapsed_time(m[n][1]) for m in marks) for n in tensors}
    prep_ms = {g[0]: statistics.mean(m[g[0]][0].elapsed_time(m[g[0]][1]) for m in marks) for g in gemms}
    main_ms = {g[0]: statistics.mean(m[g[0]][1].elapsed_time(m[g[0]][2]) for m in marks) for g in gemms}
    gemm_ms = sum(prep_ms.values()) + sum(main_ms.values())
    main_tf = flops / (sum(main_ms.values()) / 1e3) / 1e12
    fmt = next(iter(tensors.values())).fmt
    t_any = next(t for t in tensors.values() if t.k)
    out = {"workload": CONFIG_LABEL[cfg], "fmt": fmt, "k": t_any.k, "l": t_any.l, "sketch": t_any.sketch,
           "gemm_gflop": round(flops / 1e9, 2), "ms_per_step": round(step_ms, 4),
           "TFLOP/s": round(flops / (step_ms / 1e3) / 1e12, 2),
           "gemm_TFLOP/s": round(flops / (gemm_ms / 1e3) / 1e12, 2),
           "split_ms": {n: round(v, 4) for n, v in split_ms.items()},
           "split_GB/s": {n: round(split_bytes(tensors[n], tensors[n].orientations) / (v / 1e3) / 1e9, 1)
                          for n, v in split_ms.items()},
           "gemm_prepare_ms": {o: round(v, 4) for o, v in prep_ms.items()},
           "gemm_main_ms": {o: round(v, 4) for o, v in main_ms.items()},
           "main_gemm_TFLOP/s": round(main_tf, 2),
           "main_gemm_frac_fp4_peak": round(main_tf / FP4_PEAK_TFLOPS, 4)}
    if fmt == "nvfp4":
        out["main_gemm_frac_f16_peak"] = round(main_tf / F16_PEAK_TFLOPS, 4)
    log("config %d: %.3f ms/step, main GEMMs %.0f TFLOP/s" % (cfg, step_ms, main_tf))
    del ops
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


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
        ms = statistics.mean(timed_ms(torch, lambda: M.metis_mean_split(A[n], "mxfp4", out=rec), reps))
        elems = m_ * n_
        nbytes = 2 * 2 * elems + 2 * (elems // 2 + elems // 32)
        out[n] = {"ms": round(ms, 4), "GB/s": round(nbytes / (ms / 1e3) / 1e9, 1), "algorithmic_bytes": nbytes}
    return out


def power_split_leg(torch, ops, reps=5):
    """The spectral split with q = 1 power iteration (two more passes over A)
    timed alone on X_up, after the timed steps, next to q = 0."""
    t, M = ops.tensors["X_up"], ops.M
    out = {}
    for q in (0, 1):
        f = lambda: M.metis_split(ops.A["X_up"], t.l, t.k, "mxfp4", out=ops.recs["X_up"], q=q, **ops.sk["X_up"])
        f()
        torch.cuda.synchronize()
        out["q%d_ms" % q] = round(statistics.mean(timed_ms(torch, f, reps)), 4)
    return {"tensor": "X_up 8192x4096 bf16, k 64, l 80", **out}


def optim_leg(torch, ops, reps=10):
    """The optimizer-side kernels timed alone: the dual-range regularizer
    (loss and gradient) on W_up, and the adaptive spectral learning rate on
    the fp32 dW_up of the step (its split at k = 64, l = 80 first, untimed).
    HBM rate against algorithmic bytes (regularizer: W read, gradient
    written; rescale: G read and written)."""
    M = ops.M
    out = {}
    W = ops.A["W_up"]
    e = W.numel()
    loss, grad = M.metis_dual_range_reg(W, 0.002, 0.05, 10.0, 100.0)
    torch.cuda.synchronize()
    ms = statistics.median(timed_ms(torch, lambda: M.metis_dual_range_reg(W, 0.002, 0.05, 10.0, 100.0, grad=grad),
                                    reps))
    nb = 2 * e + 4 * e
    out["dual_range_W_up"] = {"ms": round(ms, 4), "GB/s": round(nb / (ms / 1e3) / 1e9, 1), "algorithmic_bytes": nb}
    G = ops.outs["dW_up"]
    t = ops.tensors["W_up"]
    om = ops.sk["W_up"]["omega"]
    rec = M.metis_split(G, t.l, t.k, "mxfp4", omega=om, orientations=("n",))
    torch.cuda.synchronize()
    ms = statistics.median(timed_ms(torch, lambda: M.metis_spectral_lr_rescale(G, rec, 8, 8.0), reps))
    nb = 8 * G.numel()
    out["spectral_lr_dW_up"] = {"ms": round(ms, 4), "GB/s": round(nb / (ms / 1e3) / 1e9, 1),
                                "algorithmic_bytes": nb, "k": t.k, "r_ref": 8, "gamma_max": 8.0}
    return out


def profile_splits(torch, ops, reps):
    """For kernel profiles of the step's kernels alone (their durations and
    HBM rates are read from the profiler, not printed): each of the six
    spectral splits reps times back to back on one stream, the standalone
    MXFP4 quantizer on X_up in both orientations reps times, then each of the
    six GEMMs (prepare + main) reps times. Replaces the steps."""
    for n in ops.tensors:
        for _ in range(reps):
            ops.split(n)
        torch.cuda.synchronize()
        log("profiled split %s x %d" % (n, reps))
    x = ops.A["X_up"]
    for _ in range(reps):
        ops.M.fp4_block_quant(x, "mxfp4")
        ops.M.fp4_block_quant(x, "mxfp4", transpose=True)
    torch.cuda.synchronize()
    log("profiled fp4_block_quant X_up (both orientations) x %d" % reps)
    for out in ops.gobj:
        for _ in range(reps):
            ops.gemm(out)
        torch.cuda.synchronize()
        log("profiled GEMM %s (prepare + main) x %d" % (out, reps))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(tensors, gemms, gemm_total_flops):
    """The fp64 oracle on a bounded sample of the step: the full split and
    quantization of X_up (8192 x 4096, both orientations) and of W_up, and
    the full forward GEMM Y_up (962 GFLOP in fp64 over the dequantized
    operands). The step time is extrapolated from them: the six splits by
    element count, the six GEMMs (equal flops) by count."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import linear as OL
    from oracle import split as OS

    t, w = tensors["X_up"], tensors["W_up"]
    A = t.values.astype(np.float64)
    t0 = time.perf_counter()
    r = OS.spectral_split(A, t.l, t.k, omega=t.omega_values().astype(np.float64))
    rec_x = OS.quantize_record("mxfp4", r["R"], r["U"], r["S"], r["V"], orientations=("n", "t"))
    t_split = time.perf_counter() - t0
    del A, r
    rw = OS.spectral_split(w.values.astype(np.float64), w.l, w.k, omega=w.omega_values().astype(np.float64))
    rec_w = OS.quantize_record("mxfp4", rw["R"], rw["U"], rw["S"], rw["V"], orientations=("n",))
    del rw
    t0 = time.perf_counter()
    OL.linear_fwd(rec_x, rec_w)
    t_gemm = time.perf_counter() - t0
    elems = {n: x.shape[0] * x.shape[1] for n, x in tensors.items()}
    split_s = t_split * sum(elems.values()) / elems["X_up"]
    gemm_s = t_gemm * len(gemms)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": round(gemm_total_flops / (split_s + gemm_s) / 1e12, 6), "unit": "TFLOP/s",
            "cores": threads, "kind": "oracle", "nproc": os.cpu_count(), "cpu_model": cpu_model(),
            "sample": "fp64 oracle (numpy, %d BLAS threads): full split + quantization of X_up 8192x4096 (both "
                      "orientations) in %.1f s and the full Y_up GEMM (962 GFLOP, 8192x14336x4096) in %.1f s; "
                      "the step extrapolated by element count (6 splits) and by count (6 equal GEMMs)"
                      % (threads, t_split, t_gemm)}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--reps", type=int, default=5, help="reps of each isolated kernel / split leg")
    ap.add_argument("--configs", default="2,3,5", help="other workloads timed after the headline step ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-legs", action="store_true", help="the headline step only")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="run a plain copy of MIB MiB ahead of the steps (counter calibration)")
    ap.add_argument("--configs-only", action="store_true",
                    help="only the --configs workloads, each as its step (for per-workload profiles); prints "
                         "their JSON")
    ap.add_argument("--profile-splits", type=int, default=0, metavar="REPS",
                    help="instead of the steps, run each split, the quantizer and each GEMM REPS times alone "
                         "(for profiles)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
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
    if args.configs_only:
        out = {}
        for c in [int(c) for c in args.configs.split(",") if c.strip()]:
            out[CONFIG_LABEL[c]] = config_leg(torch, np, M, synth, c, dev, args.steps, args.warmup)
        print(json.dumps({"configs": out}), flush=True)
        return
    names = synth.TENSOR_NAMES[CFG]
    gemms = synth.GEMMS[CFG]
    t0 = time.perf_counter()
    tensors = {}
    for n in names:
        tensors[n] = synth.make_tensor(CFG, n)
        tensors[n].orientations = ("n", "t")
        log("generated %s %s (%.1fs)" % (n, tensors[n].shape, time.perf_counter() - t0))
    shapes = {n: t.shape for n, t in tensors.items()}
    total_flops = gemm_flops(shapes, gemms)
    ops = Ops(torch, M, np, CFG, tensors, gemms, dev)
    if args.profile_splits:
        profile_splits(torch, ops, args.profile_splits)
        return
    outs = ops.outs

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
    ev = lambda: torch.cuda.Event(enable_timing=True)
    split_ev = [{n: (ev(), ev()) for n in names} for _ in range(args.steps)]
    main_ev = [{o: (ev(), ev()) for o in outs} for _ in range(args.steps)]

    def step(i):
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
                    ops.split(n)
                    if rec:
                        split_ev[i][n][1].record(s)
                    done[n].record(s)
                    enqueued.add(n)
                else:
                    _, a, ao, b, bo = gemm_of[n]
                    assert a in enqueued and b in enqueued
                    s.wait_event(done[a])
                    s.wait_event(done[b])
                    ops.gobj[n].prepare()
                    if rec:
                        main_ev[i][n][0].record(s)
                    ops.gobj[n].main(outs[n])
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
    host_s = 0.0
    for i in range(args.steps):
        h0 = time.perf_counter()
        step(i)
        host_s += time.perf_counter() - h0
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    value = total_flops / (ms_per_step / 1e3) / 1e12
    log("step %.3f ms -> %.1f TFLOP/s" % (ms_per_step, value))
    split_ms = {n: sum(e[n][0].elapsed_time(e[n][1]) for e in split_ev) / args.steps for n in names}
    main_ms = {o: sum(e[o][0].elapsed_time(e[o][1]) for e in main_ev) / args.steps for o in outs}
    in_step_main_ms = sum(main_ms.values()) / len(gemms)

    line = {
        "metric": "TFLOP/s of spectral-FP4 linear fwd+bwd at LLaMA-3-8B shapes; split ms",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4", "data": "synthetic",
        "config": {"workload": "llama3-8b-ffn-up+down-w4a4g4", "tokens": 8192, "hidden": 4096, "ffn": 14336,
                   "k": 64, "l": 80, "fmt": "mxfp4", "sketch": "gaussian", "gemm_gflop_per_step":
                   round(total_flops / 1e9, 2)},
        "split_ms": {n: round(v, 4) for n, v in split_ms.items()},
        "gemm_main_ms": {o: round(v, 4) for o, v in main_ms.items()},
        "host_enqueue_ms_per_step": round(host_s * 1e3 / args.steps, 4),
    }
    torch.cuda.synchronize()
    if not args.no_legs:
        line["roofline"] = roofline_leg(torch, ops, args.reps, in_step_main_ms)
        log("roofline: gemm_mx_kernel %.1f us per launch alone" % line["roofline"]["avg_launch_us"])
        line["split_hbm"] = split_hbm_leg(torch, ops, dev, args.reps)
        log("split HBM leg done")
        line["mean_split"] = mean_split_leg(torch, M, ops.A, tensors)
        line["power_split"] = power_split_leg(torch, ops)
        line["optim"] = optim_leg(torch, ops)
        cfgs = [int(c) for c in args.configs.split(",") if c.strip()]
        if cfgs:
            line["configs"] = {}
            for c in cfgs:
                line["configs"][CONFIG_LABEL[c]] = config_leg(torch, np, M, synth, c, dev, max(3, args.steps // 4),
                                                              2)
    del ops
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline(tensors, gemms, total_flops)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the MI355X microscaling-FP4 hot path; prints ONE JSON line.

Timed step (``value``): one pass of block-wise FP4 quantization over the
4096x4096 bf16 workload in all its variants -- two seeded distributions
(Gaussian std 0.02; Laplace b=0.02 with 16 of 4096 columns x50) x {MXFP4,
NVFP4} x {no rotation, block Hadamard of the block size}, as one
fp4_quantize_batch call: two launches of the grouped kernel (the four MXFP4
encodings and the four NVFP4 tensor maxima, then the four NVFP4 encodings).
Inputs are resident in HBM; every variant reads its own input buffers, and the
step cycles through several copies of every input and output, so that the
256 MB last-level cache serves neither one variant's read to another nor a
repeat.

``value`` = algorithmic bytes of the step (bf16 read once + codes + scales)
divided by the step time, in GB/s, over K eagerly issued steps (after W
warmup steps and an untimed settle of ``--settle`` seconds of steps); the same
step recorded as a HIP graph and replayed, and the step as eight separate
fp4_quantize calls (one stream; two streams; NVFP4 in two passes) are
reported beside it.  ``roofline`` reports the grouped kernel (its two launches
per step); their duration is measured live with HIP events on the launching
stream around a graph of back-to-back steps (a Python loop of single calls
would be bound by the host).

Also reported in the same line: NMSE of every variant (GPU, and oracle vs GPU
on a sample), the oracle's own throughput on a bounded sample
(``cpu_baseline``), and the GEMM measurements (Llama-3-8B and Llama-3-70B
linear shapes, MXFP4 on the scaled MFMA and NVFP4 on the dequantize-to-fp16
path, plus the layer-wise speedup of quantize+GEMM over torch's bf16 GEMM).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12         # B/s, MI355X HBM3E
BATCH_KERNEL = "quant_batch_kernel (2 launches per step)"
PEAK_FP4 = 10.1e15        # dense MXFP4 MFMA, flop/s
PEAK_F16 = 2.5e15         # dense fp16/bf16 MFMA, flop/s
METRIC = "quant GB/s (% HBM peak); FP4 GEMM TFLOPS (% MFMA peak); NMSE vs oracle"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of untimed steps before the measurements (the first few "
                         "hundred steps after idle run up to 15%% slower)")
    ap.add_argument("--copies", type=int, default=8)
    ap.add_argument("--streams", type=int, default=2, choices=(1, 2, 3),
                    help="streams of the eager step: 2 or 3 issue the MXFP4 quantizations on "
                         "the other stream(s) beside the NVFP4 ones")
    ap.add_argument("--no-gemm", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-search", action="store_true",
                    help="skip the timings of the searching block-scale rules")
    ap.add_argument("--gemm-iters", type=int, default=10)
    ap.add_argument("--no-copy-probe", action="store_true",
                    help="skip the untimed 64 MiB device copy used to calibrate HBM byte counters")
    ap.add_argument("--only-gemm", default=None, metavar="SHAPES",
                    help="run only these GEMMs a few times and print their timings (for profiler "
                         "runs): comma-separated fmt:MxNxK with fmt mx, nv, mxint4, nvint4 or "
                         "w4mx / w4nv (weight-only), e.g. mx:4096x4096x4096,mx:1x28672x8192")
    ap.add_argument("--vendor-mxfp4", action="store_true",
                    help="run only a side-by-side of this library's MXFP4 GEMM and hipBLASLt's "
                         "(torch._scaled_mm) on the large Llama shapes, as context")
    return ap.parse_args()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the recorded PMC runs, or None when
    no record exists or the kernel sources changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "fp4_microscaling_quantization_amd", "traffic_pmc.json")
    try:
        rec = json.load(open(path))
    except OSError:
        return None, "no PMC record"
    h = hashlib.sha256()
    for src in rec["sources"]:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    if h.hexdigest() != rec["sources_sha256"]:
        return None, "kernel sources changed since the PMC record was taken"
    b = rec["bytes_per_launch"].get(kernel)
    if b is None:
        return None, "no PMC record for this kernel"
    return b, "FETCH_SIZE + WRITE_SIZE per launch, calibrated by a 64 MiB copy (%s)" % rec["profile"]


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (quantization "
              "shards by rows with no exchange; see the design notes). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import fp4_microscaling_quantization_amd as fp4
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    fp4.lib()
    stream = torch.cuda.current_stream()

    def sh_now():
        # the launching stream: torch's current stream (the capture stream
        # while a graph is being recorded)
        return torch.cuda.current_stream().cuda_stream

    # Untimed plain device copy of known size (64 MiB read + 64 MiB written):
    # under a rocprofv3 --pmc run its FETCH_SIZE / WRITE_SIZE readings give the
    # factor that converts those counters to bytes for the kernels below.
    if not args.no_copy_probe:
        src = torch.empty(64 << 20, dtype=torch.uint8, device=dev)
        src.fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.only_gemm:
        only_gemm(args, torch, fp4, workloads, dev)
        return
    if args.vendor_mxfp4:
        vendor_mxfp4(torch, fp4, dev)
        return

    # ------------------------------------------------------------ workload
    rows, cols = 4096, 4096
    n = rows * cols
    t0 = time.time()
    host = {d: workloads.cfg2_tensor(d, 0) for d in ("gauss", "laplace")}
    log("host inputs %.1fs" % (time.time() - t0))

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    copies = max(1, args.copies)
    xs = {}
    for d, b in host.items():
        base = to_dev(b)
        xs[d] = [base] + [base.clone() for _ in range(copies - 1)]

    variants = [(d, fmt, rot) for d in ("gauss", "laplace")
                for fmt in (fp4.FMT_MXFP4, fp4.FMT_NVFP4) for rot in (False, True)]
    # every variant reads its own buffers (the same values), so no variant's
    # read is served from the cache lines another variant brought in
    xv = {v: [x.clone() for x in xs[v[0]]] for v in variants}
    FN = {fp4.FMT_MXFP4: "mxfp4", fp4.FMT_NVFP4: "nvfp4", fp4.FMT_MXINT4: "mxint4",
          fp4.FMT_NVINT4: "nvint4"}

    def vname(v):
        return "%s/%s/%s" % (v[0], FN[v[1]], "h%d" % fp4.BLOCK[v[1]] if v[2] else "plain")

    outs = {}
    for v in variants:
        d, fmt, rot = v
        lay = fp4.SCALES_GEMM if fmt == fp4.FMT_MXFP4 else fp4.SCALES_ROWMAJOR
        cfg = fp4.qconfig(fmt, rot, lay)
        lst = []
        for c in range(copies):
            codes = torch.empty(fp4.fp4_codes_bytes(rows, cols), dtype=torch.uint8, device=dev)
            scales = torch.empty(fp4.fp4_scales_bytes(cfg, rows, cols), dtype=torch.uint8, device=dev)
            gs = torch.zeros(1, dtype=torch.float32, device=dev)
            lst.append(fp4.Quantized(codes, scales, gs, cfg, rows, cols))
        outs[v] = lst
    # NVFP4 workspace: amax-pass partials, then the single-pass exchange
    # region (zero before its first use)
    wsb = fp4.fp4_workspace_bytes(fp4.qconfig(fp4.FMT_NVFP4), rows, cols)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
    # the step as one batch per buffer copy (NVFP4 computes its tensor scale)
    bwsb = fp4.fp4_quantize_batch_workspace_bytes(len(variants))
    bws = torch.zeros(bwsb, dtype=torch.uint8, device=dev)
    batch_jobs = []
    for c in range(copies):
        jl = []
        for v in variants:
            q = outs[v][c]
            jl.append(fp4.quant_job(q.cfg, xv[v][c].data_ptr(), fp4.DT_BF16, rows, cols, cols,
                                    q.codes.data_ptr(), q.scales.data_ptr(),
                                    q.global_scale.data_ptr(), fp4.GS_COMPUTE))
        batch_jobs.append(fp4.job_array(jl))

    def run_batch(c, sh=None):
        rc = fp4.fp4_quantize_batch(len(variants), batch_jobs[c], bws.data_ptr(), bwsb,
                                    sh if sh is not None else sh_now())
        if rc != 0:
            raise RuntimeError("quantize batch failed: %d" % rc)

    def alg_bytes(fmt):
        G = fp4.BLOCK[fmt]
        return n * 2 + n // 2 + n // G

    def call(v, c, mode, sh=None):
        """One C-ABI call of variant v on buffer copy c.  mode 'step' is the
        production path (NVFP4 computes its tensor scale and encodes in one
        launch); 'two_pass' the same with the amax pass and the quantize pass;
        'amax' runs only the NVFP4 tensor-scale pass; 'given' only the NVFP4
        quantize kernel with the tensor scale already in place."""
        d, fmt, rot = v
        x = xv[v][c]
        q = outs[v][c]
        h = sh if sh is not None else sh_now()
        if fmt == fp4.FMT_MXFP4:
            rc = fp4.fp4_quantize(q.cfg, x.data_ptr(), fp4.DT_BF16, rows, cols, cols,
                                  q.codes.data_ptr(), q.scales.data_ptr(), None, fp4.GS_COMPUTE,
                                  None, 0, h)
        elif mode == "amax":
            rc = fp4.fp4_global_scale(q.cfg, x.data_ptr(), fp4.DT_BF16, rows, cols, cols,
                                      q.global_scale.data_ptr(), ws.data_ptr(), wsb, h)
        else:
            gs_mode = {"given": fp4.GS_GIVEN, "two_pass": fp4.GS_COMPUTE}.get(
                mode, fp4.GS_COMPUTE_ONE_PASS)
            rc = fp4.fp4_quantize(q.cfg, x.data_ptr(), fp4.DT_BF16, rows, cols, cols,
                                  q.codes.data_ptr(), q.scales.data_ptr(),
                                  q.global_scale.data_ptr(), gs_mode, ws.data_ptr(), wsb, h)
        if rc != 0:
            raise RuntimeError("quantize failed: %d" % rc)

    def run_step(c, mode="step", sh=None):
        for v in variants:
            call(v, c, mode, sh)

    # The step's eight quantizations are independent.  With more than one
    # stream the MXFP4 ones go round-robin to the other stream(s) (default
    # priority) and overlap the NVFP4 single-pass launches, which stay in order
    # on the main stream (two of them must never run at once).
    sides = [torch.cuda.Stream() for _ in range(args.streams - 1)]
    # stream handles looked up once (torch's current-stream query costs about
    # as much host time as a launch)
    h_main = stream.cuda_stream
    h_sides = [sd.cuda_stream for sd in sides]

    def run_step_eager(c):
        if not sides:
            run_step(c, "step", h_main)
            return
        k = 0
        for v in variants:
            if v[1] == fp4.FMT_MXFP4:
                call(v, c, "step", h_sides[k % len(h_sides)])
                k += 1
            else:
                call(v, c, "step", h_main)

    one_pass = all(fp4.fp4_quantize_one_pass_fits(outs[v][0].cfg, fp4.DT_BF16, rows, cols, cols)
                   for v in variants if v[1] == fp4.FMT_NVFP4)

    def capture(fn):
        # the step's kernels recorded once; replays launch them with no host work
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    # untimed steps until the device has run the step for args.settle seconds
    t_settle = time.perf_counter()
    k = 0
    while time.perf_counter() - t_settle < args.settle:
        for _ in range(20):
            run_batch(k % copies)
            k += 1
        torch.cuda.synchronize()
    log("settled after %d untimed steps" % k)

    # the same step as one HIP graph per buffer copy, replayed
    step_graphs = [capture(lambda c=c: run_batch(c)) for c in range(copies)]
    for w in range(args.warmup):
        step_graphs[w % copies].replay()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s_ in range(args.steps):
        step_graphs[s_ % copies].replay()
    torch.cuda.synchronize()
    graph_s = (time.perf_counter() - t_start) / max(1, args.steps)
    del step_graphs

    # timed region of the reported value: K eager steps (one batch call each)
    # between two synchronisations (HIP events on the launching stream
    # alongside)
    for w in range(args.warmup):
        run_batch(w % copies, h_main)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    ev0.record(stream)
    for s_ in range(args.steps):
        run_batch(s_ % copies, h_main)
    ev1.record(stream)
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    step_s = (t_end - t_start) / max(1, args.steps)
    step_s_events = ev0.elapsed_time(ev1) * 1e-3 / max(1, args.steps)
    # the step as eight separate calls, the MXFP4 ones on other stream(s)
    for w in range(args.warmup):
        run_step_eager(w % copies)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for sd in sides:
        sd.wait_stream(stream)
    for s_ in range(args.steps):
        run_step_eager(s_ % copies)
    for sd in sides:
        stream.wait_stream(sd)
    torch.cuda.synchronize()
    calls_streams_s = (time.perf_counter() - t_start) / max(1, args.steps)
    # the same step on one stream
    for w in range(args.warmup):
        run_step(w % copies, "step", h_main)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s_ in range(args.steps):
        run_step(s_ % copies, "step", h_main)
    torch.cuda.synchronize()
    one_stream_s = (time.perf_counter() - t_start) / max(1, args.steps)
    step_bytes = sum(alg_bytes(v[1]) for v in variants)
    value_gbs = step_bytes / step_s / 1e9
    # the same step with the NVFP4 tensor scale from a separate amax pass
    for w in range(args.warmup):
        run_step(w % copies, "two_pass", h_main)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s_ in range(args.steps):
        run_step(s_ % copies, "two_pass", h_main)
    torch.cuda.synchronize()
    two_pass_s = (time.perf_counter() - t_start) / max(1, args.steps)

    # Per-kernel launch durations, live: a graph of back-to-back launches of
    # one kernel over the rotating buffer copies, replayed between one pair of
    # HIP events on the launching stream (average = kernel time + the gap
    # between graph nodes).
    reps = 4 * copies
    kern = {}
    # the grouped kernel: two launches per step, timed over a graph of steps
    amax_reads = n * 2 * sum(1 for v in variants if v[1] != fp4.FMT_MXFP4)
    run_batch(0)
    torch.cuda.synchronize()
    g = capture(lambda: [run_batch(i % copies) for i in range(reps)])
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del g
    kern[BATCH_KERNEL] = {"avg_us": us, "alg_bytes": step_bytes + amax_reads,
                          "gbs": (step_bytes + amax_reads) / (us * 1e-6) / 1e9, "launches": 2 * reps,
                          "in_step": True}
    for (d, fmt, rot) in variants:
        if d != "gauss":
            continue
        v = (d, fmt, rot)
        tag = "rot" if rot else "plain"
        if fmt == fp4.FMT_MXFP4:
            parts = [("quant_mx_gemm_kernel<%s>" % tag, "step", alg_bytes(fmt), False)]
        else:
            # the step's single launch, then the two passes it replaces
            parts = [("quant_nv_fused_kernel<nvfp4,%s,4>" % tag, "step", alg_bytes(fmt), False),
                     ("amax_chunk_kernel<%s>" % tag, "amax", n * 2, False),
                     ("quant_rows_kernel<nvfp4,%s,2>" % tag, "given", alg_bytes(fmt), False)]
        for label, mode, nbytes, in_step in parts:
            call(v, 0, mode)
            torch.cuda.synchronize()
            g = capture(lambda: [call(v, i % copies, mode) for i in range(reps)])
            g.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            kern[label] = {"avg_us": us, "alg_bytes": nbytes, "gbs": nbytes / (us * 1e-6) / 1e9,
                           "launches": reps, "in_step": in_step}
            del g
    dom = max((k for k in kern if kern[k]["in_step"]), key=lambda k: kern[k]["avg_us"])
    dk = kern[dom]
    traffic, traffic_note = measured_traffic(dom.split(" + ")[0])
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(dk["gbs"], 1),
                "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": round(dk["gbs"] * 1e9 / PEAK_HBM, 4),
                "traffic": traffic, "traffic_note": traffic_note,
                "alg_bytes_per_step": dk["alg_bytes"], "avg_step_us": round(dk["avg_us"], 3),
                "launches_per_step": 2,
                "alg_bytes_min": step_bytes,
                "achieved_min": round(step_bytes / (dk["avg_us"] * 1e-6) / 1e9, 1),
                "frac_min": round(step_bytes / (dk["avg_us"] * 1e-6) / PEAK_HBM, 4),
                "alg_bytes_min_note": "the step's own bytes only (each input read once, codes, "
                                      "scales), without the NVFP4 maximum pass's second read",
                "alg_bytes_note": "the step's bytes (each input read once, codes, scales) plus the "
                                  "second read of the four NVFP4 inputs by their tensor-maximum "
                                  "pass"}
    log("step %.3f ms (eager), %.3f ms (graph), %.1f GB/s; dominant %s %.2f us"
        % (1e3 * step_s, 1e3 * graph_s, value_gbs, dom, dk["avg_us"]))

    # ------------------------------------- scale rules, formats and variants
    # The other quantizer configurations on the same input: the searching
    # rules (MSE window, Four Over Six), the INT4-element formats, 64/128-point
    # MX rotations with a sign diagonal, stochastic rounding and NVFP4 16x16
    # blocks.  The quantize kernel alone (NV formats with their tensor scale
    # given), per launch, and the reconstruction error next to the FP4 format
    # with the same layout and absmax scales, nearest rounding.
    search = {}
    if not args.no_search:
        mask = 0x0123456789ABCDEF0FEDCBA987654321
        variants_x = []   # (name, fmt, rot, qconfig keyword arguments)
        for rot in (False, True):
            tag = "h" if rot else "plain"
            variants_x += [("mxfp4/mse/" + tag, fp4.FMT_MXFP4, rot, dict(rule=fp4.SCALE_MSE)),
                           ("nvfp4/mse/" + tag, fp4.FMT_NVFP4, rot, dict(rule=fp4.SCALE_MSE)),
                           ("nvfp4/4over6/" + tag, fp4.FMT_NVFP4, rot, dict(rule=fp4.SCALE_FOUR_OVER_SIX)),
                           ("mxint4/absmax/" + tag, fp4.FMT_MXINT4, rot, {}),
                           ("nvint4/absmax/" + tag, fp4.FMT_NVINT4, rot, {}),
                           ("mxfp4/stochastic/" + tag, fp4.FMT_MXFP4, rot, dict(rounding=1, seed=(1, 2))),
                           ("nvfp4/stochastic/" + tag, fp4.FMT_NVFP4, rot, dict(rounding=1, seed=(1, 2)))]
        variants_x += [("mxfp4/h64-signed", fp4.FMT_MXFP4, 64, dict(signs=mask)),
                       ("mxfp4/h128", fp4.FMT_MXFP4, 128, {}),
                       ("mxfp4/h128-signed", fp4.FMT_MXFP4, 128, dict(signs=mask)),
                       ("nvfp4/h16-signed", fp4.FMT_NVFP4, True, dict(signs=mask)),
                       ("nvfp4/16x16-blocks", fp4.FMT_NVFP4, False, dict(block_rows=16))]
        for name, fmt, rot, kw in variants_x:
            lay = fp4.SCALES_GEMM if fmt in fp4.MX_FORMATS else fp4.SCALES_ROWMAJOR
            cfg = fp4.qconfig(fmt, rot, lay, **kw)
            twin_rot = rot is not False
            fp_twin = fp4.FMT_MXFP4 if fmt in fp4.MX_FORMATS else fp4.FMT_NVFP4
            qs = []
            for c in range(copies):
                base = outs[("gauss", fp_twin, twin_rot)][c]
                qs.append(fp4.Quantized(torch.empty_like(base.codes), torch.empty_like(base.scales),
                                        base.global_scale.clone(), cfg, rows, cols))

            def qcall(c, d="gauss", qs=qs):
                q = qs[c]
                rc = fp4.fp4_quantize(q.cfg, xs[d][c].data_ptr(), fp4.DT_BF16, rows, cols, cols,
                                      q.codes.data_ptr(), q.scales.data_ptr(),
                                      q.global_scale.data_ptr(), fp4.GS_GIVEN, None, 0, sh_now())
                if rc != 0:
                    raise RuntimeError("quantize failed: %d" % rc)

            if fmt not in fp4.MX_FORMATS:  # its own tensor scale, set once
                for q_ in qs:
                    fp4.global_scale(xs["gauss"][0], rotate=rot, out=q_.global_scale, fmt=fmt,
                                     signs=kw.get("signs", 0))
            qcall(0)
            torch.cuda.synchronize()
            g = capture(lambda: [qcall(i % copies) for i in range(reps)])
            g.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            del g
            ent = {"avg_us": round(us, 3), "gbs": round(alg_bytes(fmt) / (us * 1e-6) / 1e9, 1),
                   "frac": round(alg_bytes(fmt) / (us * 1e-6) / PEAK_HBM, 4)}
            for d in ("gauss", "laplace"):
                qd = fp4.quantize(xs[d][0], fmt, rotate=rot, scale_layout=lay, **kw)
                sd = fp4.error_sums(xs[d][0], qd).cpu().numpy()
                qa = outs[(d, fp_twin, twin_rot)][0]
                sa = fp4.error_sums(xs[d][0], qa).cpu().numpy()
                ent["nmse_" + d] = float(sd[0] / sd[1])
                ent["nmse_fp4_absmax_" + d] = float(sa[0] / sa[1])
            search[name] = ent
        log("variant timings done")

    # -------------------------------------------------------------- NMSE
    nmse = {}
    for v in variants:
        d, fmt, rot = v
        q = outs[v][0]
        sums = fp4.error_sums(xs[d][0], q).cpu().numpy()
        nmse[vname(v)] = {"gpu_full": float(sums[0] / sums[1])}

    # -------------------------------------------------------- CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(variants, host, alg_bytes, workloads, fp4)
        log("cpu baseline %.4f GB/s on 1 core (%.1fs), %.4f GB/s on %d threads (%.1fs)"
            % (cpu["value_1core"], cpu["seconds_1core"], cpu["value"], cpu["cores"],
               cpu["seconds"]))
    if not args.no_cpu_baseline:
        import oracle
        # NMSE of a 256-row sample, oracle vs GPU on the same rows (untimed)
        sample_rows = 256
        for v in variants:
            d, fmt, rot = v
            xh = workloads.bf16_bits_to_f32(host[d][:sample_rows])
            c_, s_, ts_ = oracle.quantize(xh, fmt, rotate=rot)
            ref = oracle.dequantize(c_, s_, fmt, ts_, inverse_rotate=rot)
            xd = to_dev(np.ascontiguousarray(host[d][:sample_rows]))
            qg = fp4.quantize(xd, fmt, rotate=rot)
            sg = fp4.error_sums(xd, qg).cpu().numpy()
            nmse[vname(v)].update({"oracle_sample": oracle.nmse(xh, ref),
                                   "gpu_sample": float(sg[0] / sg[1])})

    # ------------------------------------------ cfg1 / cfg3 (parity configs)
    cfg1 = bench_cfg1(torch, fp4, workloads, stream, sh_now, capture, args.no_cpu_baseline)
    log("cfg1 quantize %.2f us, dequantize %.2f us, error sums %.2f us"
        % (cfg1["quantize_us"], cfg1["dequantize_us"], cfg1["error_sums_us"]))
    cfg3 = bench_cfg3(torch, fp4, workloads, dev, stream, sh_now, capture)
    log("cfg3 " + ", ".join("%s %.2f us (%.3f of HBM)" % (k, v["avg_us"], v["frac"])
                            for k, v in cfg3["kernels"].items()))

    # --------------------------------------------------------------- GEMM
    gemm = None
    if not args.no_gemm:
        gemm = bench_gemm(args, torch, fp4, workloads, dev, stream)

    line = {
        "metric": METRIC, "value": round(value_gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(1e3 * step_s, 4),
        "ms_per_step_events": round(1e3 * step_s_events, 4),
        "ms_per_step_graph": round(1e3 * graph_s, 4),
        "ms_per_step_calls": round(1e3 * one_stream_s, 4),
        "ms_per_step_calls_streams": round(1e3 * calls_streams_s, 4),
        "ms_per_step_calls_two_pass": round(1e3 * two_pass_s, 4),
        "launch": ("eager: one fp4_quantize_batch call per step (2 launches of the grouped "
                   "kernel: 4 MXFP4 encodings + 4 NVFP4 tensor maxima, then 4 NVFP4 encodings); "
                   "ms_per_step_graph: that step as a replayed HIP graph; ms_per_step_calls: 8 "
                   "fp4_quantize calls on one stream (NVFP4 tensor amax and encoding in one "
                   "launch%s); ms_per_step_calls_streams: the same with the MXFP4 calls on %d "
                   "other stream(s); ms_per_step_calls_two_pass: 8 calls, NVFP4 with a separate "
                   "amax pass" % ("" if one_pass else ": not taken, two passes", args.streams - 1)),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "quantize 4096x4096 bf16 x {Gaussian 0.02, Laplace 0.02 + 16/4096 "
                               "cols x50} x {MXFP4 G32, NVFP4 G16 (tensor amax computed)} x {plain, "
                               "block Hadamard 32/16}", "rows": rows, "cols": cols,
                   "variants": len(variants), "buffer_copies": copies,
                   "step_alg_bytes": step_bytes},
        "frac_hbm_step": round(value_gbs * 1e9 / PEAK_HBM, 4),
        "roofline": roofline,
        "kernels": {k: {"avg_us": round(v["avg_us"], 3), "gbs": round(v["gbs"], 1),
                        "frac": round(v["gbs"] * 1e9 / PEAK_HBM, 4), "in_step": v["in_step"]}
                    for k, v in sorted(kern.items())},
        "kernel_timing": "per-kernel: a HIP graph of %d back-to-back launches over rotating copies, "
                         "replayed between one HIP event pair (Gaussian input; both inputs run the "
                         "same kernels)" % reps,
        "cpu_baseline": cpu,
        "nmse": nmse,
        "quantizer_variants": search,
        "cfg1_mxfp4_131072_fp32": cfg1,
        "cfg3_fused_activation_8192x4096": cfg3,
        "gemm": gemm,
    }
    print(json.dumps(line), flush=True)


def only_gemm(args, torch, fp4, workloads, dev):
    """A few calls of each listed GEMM (a short program for profiler runs):
    seeded operands as in the GEMM section (Gaussian weights, Laplace
    activations with outlier channels, the block Hadamard of the format,
    GEMM-layout scales, weights in the tiled code layout, four weight copies
    used in turn as in the GEMM section, so that decode streams its weights
    from HBM rather than the last-level cache), bf16 output, `--gemm-iters`
    timed calls each."""
    fmts = {"mx": fp4.FMT_MXFP4, "nv": fp4.FMT_NVFP4, "mxint4": fp4.FMT_MXINT4,
            "nvint4": fp4.FMT_NVINT4, "w4mx": fp4.FMT_MXFP4, "w4nv": fp4.FMT_NVFP4}
    res = {}
    for item in args.only_gemm.split(","):
        name, shape = item.split(":")
        M, N, K = (int(v) for v in shape.split("x"))
        fmt = fmts[name]
        w = torch.from_numpy(workloads.gemm_weight(N, K, seed=1).view(np.int16)).to(dev).view(torch.bfloat16)
        a = torch.from_numpy(workloads.gemm_activation(M, K, seed=1).view(np.int16)).to(dev).view(torch.bfloat16)
        q0 = fp4.quantize(w, fmt, rotate=True, scale_layout=fp4.SCALES_GEMM, code_layout=fp4.CODES_TILED)
        qw = [q0] + [fp4.Quantized(q0.codes.clone(), q0.scales.clone(), q0.global_scale.clone(),
                                   q0.cfg, q0.rows, q0.cols) for _ in range(3)]
        y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        if name.startswith("w4"):
            wsb = fp4.fp4_gemm_w4a16_workspace_bytes(fmt, M, N, K)
            ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev)

            def call(i):
                fp4.gemm_w4a16(a, qw[i % 4], out=y, workspace=ws if wsb else None)
        else:
            qa = fp4.quantize(a, fmt, rotate=True, scale_layout=fp4.SCALES_GEMM)
            wsb = fp4.fp4_gemm_workspace_bytes(fmt, M, N, K)
            ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev)

            def call(i):
                fp4.gemm(qa, qw[i % 4], out=y, workspace=ws if wsb else None)
        call(3)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(max(1, args.gemm_iters)):
            call(i)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / max(1, args.gemm_iters)
        res[item] = {"us_per_call": round(us, 2), "tflops": round(2.0 * M * N * K / us / 1e6, 1)}
        log("%s %.2f us" % (item, us))
        del w, a, q0, qw, y
    print(json.dumps({"only_gemm": res}), flush=True)


def vendor_mxfp4(torch, fp4, dev):
    """This library's MXFP4 GEMM beside hipBLASLt's (torch._scaled_mm with
    float4_e2m1fn_x2 operands and float8_e8m0fnu scales), bf16 output, on the
    same random E2M1 codes with every E8M0 scale 2^0, alternating three times
    (ten calls each, best run).  Context for the MFMA fraction, not a bench
    value; the two outputs are compared entry by entry (within bf16
    rounding of each other)."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    cfg = fp4.qconfig(fp4.FMT_MXFP4, False, fp4.SCALES_GEMM)

    def operand(rows, K):
        c = torch.randint(0, 256, (rows, K // 2), dtype=torch.uint8, device=dev, generator=gen)
        sc = torch.full((fp4.fp4_scales_bytes(cfg, rows, K),), 127, dtype=torch.uint8, device=dev)
        return c, fp4.Quantized(c.reshape(-1), sc, torch.ones(1, device=dev), cfg, rows, K)

    def best_us(f, n=10):
        f()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    res = {}
    for (M, N, K) in ((4096, 4096, 4096), (4096, 14336, 4096), (4096, 4096, 14336),
                      (8192, 28672, 8192), (8192, 8192, 28672)):
        key = "%dx%dx%d" % (M, N, K)
        ca, qa = operand(M, K)
        cb, qb = operand(N, K)
        y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        sa = torch.full((M, K // 32), 127, dtype=torch.uint8, device=dev).view(torch.float8_e8m0fnu)
        sb = torch.full((N, K // 32), 127, dtype=torch.uint8, device=dev).view(torch.float8_e8m0fnu)
        a4, b4 = ca.view(torch.float4_e2m1fn_x2), cb.view(torch.float4_e2m1fn_x2)

        def ours():
            fp4.gemm(qa, qb, out=y)

        def vendor():
            return torch._scaled_mm(a4, b4.t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16)
        flops = 2.0 * M * N * K
        try:
            yv = vendor()
            ours()
            torch.cuda.synchronize()
            agree = bool(((yv.float() - y.float()).abs() <= 2.0 ** -7 * y.float().abs() + 1e-6).all())
            to, tv = [], []
            for _ in range(3):
                to.append(best_us(ours))
                tv.append(best_us(vendor))
            res[key] = {"ours_us": round(min(to), 1), "ours_frac_fp4_peak": round(flops / min(to) / 1e9 / 10.1, 3),
                        "hipblaslt_us": round(min(tv), 1),
                        "hipblaslt_frac_fp4_peak": round(flops / min(tv) / 1e9 / 10.1, 3),
                        "outputs_agree": agree}
        except RuntimeError as e:  # the library call rejected the shape
            res[key] = {"hipblaslt": "not available: " + str(e)[:160]}
        log("%s %s" % (key, res[key]))
        del ca, qa, cb, qb, y, sa, sb, a4, b4
        torch.cuda.empty_cache()
    print(json.dumps({"vendor_mxfp4": res}), flush=True)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(variants, host, alg_bytes, workloads, fp4):
    """The plain-C oracle on one complete step: single-threaded, and split
    over row chunks on every host core (a thread pool; the oracle's ctypes
    calls release the interpreter lock).  NV variants that compute their
    tensor scale do it as two parallel phases, the oracle's tensor scale of
    each chunk (whose maximum is the tensor's) and then the chunks' encoding
    with that scale; rotated NV variants therefore rotate twice."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    xs = {d: workloads.bf16_bits_to_f32(h) for d, h in host.items()}
    t1 = 0.0
    nbytes = 0
    for (d, fmt, rot) in variants:
        t = time.perf_counter()
        oracle.quantize(xs[d], fmt, rotate=rot)
        t1 += time.perf_counter() - t
        nbytes += alg_bytes(fmt)
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count() or 1
    ncpu = max(1, min(ncpu, 16))
    rows = next(iter(xs.values())).shape[0]
    chunk = max(1, (rows + 4 * ncpu - 1) // (4 * ncpu))
    spans = [(r, min(rows, r + chunk)) for r in range(0, rows, chunk)]
    with ThreadPoolExecutor(max_workers=ncpu) as ex:
        t = time.perf_counter()
        for (d, fmt, rot) in variants:
            x = xs[d]
            ts = None
            if fmt not in fp4.MX_FORMATS:
                parts = ex.map(lambda sp: oracle.tensor_scale(x[sp[0]:sp[1]], fmt, rotate=rot), spans)
                ts = max(parts)
            list(ex.map(lambda sp: oracle.quantize(x[sp[0]:sp[1]], fmt, rotate=rot, ts=ts), spans))
        tp = time.perf_counter() - t
    return {"value": round(nbytes / tp / 1e9, 4), "unit": "GB/s", "cores": ncpu, "kind": "oracle",
            "sample": "one complete step: all 4096 rows of each of the 8 variants (the same "
                      "algorithmic bytes as the GPU line), the plain-C oracle split over %d row "
                      "chunks on %d threads; value_1core: the same step single-threaded" % (
                          len(spans), ncpu),
            "seconds": round(tp, 2), "value_1core": round(nbytes / t1 / 1e9, 4),
            "seconds_1core": round(t1, 2), "nproc": os.cpu_count(), "cpu_model": cpu_model()}


def time_graph(torch, stream, capture, fn, reps):
    """Average us per call of fn(i): reps calls recorded as one HIP graph and
    replayed between two HIP events on the launching stream."""
    fn(0)
    torch.cuda.synchronize()
    g = capture(lambda: [fn(i) for i in range(reps)])
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e3 / reps


def bench_cfg1(torch, fp4, workloads, stream, sh_now, capture, no_oracle):
    """MXFP4 quantize -> dequantize -> error sums of the fp32 [1, 131072]
    tensor (Laplace(0,1), 1 % of entries x50): microseconds per launch and the
    NMSE from the GPU's error sums beside the oracle's."""
    x = workloads.cfg1_tensor(0)
    xd = torch.from_numpy(x).to("cuda")
    q = fp4.quantize(xd, fp4.FMT_MXFP4)
    y = torch.empty_like(xd)
    rows, cols = x.shape
    ewsb = fp4.fp4_error_workspace_bytes(q.cfg, rows, cols)
    ews = torch.empty(max(ewsb, 64), dtype=torch.uint8, device="cuda")
    sums = torch.empty(4, dtype=torch.float64, device="cuda")

    def qf(i=0):
        rc = fp4.fp4_quantize(q.cfg, xd.data_ptr(), fp4.DT_F32, rows, cols, cols, q.codes.data_ptr(),
                              q.scales.data_ptr(), None, fp4.GS_COMPUTE, None, 0, sh_now())
        assert rc == 0

    def df(i=0):
        rc = fp4.fp4_dequantize(q.cfg, q.codes.data_ptr(), q.scales.data_ptr(), None, rows, cols,
                                y.data_ptr(), fp4.DT_F32, cols, 0, sh_now())
        assert rc == 0

    def ef(i=0):
        rc = fp4.fp4_error_sums(q.cfg, xd.data_ptr(), fp4.DT_F32, rows, cols, cols, q.codes.data_ptr(),
                                q.scales.data_ptr(), None, sums.data_ptr(), ews.data_ptr(), ewsb,
                                sh_now())
        assert rc == 0

    def allf(i=0):
        qf(); df(); ef()

    out = {"quantize_us": round(time_graph(torch, stream, capture, qf, 50), 3),
           "dequantize_us": round(time_graph(torch, stream, capture, df, 50), 3),
           "error_sums_us": round(time_graph(torch, stream, capture, ef, 50), 3),
           "all_three_us": round(time_graph(torch, stream, capture, allf, 50), 3)}
    allf()
    torch.cuda.synchronize()
    s = sums.cpu().numpy()
    out["nmse_gpu"] = float(s[0] / s[1])
    if not no_oracle:
        import oracle
        c, sc, _ = oracle.quantize(x, fp4.FMT_MXFP4)
        out["nmse_oracle"] = oracle.nmse(x, oracle.dequantize(c, sc, fp4.FMT_MXFP4))
        out["codes_equal_oracle"] = bool(np.array_equal(fp4.codes_view(q).cpu().numpy(), c))
    out["bytes_note"] = ("alg bytes: read 4 B/elem fp32, codes 0.5 B/elem, scales 1/32 B/elem; "
                         "launch-latency bound at this size (0.59 MB), reported in us")
    return out


def bench_cfg3(torch, fp4, workloads, dev, stream, sh_now, capture):
    """The fused activation path on 8192x4096 bf16 (Laplace(0,1), 8 of 4096
    channels x50): block-Hadamard(32) + MXFP4 with GEMM-layout scales, and
    the NVFP4 + Hadamard(16) variant with its tensor scale computed (one
    launch, and the two passes).  Six input copies rotate so that the
    256 MB last-level cache serves no repeat."""
    rows, cols = 8192, 4096
    n = rows * cols
    base = torch.from_numpy(workloads.cfg3_tensor(0).view(np.int16)).to(dev).view(torch.bfloat16)
    ncopy = 6
    xs = [base] + [base.clone() for _ in range(ncopy - 1)]
    res = {}
    wsb = 8192
    ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
    for name, fmt, lay, mode in (("mxfp4_h32_gemm_layout", fp4.FMT_MXFP4, fp4.SCALES_GEMM, None),
                                 ("nvfp4_h16_one_pass", fp4.FMT_NVFP4, fp4.SCALES_ROWMAJOR,
                                  fp4.GS_COMPUTE_ONE_PASS),
                                 ("nvfp4_h16_two_pass", fp4.FMT_NVFP4, fp4.SCALES_ROWMAJOR,
                                  fp4.GS_COMPUTE)):
        cfg = fp4.qconfig(fmt, True, lay)
        outs = [fp4.quantize(xs[0], fmt, rotate=True, scale_layout=lay) for _ in range(ncopy)]

        def f(i, outs=outs, cfg=cfg, fmt=fmt, mode=mode):
            q = outs[i % ncopy]
            rc = fp4.fp4_quantize(cfg, xs[i % ncopy].data_ptr(), fp4.DT_BF16, rows, cols, cols,
                                  q.codes.data_ptr(), q.scales.data_ptr(),
                                  q.global_scale.data_ptr(), mode if mode is not None else 0,
                                  ws.data_ptr(), wsb, sh_now())
            assert rc == 0

        us = time_graph(torch, stream, capture, f, 4 * ncopy)
        G = fp4.BLOCK[fmt]
        nbytes = n * 2 + n // 2 + n // G
        ent = {"avg_us": round(us, 3), "alg_bytes": nbytes,
               "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
               "frac": round(nbytes / (us * 1e-6) / PEAK_HBM, 4)}
        if mode == fp4.GS_COMPUTE:
            ent["note"] = "two launches (maximum pass, encode); alg_bytes count the input once"
        res[name] = ent
        del outs
    return {"kernels": res, "shape": [rows, cols],
            "note": "per call: a HIP graph of back-to-back calls over 6 rotating input copies, "
                    "between one HIP event pair; bytes = bf16 read once + codes + scales"}


def bench_gemm(args, torch, fp4, workloads, dev, stream):
    res = {"weight_code_layout": "tiled: 8 KB tiles of 128 rows x 128 elements"}
    iters = max(1, args.gemm_iters)

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    def time_it(fn, reps, graph=True):
        """Average us per call: reps calls recorded as one HIP graph and replayed
        between two HIP events (graph=False: launched eagerly from Python)."""
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        if graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(reps):
                    fn(i)
            g.replay()
            torch.cuda.synchronize()
            e0.record(stream)
            g.replay()
            e1.record(stream)
        else:
            e0.record(stream)
            for i in range(reps):
                fn(i)
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps  # us

    def quant_copies(x_bf16, fmt, rot, ncopy):
        # weights: tiled codes (whole 8 KB blocks per GEMM stage)
        q0 = fp4.quantize(x_bf16, fmt, rotate=rot, scale_layout=fp4.SCALES_GEMM,
                          code_layout=fp4.CODES_TILED)
        out = [q0]
        for _ in range(ncopy - 1):
            out.append(fp4.Quantized(q0.codes.clone(), q0.scales.clone(), q0.global_scale.clone(),
                                     q0.cfg, q0.rows, q0.cols))
        return out

    # Llama-3-8B linears at M = 4096 (MXFP4, H32), plus the bf16 reference
    M = 4096
    for (K, N) in [(4096, 4096), (4096, 6144), (4096, 14336), (14336, 4096)]:
        t0 = time.time()
        w = to_dev(workloads.gemm_weight(N, K, seed=0))
        a = to_dev(workloads.gemm_activation(M, K, seed=0))
        qw = quant_copies(w, fp4.FMT_MXFP4, True, 2)
        qa = fp4.quantize(a, fp4.FMT_MXFP4, rotate=True, scale_layout=fp4.SCALES_GEMM)
        y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        wsb = fp4.fp4_gemm_workspace_bytes(fp4.FMT_MXFP4, M, N, K)
        gw = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev)

        def g(i=0):
            fp4.gemm(qa, qw[i % 2], out=y, workspace=gw if wsb else None)

        def qfn(i=0):
            fp4.quantize(a, fp4.FMT_MXFP4, rotate=True, scale_layout=fp4.SCALES_GEMM, out=qa)

        def layer(i=0):
            qfn()
            g(i)

        wt = w.t().contiguous()

        def bf(i=0):
            torch.mm(a, wt, out=y)

        us_g = time_it(g, iters)
        us_q = time_it(qfn, iters)
        us_l = time_it(layer, iters)
        us_b = time_it(bf, iters, graph=False)
        fl = 2.0 * M * N * K
        res["llama8b_M%d_K%d_N%d" % (M, K, N)] = {
            "fmt": "mxfp4+h32", "gemm_us": round(us_g, 2), "tflops": round(fl / us_g / 1e6, 1),
            "frac_fp4_peak": round(fl / (us_g * 1e-6) / PEAK_FP4, 4),
            "act_quant_us": round(us_q, 2), "layer_us": round(us_l, 2),
            "bf16_torch_us": round(us_b, 2), "layer_speedup_vs_bf16": round(us_b / us_l, 2)}
        del w, a, qw, qa, y, wt
        log("gemm 8b K%d N%d %.1f us (%.0fs)" % (K, N, us_g, time.time() - t0))

    # Llama-3-70B MLP linears on one GPU, MXFP4 (H32) and NVFP4 (H16)
    for (K, N) in [(8192, 28672), (28672, 8192)]:
        t0 = time.time()
        w = to_dev(workloads.gemm_weight(N, K, seed=1))
        wt = w.t().contiguous()
        amax = to_dev(workloads.gemm_activation(8192, K, seed=1, outlier_frac=0.001))
        for fmt in (fp4.FMT_MXFP4, fp4.FMT_NVFP4, fp4.FMT_MXINT4, fp4.FMT_NVINT4):
            fname = {fp4.FMT_MXFP4: "mxfp4+h32", fp4.FMT_NVFP4: "nvfp4+h16",
                     fp4.FMT_MXINT4: "mxint4+h32", fp4.FMT_NVINT4: "nvint4+h16"}[fmt]
            qw = quant_copies(w, fmt, True, 4)
            wbytes = qw[0].codes.numel() + qw[0].scales.numel()
            for Mm in ((1, 16, 128, 8192) if fmt in (fp4.FMT_MXFP4, fp4.FMT_NVFP4) else (1, 8192)):
                a = amax[:Mm]
                qa = fp4.quantize(a, fmt, rotate=True, scale_layout=fp4.SCALES_GEMM)
                y = torch.empty(Mm, N, dtype=torch.bfloat16, device=dev)
                wsb = fp4.fp4_gemm_workspace_bytes(fmt, Mm, N, K)
                gw = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev)

                def g(i=0):
                    fp4.gemm(qa, qw[i % 4], out=y, workspace=gw if wsb else None)

                def layer(i=0):
                    fp4.quantize(a, fmt, rotate=True, scale_layout=fp4.SCALES_GEMM, out=qa)
                    g(i)

                def bf(i=0):
                    torch.mm(a, wt, out=y)

                us_g = time_it(g, iters)
                us_l = time_it(layer, iters)
                us_b = time_it(bf, iters, graph=False) if fmt == fp4.FMT_MXFP4 else None
                fl = 2.0 * Mm * N * K
                peak = PEAK_FP4 if fmt == fp4.FMT_MXFP4 else PEAK_F16  # INT4: bf16 / fp16 MFMA
                traffic = wbytes + qa.codes.numel() + qa.scales.numel() + Mm * N * 2
                ent = {"fmt": fname, "gemm_us": round(us_g, 2),
                       "tflops": round(fl / us_g / 1e6, 2),
                       "frac_mfma_peak": round(fl / (us_g * 1e-6) / peak, 4),
                       "alg_gbs": round(traffic / us_g / 1e3, 1),
                       "frac_hbm": round(traffic / (us_g * 1e-6) / PEAK_HBM, 4),
                       "layer_us": round(us_l, 2)}
                if us_b is not None:
                    ent["bf16_torch_us"] = round(us_b, 2)
                    ent["layer_speedup_vs_bf16"] = round(us_b / us_l, 2)
                if Mm <= 128:
                    # weight-only product: bf16 activations, the same FP4 weights
                    w4b = fp4.fp4_gemm_w4a16_workspace_bytes(fmt, Mm, N, K)
                    w4w = torch.zeros(max(w4b, 16), dtype=torch.uint8, device=dev)

                    def w4(i=0):
                        fp4.gemm_w4a16(a, qw[i % 4], out=y, workspace=w4w if w4b else None)

                    us_w4 = time_it(w4, iters)
                    t_w4 = wbytes + Mm * K * 2 + Mm * N * 2
                    ent["w4a16_us"] = round(us_w4, 2)
                    ent["w4a16_frac_hbm"] = round(t_w4 / (us_w4 * 1e-6) / PEAK_HBM, 4)
                    ent["w4a16_frac_bf16_peak"] = round(fl / (us_w4 * 1e-6) / PEAK_F16, 4)
                res["llama70b_%s_M%d_K%d_N%d" % (fname.split("+")[0], Mm, K, N)] = ent
                log("gemm 70b %s M%d K%d N%d %.1f us" % (fname, Mm, K, N, us_g))
            del qw
        del w, wt, amax
        log("70b shape done (%.0fs)" % (time.time() - t0))
    return res


if __name__ == "__main__":
    main()

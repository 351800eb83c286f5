#!/usr/bin/env python3
"""Benchmark of the fused MXFP8 grouped-matmul + finalize-routing operator.

One step = one full call of the operator (grouped block-scaled FP8 matmul,
logit weighting, scatter-add into out, shared-expert axpy) over the headline
workload (M=768 routed tokens, K=8192, N=4096, E=32 experts of 24 tokens,
batch 256), inputs resident in HBM.  Prints ONE JSON line.

value      = effective TFLOP/s = 2*M*K*N / (time per step)
roofline   = the fused kernel against the HBM roofline (its algorithmic bytes
             per launch / its mean launch time, timed with events on the launch
             stream), the binding roof for every configuration here
             (mean, median and minimum of the per-launch event times are
             reported; frac_per_step is the same bytes over the whole-run
             time per step, launch gaps included)
cpu_baseline = the CPU oracle on a bounded sample of output rows of the same
             workload (plain C in double precision, output rows spread over
             the host's OpenMP threads; cores = threads used, host_cores =
             os.cpu_count())

``--workload g1_*`` measures the upstream step of the FFN instead
(gfr_gemm1_swiglu_quant: gate||up grouped matmul, SwiGLU, MX quantisation;
default g1_c3, the step that produces c3's x1): value = 2*M*H*2I / t, the
same roofline and CPU-oracle legs.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MXFP8_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
MXFP4_PEAK_TFLOPS = 10100.0  # MI355X dense FP4 MFMA
INT8_PEAK_TOPS = 5000.0      # MI355X dense INT8 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c3",
                    help="a finalize-routing workload (c1..c5, ...) or an upstream-step one (g1_*)")
    ap.add_argument("--deterministic", action="store_true")
    ap.add_argument("--split-k", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="instead of the operator, run a plain 1 GiB device-to-device copy per "
                         "step (the known-size reference for HBM byte counters)")
    return ap.parse_args()


def copy_calibration(args):
    """Plain copy of a known size: each step reads and writes exactly 1 GiB."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(7)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    print(json.dumps({"calibration": "copy", "bytes_read": n, "bytes_written": n,
                      "steps": args.steps, "ms_per_copy": round(ms, 5),
                      "GBps_read_plus_write": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


def cpu_baseline(w, inp, budget_s):
    """Time the oracle on a growing seeded sample of output rows."""
    import numpy as np
    import torch
    import oracle
    from mxfp8_grouped_gemm_group_amd.workloads import as_numpy

    if w.fp8 == "w4a8":
        c = lambda t: None if t is None else t.cpu().numpy()
        sh = inp["shared_input"]
        sh = None if sh is None else sh.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        args = (c(inp["x1"]), c(inp["x2"]), c(inp["scale"]), c(inp["offset"]),
                c(inp["pertoken_scale"]), c(inp["group_list"]), inp["group_list_type"],
                c(inp["logit"]), c(inp["row_index"]), sh, inp["shared_input_weight"],
                inp["shared_input_offset"], c(inp["out"]))
        run = lambda rows: oracle.w4a8_finalize_routing(*args, rows=rows)
        ri = args[8]
    else:
        h = as_numpy(inp)
        run = lambda rows: oracle.gmm_finalize_routing(
            h["x1"], h["x2"], h["scale"], h["pertoken_scale"], h["group_list"],
            h["group_list_type"], h["logit"], h["row_index"], h["shared_input"],
            h["shared_input_weight"], h["shared_input_offset"], h["out_init"],
            h["transpose_x2"], h["fp8_kind"], rows=rows)
        ri = h["row_index"]
    total_tokens = int(w.counts().sum())
    routed = ri[:total_tokens]
    rng = np.random.default_rng(12345)
    order = rng.permutation(w.batch)
    threads = oracle.num_threads()
    n, spent, rows_done, tok_done = threads, 0.0, 0, 0
    while True:
        rows = order[rows_done:rows_done + n]
        if rows.size == 0:
            break
        t0 = time.perf_counter()
        run(rows)
        spent += time.perf_counter() - t0
        rows_done += rows.size
        tok_done += int(np.isin(routed, rows).sum())
        if spent >= budget_s:
            break
        n = max(threads, int(rows_done * (budget_s - spent) / max(spent, 1e-9) / 2)) if spent > 0.5 else n * 2
    flops = 2.0 * tok_done * w.K * w.N
    return {"value": flops / spent / 1e12, "unit": "TOP/s" if w.fp8 == "w4a8" else "TFLOP/s",
            "cores": threads, "host_cores": os.cpu_count(), "kind": "oracle",
            "sample": f"{rows_done} of {w.batch} output rows ({tok_done} routed tokens, all "
                      f"{w.N} columns) of workload {w.name}; {spent:.1f} s on {threads} threads "
                      "(one output row per thread at a time)"}


def time_steps(step, args, dev):
    """Warm up, then time exactly args.steps back-to-back calls between two
    events on the launch stream (synchronised on both sides): ms_per_step.
    Then a second pass of args.steps calls with an event pair around each
    launch gives the per-launch times (ms) for the roofline.  The event
    pairs are kept out of the first pass: on the GPU they cost about 7 µs a
    step (c1 44.3 -> 51.7 µs a step), which is measurement, not work.
    Returns (ms_per_step, per-launch times in ms)."""
    import torch
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per_launch_ms = [a.elapsed_time(b) for a, b in ev]
    return ms_per_step, per_launch_ms


def launch_stats(per_launch_ms):
    """Mean, median and minimum of the per-launch event times (ms)."""
    v = sorted(per_launch_ms)
    n = len(v)
    med = v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])
    return {"mean_launch_ms": round(sum(v) / n, 5), "median_launch_ms": round(med, 5),
            "min_launch_ms": round(v[0], 5)}


def gemm1_cpu_baseline(w, inp, budget_s):
    """Time the upstream-step oracle on a growing seeded sample of tokens."""
    import numpy as np
    import torch
    import oracle
    from oracle import gemm1 as og
    threads = oracle.num_threads()
    u8 = lambda x: x.detach().contiguous().view(torch.uint8).cpu().numpy()
    h = [u8(inp["xin"]), u8(inp["w13"]), u8(inp["scale"]), u8(inp["xin_scale"]),
         inp["group_list"].cpu().numpy()]
    kind = 0 if w.fp8 == "e4m3fn" else 1
    okind = 0 if w.out_fp8 == "e4m3fn" else 1
    routed = np.flatnonzero(og.routed_tokens(h[4], w.group_list_type, w.M))
    order = np.random.default_rng(12345).permutation(routed)
    n, spent, done = threads, 0.0, 0
    while done < order.size:
        rows = order[done:done + n]
        t0 = time.perf_counter()
        og.gemm1_swiglu_quant(*h, w.group_list_type, w.transpose_w13, kind, okind, rows=rows)
        spent += time.perf_counter() - t0
        done += rows.size
        if spent >= budget_s:
            break
        n = max(threads, int(done * (budget_s - spent) / max(spent, 1e-9) / 2)) if spent > 0.5 else n * 2
    flops = 2.0 * done * w.H * 2 * w.I
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": threads,
            "host_cores": os.cpu_count(), "kind": "oracle",
            "sample": f"{done} of {routed.size} routed tokens (all {w.I} outputs) of workload "
                      f"{w.name}; {spent:.1f} s on {threads} threads (the gate||up matmul "
                      "one token row per thread at a time; SwiGLU and quantisation in numpy)"}


def gemm1_main(args, w):
    import torch
    import mxfp8_grouped_gemm_group_amd as gfr
    from mxfp8_grouped_gemm_group_amd import traffic as traffic_mod
    from mxfp8_grouped_gemm_group_amd.workloads import make_gemm1_inputs

    gfr.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_gemm1_inputs(w, dev)
    wb = inp["w13"].numel()
    n_sets = max(1, -(-(1 << 30) // wb)) if wb < (1 << 29) else 1
    w_sets = [inp["w13"]] + [inp["w13"].clone() for _ in range(n_sets - 1)]
    q = torch.zeros((w.M, w.I), dtype=torch.uint8, device=dev).view(inp["out_dtype"])
    qs = torch.zeros((w.M, w.I // 64, 2), dtype=torch.uint8, device=dev)

    def step(i):
        gfr.gemm1_swiglu_quant(inp["xin"], w_sets[i % n_sets], inp["scale"], inp["xin_scale"],
                               inp["group_list"], inp["group_list_type"], inp["transpose_w13"],
                               inp["out_dtype"], x1_out=q, x1_scale_out=qs)

    ms_per_step, per_launch = time_steps(step, args, dev)
    st = launch_stats(per_launch)
    flops, alg_bytes = w.flops(), w.algorithmic_bytes()
    # average launch duration: the timed back-to-back run's total / steps (one
    # launch per step in atomic mode); it agrees with rocprofv3's kernel-trace
    # average, where an event pair around each launch also times its dispatch
    achieved_gbs = alg_bytes / (ms_per_step * 1e-3) / 1e9
    line = {
        "metric": "effective TFLOP/s (2*M*H*2I/t) + % of binding roofline, upstream gate||up "
                  "step (SwiGLU + MX quantisation)",
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8 (fp8 x fp8 x e8m0 -> f32 -> mx fp8)",
        "data": "synthetic (seeded; FP8 from N(0,1), E8M0 exponents uniform)",
        "config": {
            "workload": f"{w.name}: M={w.M} H={w.H} I={w.I} E={w.E} fp8={w.fp8} "
                        f"out={w.out_fp8} transpose_w13={w.transpose_w13} "
                        f"group_list_type={w.group_list_type}",
            "weight_copies_rotated": n_sets,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic_mod.recorded_traffic(w.name),
            "kernel": "gemm1_swiglu_kernel (gfr gate||up grouped MXFP8 GEMM + SwiGLU + MX quant)",
            "algorithmic_bytes_per_launch": alg_bytes,
            **st,
            "launch_timing": "achieved = bytes / (timed back-to-back run / steps); "
                             "mean/median/min_launch_ms: an event pair around each launch "
                             "(including its dispatch), in a second pass after the timed one",
            "mfma_frac": round(flops / (ms_per_step * 1e-3) / 1e12 / MXFP8_PEAK_TFLOPS, 4),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = gemm1_cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this operator is "
              "built and measured on a single MI355X", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args)
        return
    import torch
    import mxfp8_grouped_gemm_group_amd as gfr
    from mxfp8_grouped_gemm_group_amd import traffic as traffic_mod
    from mxfp8_grouped_gemm_group_amd.workloads import (GEMM1_WORKLOADS, WORKLOADS, make_inputs,
                                                        make_w4a8_inputs)

    if args.workload in GEMM1_WORKLOADS:
        gemm1_main(args, GEMM1_WORKLOADS[args.workload])
        return
    gfr.load_library()
    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w4a8 = w.fp8 == "w4a8"
    inp = make_w4a8_inputs(w, dev) if w4a8 else make_inputs(w, dev)
    # Rotate weight copies so the 256 MB last-level cache never holds the
    # next step's weights (cold HBM every step).
    x2_bytes = inp["x2"].numel()
    n_sets = max(1, -(-(1 << 30) // x2_bytes)) if x2_bytes < (1 << 29) else 1
    x2_sets = [inp["x2"]] + [inp["x2"].clone() for _ in range(n_sets - 1)]
    out = inp["out"].clone()
    ws = None
    if args.deterministic:
        ws = torch.empty(max(1, gfr.workspace_size(w.M, w.K, w.N, w.E, w.batch, True)),
                         dtype=torch.uint8, device=dev)

    def step(i):
        if w4a8:
            gfr.w4a8_finalize_routing(
                inp["x1"], x2_sets[i % n_sets], inp["scale"], inp["offset"],
                inp["pertoken_scale"], inp["group_list"], inp["group_list_type"], inp["logit"],
                inp["row_index"], inp["shared_input"], inp["shared_input_weight"],
                inp["shared_input_offset"], out, deterministic=args.deterministic,
                workspace=ws, split_k=args.split_k)
            return
        gfr.gmm_finalize_routing(
            inp["x1"], x2_sets[i % n_sets], inp["scale"], inp["pertoken_scale"],
            inp["group_list"], inp["group_list_type"], inp["logit"], inp["row_index"],
            inp["shared_input"], inp["shared_input_weight"], inp["shared_input_offset"], out,
            inp["transpose_x2"], deterministic=args.deterministic, workspace=ws,
            split_k=args.split_k)

    ms_per_step, per_launch = time_steps(step, args, dev)
    st = launch_stats(per_launch)

    flops = w.flops()
    alg_bytes = w.algorithmic_bytes()
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    # average launch duration: the timed back-to-back run's total / steps (one
    # launch per step in atomic mode); it agrees with rocprofv3's kernel-trace
    # average, where an event pair around each launch also times its dispatch
    achieved_gbs = alg_bytes / (ms_per_step * 1e-3) / 1e9
    # HBM bytes per launch from rocprofv3 counters of this very kernel source
    # (null when the kernel changed after the counters were taken)
    traffic = None
    if not args.deterministic and args.split_k == 0:
        traffic = traffic_mod.recorded_traffic(w.name)

    line = {
        "metric": "effective TFLOP/s (2*M*K*N/t) + % of binding roofline, M=768 K=8192 N=4096 E=32",
        "value": round(tflops, 2),
        "unit": "TOP/s" if w4a8 else "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("w4a8 (int8 x int4 -> i32, f32 scales)" if w4a8
                  else "mxfp4 (e2m1 x e2m1 x e8m0 -> f32)" if w.fp8 == "e2m1"
                  else "mxfp8 (fp8 x fp8 x e8m0 -> f32)"),
        "data": ("synthetic (seeded; int8 and int4 uniform, FP32 scales uniform)" if w4a8 else
                 f"synthetic (seeded; {'E2M1' if w.fp8 == 'e2m1' else 'FP8'} from N(0,1), "
                 "E8M0 exponents uniform)"),
        "config": {
            "workload": f"{w.name}: M={w.M} K={w.K} N={w.N} E={w.E} batch={w.batch} "
                        f"fp8={w.fp8} transpose_x2={w.transpose_x2} "
                        f"group_list_type={w.group_list_type} shared_rows={w.R}",
            "mode": "deterministic" if args.deterministic else "atomic",
            "split_k": args.split_k,
            "weight_copies_rotated": n_sets,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "fused_kernel (gfr grouped MXFP8 GEMM + finalize routing)",
            "algorithmic_bytes_per_launch": alg_bytes,
            **st,
            "launch_timing": "achieved = bytes / (timed back-to-back run / steps); "
                             "mean/median/min_launch_ms: an event pair around each launch "
                             "(including its dispatch), in a second pass after the timed one",
            "mfma_frac": round(flops / (ms_per_step * 1e-3) / 1e12 /
                               (MXFP4_PEAK_TFLOPS if w.fp8 == "e2m1" else
                                INT8_PEAK_TOPS if w4a8 else MXFP8_PEAK_TFLOPS), 4),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

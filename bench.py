#!/usr/bin/env python3
"""Benchmark of the block-scale quantiser hot path on one MI355X.

Workload (one "step"): the INT8 / E4M3-scale case on the qwantize "Results"
page's layer shape -- W 2560 x 9728 bf16 (a seeded Student-t(4) x 0.02 stand-in
with per-row lognormal gain for the down_proj weight) and calibration X
16384 x 9728 bf16 (N(0,1), 8 outlier channels x 50):
    hdiag(X), output_gram(X) (G = X^T X, stored as float16 correlations) and
    output_reference_gram (||X W^T||^2 from G), then for B in
    {32, 64, 128, 256} and each of Naive, SSE-Optimal, H-Optimal:
    quantize_blocks (scale choice + encode), dequantize, weight error and
    output error (output_error_gram_batch after the loop: sum_n d_n^T G d_n
    for D = Wq - W of all 12 quantisations, one MFMA walk of 12 N x K x K over
    G's upper block triangle).
    --output-route direct measures the output error with X instead:
    output_reference (Y = X W^T) once and output_error_codes (X Wq^T - Y, one
    M x N x K MFMA product) per quantisation.
value = 12 quantisations x 2560 x 9728 weights / step time, in Gweights/s.
Inputs are resident in HBM before timing starts.  The step is timed twice:
as individual launches (per-call GPU times from HIP events recorded on the
stream the kernels run on: the per-stage figures and the roofline) and as
replays of the same step captured once in a HIP graph (no host launch gaps;
a replay must first reproduce the eager step's errors bit for bit), which
gives ms_per_step and value unless --eager is given.

Prints one JSON line (the metric, per-stage figures, the roofline of the
dominant kernel and the CPU oracle timed on a bounded sample).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Gweights/s for SSE/H-Optimal block-scale search; % of VALU & HBM peak"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
# 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz: VALU lane-operations per second
# without packed FP32 (the kernels are compiled without packed FP32 instructions).
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# counting convention for the search: VALU lane-ops per (weight, candidate)
SEARCH_OPS = {"sse": 6, "h": 7}


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "int8_down_proj_2560x9728_hbm_traffic.md")
COUNTERS_PROFILE = os.path.join(ROOT, "profiles", "int8_down_proj_2560x9728_counters.md")


# sources whose kernels the INT8 step never launches (other formats' searches,
# the FP16-scale alternation, GPTQ, per-tensor scaling), and the host-only C
# ABI wrapper and launcher declarations (no device code)
_NOT_IN_STEP = {"alt_f16.hip", "gptq.hip", "tscale.hip", "search_fp8s.hip", "search_mxfp4.hip", "search_mxfp8.hip",
                "search_nvfp4.hip", "search_nvfp4_ue4m4.hip", "search_nvfp4_ue5m3.hip", "search_nvint4.hip",
                "abi.cpp", "kernels.hpp"}


def source_hash():
    """Hash of the HIP sources the step's kernels are built from (every file of
    csrc/ but those listed above); counter-derived traffic is valid only for
    the kernels it was measured on."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "block_scaled_precision_hdiag_amd", "csrc", "*"))):
        if os.path.basename(f) in _NOT_IN_STEP:
            continue
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _profile_record(path, tag):
    """Per-stage figures from a committed rocprofv3 --pmc record, or {} if the
    kernels changed since it was taken."""
    try:
        with open(path) as f:
            for line in f:
                if line.startswith(tag + ":"):
                    rec = json.loads(line.split(":", 1)[1])
                    return rec["stages"] if rec.get("source_hash") == source_hash() else {}
    except OSError:
        pass
    return {}


def measured_traffic():
    """Per-stage HBM bytes (FETCH_SIZE / WRITE_SIZE, calibrated)."""
    return _profile_record(TRAFFIC_PROFILE, "traffic-json")


def measured_counters():
    """Per-stage executed VALU instructions and MFMA-busy cycles."""
    return _profile_record(COUNTERS_PROFILE, "counters-json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=8, help="rows of W in the CPU sample")
    ap.add_argument("--suite", choices=["headline", "formats", "gptq", "sigma", "gemm", "hbm"], default="headline",
                    help="headline: the step above (one JSON line, the default); formats: every element / "
                         "scale format x B in {16, 32} x scale choice on the same W and h (one JSON line)")
    ap.add_argument("--eager", action="store_true",
                    help="time the step as individual launches instead of replays of one captured HIP graph")
    ap.add_argument("--output-route", choices=["gram", "direct"], default="gram",
                    help="output error through G = X^T X (gram) or through X W^T (direct)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="before timing, run one device copy of this many MB (a known-size kernel that "
                         "calibrates HBM byte counters)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the work would shard by rows "
              "of W and X). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_scaled_precision_hdiag_amd as hd
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hd.lib()
    if args.suite == "formats":
        return formats_suite(args, dev)
    if args.suite == "gptq":
        return gptq_suite(args, dev)
    if args.suite == "sigma":
        return sigma_suite(args, dev)
    if args.suite == "gemm":
        return gemm_suite(args, dev)
    if args.suite == "hbm":
        return hbm_suite(args, dev)

    cfg = synth.CONFIGS[2]
    W_cpu, X_cpu = synth.config_inputs(2)
    N, K = W_cpu.shape
    M = X_cpu.shape[0]
    W = W_cpu.to(dev)
    X = X_cpu.to(dev)
    fmt = hd.INT8_E4M3
    blocks = cfg["blocks"]
    methods = [("naive", hd.NAIVE), ("sse", hd.SSE_OPT), ("h", hd.H_OPT)]
    n_cand = hd.hdiag_format_info(fmt, 32)[2]

    # outputs and workspaces, allocated once outside the timed region
    h = torch.empty(K, dtype=torch.float32, device=dev)
    ws_h = torch.empty(hd.hdiag_workspace_size(M, K), dtype=torch.uint8, device=dev)
    ws_w = torch.empty(hd.lib().weight_error_workspace_size(N, K), dtype=torch.uint8, device=dev)
    gram_route = args.output_route == "gram"
    if gram_route:
        gram = torch.empty(hd.output_gram_size(K), dtype=torch.uint8, device=dev)
        ws_g = torch.empty(hd.output_gram_workspace_size(M, K), dtype=torch.uint8, device=dev)
        ws_o = torch.empty(hd.output_error_gram_batch_workspace_size(len(blocks) * len(methods), N, K),
                           dtype=torch.uint8, device=dev)
        ysq = torch.empty(1, dtype=torch.float64, device=dev)
    else:
        ref = torch.empty(hd.output_reference_size(M, N, K), dtype=torch.uint8, device=dev)
        ws_o = torch.empty(hd.output_error_codes_workspace_size(M, N, K), dtype=torch.uint8, device=dev)
    # one code / scale buffer per quantisation (B, method): the Gram route
    # scores all of them together after the loop
    codes = {(B, m): torch.empty((N, K), dtype=torch.uint8, device=dev) for B in blocks for _, m in methods}
    scales = {(B, m): torch.empty((N, K // B), dtype=torch.uint8, device=dev) for B in blocks for _, m in methods}
    Wq = torch.empty((N, K), dtype=torch.float32, device=dev)
    werr = torch.empty((len(blocks), 3), dtype=torch.float64, device=dev)
    oerr = torch.empty((len(blocks), 3), dtype=torch.float64, device=dev)

    if args.copy_probe_mb:
        # a plain device-to-device copy of a known size (hipMemcpyAsync runs it
        # as one copy kernel): reads and writes args.copy_probe_mb MiB
        src = torch.empty(args.copy_probe_mb << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    events = []  # (stage, B, start, end) during timed steps

    def timed(stage, B, fn, rec):
        if rec:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            events.append((stage, B, a, b))
        else:
            fn()

    def step(rec):
        timed("hdiag", 0, lambda: hd.hdiag(X, out=h, workspace=ws_h), rec)
        if gram_route:
            timed("output_gram", 0, lambda: hd.output_gram(X, h=h, gram=gram, workspace=ws_g), rec)
            timed("output_reference", 0, lambda: hd.output_reference_gram(W, gram, workspace=ws_o, out=ysq), rec)
        else:
            timed("output_reference", 0, lambda: hd.output_reference(X, W, ref=ref), rec)
        for bi, B in enumerate(blocks):
            for mi, (mname, m) in enumerate(methods):
                stage = "naive" if m == hd.NAIVE else "search_" + mname
                cb, sb = codes[(B, m)], scales[(B, m)]
                timed(stage, B, lambda: hd.quantize_blocks(m, fmt, B, W, h=h, codes=cb, scales=sb), rec)
                timed("dequantize", B, lambda: hd.dequantize(fmt, B, cb, sb, N, K, out=Wq), rec)
                timed("weight_error", B, lambda: hd.weight_error(W, Wq, workspace=ws_w, out=werr[bi, mi:mi + 1]),
                      rec)
                if not gram_route:
                    timed("output_error", B,
                          lambda: hd.output_error_codes(fmt, B, X, cb, sb, ref, N, K, workspace=ws_o,
                                                        out=oerr[bi, mi:mi + 1]), rec)
        if gram_route:
            # the 12 output errors in one call (one MFMA walk over their stacked operand)
            items = [(fmt, B, codes[(B, m)], scales[(B, m)]) for B in blocks for _, m in methods]
            timed("output_error", 0,
                  lambda: hd.output_error_gram_batch(items, W, gram, ysq, workspace=ws_o, out=oerr.view(-1)), rec)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_eager = (t1 - t0) * 1e3 / args.steps
    ms_per_step, launch = ms_eager, "eager"
    if not args.eager:
        # the same step captured once as a HIP graph (every launch of the step,
        # same buffers) and replayed: a replay must reproduce the eager errors
        # bit for bit before its time is used
        eager_w, eager_o = werr.clone(), oerr.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(False)
        werr.zero_()
        oerr.zero_()
        graph.replay()
        torch.cuda.synchronize()
        if not (torch.equal(werr, eager_w) and torch.equal(oerr, eager_o)):
            raise SystemExit("graph replay does not reproduce the eager step")
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms_per_step, launch = (t1 - t0) * 1e3 / args.steps, "hip_graph"
    value = len(blocks) * len(methods) * N * K / (ms_per_step * 1e-3) / 1e9

    # per-stage GPU times (ms per launch), from the events
    stage_ms = {}
    for stage, B, a, b in events:
        stage_ms.setdefault(stage, []).append(a.elapsed_time(b))
    per_step = {s: sum(v) / args.steps for s, v in stage_ms.items()}
    avg = {s: sum(v) / len(v) for s, v in stage_ms.items()}

    # algorithmic work per launch of each stage
    bytes_w = N * K * 2
    work = {
        "hdiag": ("hbm", M * K * 2 + K * 4),
        "naive": ("hbm", sum(bytes_w + N * K + N * K // B for B in blocks) / len(blocks)),
        "dequantize": ("hbm", sum(N * K + N * K // B + N * K * 4 for B in blocks) / len(blocks)),
        "weight_error": ("hbm", bytes_w + N * K * 4),
        # the gram route: G's K (K + 1) / 2 distinct entries (2 M flops each),
        # and the quadratic forms d^T G d over G's symmetric halves (N K^2)
        "output_gram": ("mfma", 1.0 * M * K * (K + 1)),
        "output_reference": ("mfma", 1.0 * N * K * K if gram_route else 2.0 * M * N * K),
        "output_error": ("mfma", len(blocks) * len(methods) * 1.0 * N * K * K if gram_route else 2.0 * M * N * K),
        "search_sse": ("alu", N * K * n_cand * SEARCH_OPS["sse"]),
        "search_h": ("alu", N * K * n_cand * SEARCH_OPS["h"]),
    }

    counters = measured_counters()

    def roof(stage):
        bound, units = work[stage]
        t = avg[stage] * 1e-3
        if bound == "hbm":
            ach, peak, unit = units / t / 1e9, HBM_PEAK_GBS, "GB/s"
        elif bound == "mfma":
            ach, peak, unit = units / t / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
        else:
            ach, peak, unit = units / t / 1e12, VALU_PEAK_TOPS, "Tops/s"
        r = {"bound": bound, "achieved": round(ach, 3), "peak": round(peak, 3), "unit": unit,
             "frac": round(ach / peak, 4), "avg_ms": round(avg[stage], 4)}
        c = counters.get(stage)
        if bound == "alu":
            # the full-grid count above is a convention (the search evaluates a
            # fraction of the grid); the executed VALU rate comes from counters
            r["basis"] = "full-grid equivalent (%d lane-ops per weight and candidate)" % SEARCH_OPS[stage[7:]]
            if c:
                ex = c["SQ_INSTS_VALU"] * 64 / t / 1e12
                r["executed_valu_tops"] = round(ex, 3)
                r["executed_valu_frac"] = round(ex / VALU_PEAK_TOPS, 4)
        elif bound == "mfma" and c:
            r["mfma_busy_frac"] = round(c["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * t * 2.4e9), 4)
        return r

    stages = {s: roof(s) for s in avg}
    dominant = max(per_step, key=per_step.get)
    roofline = dict(stages[dominant])
    roofline["kernel"] = dominant
    tr = measured_traffic().get(dominant)
    roofline["traffic"] = round(tr["read_bytes"] + tr["write_bytes"]) if tr else None
    roofline["traffic_unit"] = "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated)"
    roofline.pop("avg_ms")

    search_gwps = {s: round(N * K / (avg[s] * 1e-3) / 1e9, 3) for s in avg if s.startswith("search") or s == "naive"}

    errs = {}
    we, oe = werr.cpu().numpy(), oerr.cpu().numpy()
    for bi, B in enumerate(blocks):
        for mi, (mname, _) in enumerate(methods):
            errs["B%d_%s" % (B, mname)] = {"weight_error": round(float(we[bi, mi]), 6),
                                           "output_error": round(float(oe[bi, mi]), 6)}

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "Gweights/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3),
        "launch": launch, "ms_per_step_eager": round(ms_eager, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "INT8 (E4M3 scales) on W 2560x9728 bf16, h from X 16384x9728 bf16; "
                               "B in {32,64,128,256}; Naive + SSE-Optimal + H-Optimal; hdiag, "
                               + ("X^T X Gram matrix and ||X W^T||^2 from it, " if gram_route else
                                  "X W^T reference, ")
                               + "quantize, dequantize, weight and output error per step",
                   "output_route": args.output_route,
                   "W": [N, K], "X": [M, K], "format": "INT8_E4M3", "blocks": blocks,
                   "quantizations_per_step": len(blocks) * len(methods)},
        "roofline": roofline,
        "stages_ms_per_step": {s: round(v, 4) for s, v in per_step.items()},
        "stages": stages,
        "kernel_gweights_per_s": search_gwps,
        "errors": errs,
    }

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(W_cpu, X_cpu, blocks, methods, fmt, args.cpu_rows, value)
    print(json.dumps(out), flush=True)


def formats_suite(args, dev):
    """Scale choice for every format on the down_proj stand-in (W 2560x9728,
    h from X 16384x9728): per (format, B, method) the kernel time of
    quantize_blocks (median of `steps` launches after `warmup`, HIP events),
    Gweights/s, and the weight / output error of the result (the output error
    against one stored X W^T reference: from the codes for 8-bit scales, from
    the dequantised weights for FP16 scales)."""
    import torch

    import block_scaled_precision_hdiag_amd as hd
    import synth

    W_cpu, X_cpu = synth.config_inputs(2)
    N, K = W_cpu.shape
    M = X_cpu.shape[0]
    W, X = W_cpu.to(dev), X_cpu.to(dev)
    h = hd.hdiag(X)
    ref = hd.output_reference(X, W)
    ws_o = torch.empty(hd.output_error_codes_workspace_size(M, N, K), dtype=torch.uint8, device=dev)
    ysq = hd.reference_ysq(ref)
    ws_g = torch.empty(hd.output_error_workspace_size(M, N, K), dtype=torch.uint8, device=dev)
    rows = []
    names = {v: k for k, v in hd.FORMATS.items()}
    for fmt in sorted(names):
        nc = hd.hdiag_format_info(fmt, 16)[2]
        meths = [("naive", hd.NAIVE), ("sse", hd.SSE_OPT), ("h", hd.H_OPT)]
        if fmt in (hd.MXFP4, hd.MXFP8):
            meths.append(("naive_ocp", hd.NAIVE_OCP))
        # the FP16-scale formats at the pages' B = 128; NVFP4 / NVINT4 also at
        # B = 64, the E4M3-scale point of the same 4.125 bits per weight
        blocks = (128,) if fmt in hd.F16_SCALES else (16, 32, 64) if fmt in (hd.NVFP4, hd.NVINT4) else (16, 32)
        for B in blocks:
            for mname, m in meths:
                codes = torch.empty(hd.codes_shape(fmt, N, K), dtype=torch.uint8, device=dev)
                scales = torch.empty((N, K // B), dtype=hd.scale_dtype(fmt), device=dev)
                run = lambda: hd.quantize_blocks(m, fmt, B, W, h=h, codes=codes, scales=scales)
                for _ in range(max(args.warmup, 1)):
                    run()
                ts = []
                for _ in range(max(args.steps, 1)):
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record()
                    run()
                    b.record()
                    torch.cuda.synchronize()
                    ts.append(a.elapsed_time(b))
                ms = sorted(ts)[len(ts) // 2]
                Wq = hd.dequantize(fmt, B, codes, scales, N, K)
                we = hd.weight_error(W, Wq).item()
                if fmt in hd.F16_SCALES:  # no exact 16-bit operand: the generic product
                    oe = hd.output_error_given_ref(X, W, Wq, ysq, workspace=ws_g).item()
                else:
                    oe = hd.output_error_codes(fmt, B, X, codes, scales, ref, N, K, workspace=ws_o).item()
                rows.append({"format": names[fmt], "B": B, "method": mname, "candidates": nc,
                             "bits_per_weight": hd.hdiag_format_info(fmt, B)[3],
                             "ms": round(ms, 4), "gweights_per_s": round(N * K / (ms * 1e-3) / 1e9, 2),
                             "weight_error": round(we, 6), "output_error": round(oe, 6)})
    print(json.dumps({"suite": "formats", "unit": "Gweights/s",
                      "config": {"workload": "scale choice on W 2560x9728 bf16 (Student-t(4) x 0.02, row gains), "
                                             "h from X 16384x9728 bf16; every format at B in {16, 32} (NVFP4 and "
                                             "NVINT4 also 64), the FP16-scale formats at B = 128",
                                 "W": [N, K], "X": [M, K]},
                      "data": "synthetic", "rows": rows}), flush=True)


def gptq_suite(args, dev):
    """GPTQ on the down_proj stand-in (W 2560x9728, X 16384x9728): for NVFP4,
    MXFP4 and NVINT4 at B = 16 and 32, each of Naive / SSE-Optimal /
    H-Optimal without GPTQ, with GPTQ-Seq and with GPTQ-Ord: the call's time
    (HIP events, one warm-up) and the weight / output error of the result.
    H = X^T X is computed once (its time is reported separately), and so is
    the sequential order's factor of H (gptq_factor): "seq_factored" rows are
    GPTQ-Seq from it (gptq_quantize_factored, the same results as "seq")."""
    import torch

    import block_scaled_precision_hdiag_amd as hd
    import synth

    W_cpu, X_cpu = synth.config_inputs(2)
    N, K = W_cpu.shape
    M = X_cpu.shape[0]
    W, X = W_cpu.to(dev), X_cpu.to(dev)
    ref = hd.output_reference(X, W)
    ysq = hd.reference_ysq(ref)
    ws_g = torch.empty(hd.output_error_workspace_size(M, N, K), dtype=torch.uint8, device=dev)

    def timed(f):
        f()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        r = f()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b), r

    ws_h = torch.empty(hd.gptq_hessian_workspace_size(M, K), dtype=torch.uint8, device=dev)
    H = torch.empty((K, K), dtype=torch.float32, device=dev)
    h_ms, _ = timed(lambda: hd.gptq_hessian(X, H=H, workspace=ws_h))
    h = hd.hdiag(X)
    ws_f = torch.empty(hd.gptq_factor_workspace_size(K), dtype=torch.uint8, device=dev)
    factor = torch.empty(hd.gptq_factor_size(K), dtype=torch.uint8, device=dev)
    f_ms, (_, finfo) = timed(lambda: hd.gptq_factor(H, factor=factor, workspace=ws_f))
    assert int(finfo.item()) == 0
    names = {v: k for k, v in hd.FORMATS.items()}
    rows = []
    for fmt in (hd.NVFP4, hd.MXFP4, hd.NVINT4):
        for B in (16, 32):
            ws = torch.empty(hd.gptq_workspace_size(B, N, K), dtype=torch.uint8, device=dev)
            for mname, m in (("naive", hd.NAIVE), ("sse", hd.SSE_OPT), ("h", hd.H_OPT)):
                for mode in ("none", "seq", "ord", "seq_factored"):
                    if mode == "none":
                        ms, (c, sc, _) = timed(lambda: hd.quantize_blocks(m, fmt, B, W, h=h))
                    elif mode == "seq_factored":
                        ms, (c, sc, _, info) = timed(lambda: hd.gptq_quantize_factored(m, fmt, B, W, H, factor,
                                                                                       workspace=ws))
                        assert int(info.item()) == 0
                    else:
                        ms, (c, sc, _, info) = timed(lambda: hd.gptq_quantize(m, fmt, B, W, H, ordered=mode == "ord",
                                                                              workspace=ws))
                        assert int(info.item()) == 0
                    Wq = hd.dequantize(fmt, B, c, sc, N, K)
                    rows.append({"format": names[fmt], "B": B, "method": mname, "gptq": mode, "ms": round(ms, 3),
                                 "weight_error": round(hd.weight_error(W, Wq).item(), 6),
                                 "output_error": round(hd.output_error_given_ref(X, W, Wq, ysq,
                                                                                  workspace=ws_g).item(), 6)})
                    print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
    print(json.dumps({"suite": "gptq", "config": {"workload": "GPTQ on W 2560x9728 bf16 with H = X^T X from X "
                                                              "16384x9728 bf16 (synthetic stand-ins)",
                                                  "W": [N, K], "X": [M, K]},
                      "hessian_ms": round(h_ms, 3), "factor_ms": round(f_ms, 3), "data": "synthetic", "rows": rows}),
          flush=True)


def sigma_suite(args, dev):
    """Block size against tensor width ("Is Finer Better?", §3.2, §4.3,
    §5.2): a seeded N(0, 1) tensor of 4096 x 4096 is scaled by sigma (40
    values, 1e-4 .. 1) and quantised with E2M1 elements and Naive scales on
    the UE4M3 (E4M3), UE4M4, UE5M3 and binary16 grids and UE4M3 under a
    per-tensor scale (UE4M3-S, §5.1) at B = 8 .. 64; the
    per-tensor MSE (from weight_error's sums) is reported as MSE / sigma^2,
    with the sigma where B = 8 and B = 16 cross for each grid."""
    import numpy as np
    import torch

    import block_scaled_precision_hdiag_amd as hd
    import synth

    N = K = 4096
    Z = synth.weights("normal", N, K, std=1.0, seed=61, dtype=torch.float32).to(dev)
    sigmas = [float(x) for x in np.geomspace(1e-4, 1.0, 40)]
    fmts = (hd.NVFP4, hd.NVFP4_UE4M4, hd.NVFP4_UE5M3, hd.FP4_F16)
    TS = -1  # marker: NVFP4 with a per-tensor scale (UE4M3-S)
    blocks = (8, 16, 32, 64)
    names = {v: k for k, v in hd.FORMATS.items()}
    names[TS] = "NVFP4_TENSOR_SCALED"
    Wq = torch.empty((N, K), dtype=torch.float32, device=dev)
    rows = []
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    ws_t = torch.empty(hd.quantize_blocks_tensor_scaled_workspace_size(N, K), dtype=torch.uint8, device=dev)
    for sg in sigmas:
        W = (Z * sg).contiguous()  # the synthetic input at this width
        for fmt in fmts + (TS,):
            for B in blocks:
                if fmt == TS:  # UE4M3 block scales under a per-tensor scale
                    c, sc, ts, _ = hd.quantize_blocks_tensor_scaled(hd.NAIVE, hd.NVFP4, B, W, workspace=ws_t)
                    hd.dequantize_tensor_scaled(hd.NVFP4, B, c, sc, ts, N, K, out=Wq)
                else:
                    c, sc, _ = hd.quantize_blocks(hd.NAIVE, fmt, B, W)
                    hd.dequantize(fmt, B, c, sc, N, K, out=Wq)
                _, sums = hd.weight_error(W, Wq, sums=True)
                rows.append((sg, fmt, B, sums))
    t1.record()
    torch.cuda.synchronize()
    out = []
    for sg, fmt, B, sums in rows:
        mse = sums[0].item() / (N * K)
        out.append({"sigma": round(sg, 8), "format": names[fmt], "B": B, "mse": mse, "mse_over_sigma2": mse / sg ** 2})
    crossings = {}
    for fmt in fmts + (TS,):
        d = [next(r["mse"] for r in out if r["sigma"] == round(sg, 8) and r["format"] == names[fmt] and r["B"] == 8) -
             next(r["mse"] for r in out if r["sigma"] == round(sg, 8) and r["format"] == names[fmt] and r["B"] == 16)
             for sg in sigmas]
        xs = []
        for i in range(1, len(sigmas)):
            if d[i - 1] > 0 >= d[i]:  # B = 8 worse below, better above
                f = d[i - 1] / (d[i - 1] - d[i])
                xs.append(float(np.exp(np.log(sigmas[i - 1]) + f * (np.log(sigmas[i]) - np.log(sigmas[i - 1])))))
        crossings[names[fmt]] = xs
    print(json.dumps({"suite": "sigma", "config": {"workload": "N(0, sigma^2) 4096x4096 fp32 (one seeded draw scaled), "
                                                               "E2M1 elements, Naive scales", "sigmas": len(sigmas)},
                      "data": "synthetic", "quantizations": len(rows), "total_ms": round(t0.elapsed_time(t1), 3),
                      "b8_b16_crossing_sigma": crossings, "rows": out}), flush=True)


def hbm_suite(args, dev):
    """The HBM-bound stages at the large layer's size (W 8192x28672 bf16,
    470 MB; X 65536x28672 bf16, 3.76 GB), each timed launch preceded by a
    512 MB scratch write so the 256 MB Infinity Cache holds none of its input:
    hdiag, Naive quantize (NVFP4 B = 16, INT8 B = 128), dequantize (to float32
    and to bfloat16) and the weight error; median of 10 launches (HIP events
    around the launch alone), algorithmic bytes / time against 8 TB/s, beside
    a 4 GiB device-to-device copy as the measured ceiling."""
    import torch

    import block_scaled_precision_hdiag_amd as hd
    import synth

    W = synth.config_inputs(5, x_rows=0)[0].to(dev)
    cfg = synth.CONFIGS[5]["X"]
    M, K = cfg["M"], cfg["K"]
    X = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    r = 0
    for ch in synth.activation_chunks(M, K, cfg["seed"], cfg["n_out"], cfg["out_gain"], cfg["idx_seed"],
                                      rows_per_chunk=8192):
        X[r:r + ch.shape[0]] = ch.to(dev)
        r += ch.shape[0]
    N = W.shape[0]
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def timed(f, reps=10):
        f()
        ts = []
        for _ in range(reps):
            scratch.fill_(1)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            f()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return sorted(ts)[reps // 2]

    res = {}

    def put(name, ms, nbytes):
        res[name] = {"ms": round(ms, 4), "bytes": int(nbytes), "gbs": round(nbytes / ms / 1e6, 1),
                     "frac": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}

    src = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    put("device_copy_4GiB", timed(lambda: dst.copy_(src)), 2 * src.numel())
    del src, dst
    h = torch.empty(K, dtype=torch.float32, device=dev)
    ws_h = torch.empty(hd.hdiag_workspace_size(M, K), dtype=torch.uint8, device=dev)
    put("hdiag", timed(lambda: hd.hdiag(X, out=h, workspace=ws_h)), M * K * 2 + K * 4)
    del X
    nw = N * K
    for fmt, B, name, cbytes in ((hd.NVFP4, 16, "nvfp4_b16", 0.5), (hd.INT8_E4M3, 128, "int8_b128", 1.0)):
        codes, scales, _ = hd.quantize_blocks(hd.NAIVE, fmt, B, W)
        put("naive_" + name, timed(lambda: hd.quantize_blocks(hd.NAIVE, fmt, B, W, codes=codes, scales=scales)),
            nw * (2 + cbytes) + nw // B)
        Wq = torch.empty((N, K), dtype=torch.float32, device=dev)
        put("dequantize_f32_" + name, timed(lambda: hd.dequantize(fmt, B, codes, scales, N, K, out=Wq)),
            nw * (cbytes + 4) + nw // B)
        Wb = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
        put("dequantize_bf16_" + name, timed(lambda: hd.dequantize(fmt, B, codes, scales, N, K, dtype=torch.bfloat16,
                                                                  out=Wb)),
            nw * (cbytes + 2) + nw // B)
        ws_e = torch.empty(hd.weight_error_workspace_size(N, K), dtype=torch.uint8, device=dev)
        put("weight_error_" + name, timed(lambda: hd.weight_error(W, Wq, workspace=ws_e)), nw * (2 + 4))
        del Wq, Wb
    print(json.dumps({"suite": "hbm", "config": {"workload": "HBM-bound stages, W 8192x28672 bf16, X 65536x28672 bf16, "
                                                             "Infinity Cache flushed before each launch",
                                                 "W": [N, K], "X": [M, K]},
                      "data": "synthetic", "peak_gbs": HBM_PEAK_GBS, "results": res}), flush=True)


def gemm_suite(args, dev):
    """The MFMA products of the step on their own (X 16384x9728, W 2560x9728
    bf16): output_reference (Y = X W^T stored, fp32), output_error_codes for
    INT8 codes (fp16 operands) and NVFP4 codes (bf16 operands), and torch's
    matmul of the same bf16 product (the vendor library) for comparison.
    Median of 9 timed calls after 2 warm-ups, HIP events on torch's stream."""
    import torch

    import block_scaled_precision_hdiag_amd as hd
    import synth

    W_cpu, X_cpu = synth.config_inputs(2)
    N, K = W_cpu.shape
    M = X_cpu.shape[0]
    W, X = W_cpu.to(dev), X_cpu.to(dev)
    flops = 2.0 * M * N * K

    def timed(f, reps=9):
        for _ in range(2):
            f()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            f()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return sorted(ts)[reps // 2]

    res = {}
    ref = hd.output_reference(X, W)
    res["output_reference"] = timed(lambda: hd.output_reference(X, W, ref=ref))
    ws = torch.empty(hd.output_error_codes_workspace_size(M, N, K), dtype=torch.uint8, device=dev)
    for name, fmt, B in (("output_error_codes_int8", hd.INT8_E4M3, 32), ("output_error_codes_nvfp4", hd.NVFP4, 16)):
        c, sc, _ = hd.quantize_blocks(hd.SSE_OPT, fmt, B, W)
        res[name] = timed(lambda: hd.output_error_codes(fmt, B, X, c, sc, ref, N, K, workspace=ws))
    Wc = W.contiguous()
    res["torch_matmul_bf16"] = timed(lambda: torch.matmul(X, Wc.t()))
    out = {k: {"ms": round(v, 4), "tflops": round(flops / v / 1e9, 1), "frac": round(flops / v / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4)}
           for k, v in res.items()}
    print(json.dumps({"suite": "gemm", "config": {"workload": "X W^T products, X 16384x9728 bf16, W 2560x9728 bf16",
                                                  "M": M, "N": N, "K": K}, "data": "synthetic",
                      "peak_tflops": MFMA_BF16_PEAK_TFLOPS, "results": out}), flush=True)


def cpu_baseline(W_cpu, X_cpu, blocks, methods, fmt, rows, gpu_value):
    """The CPU oracle on a bounded sample of the same step, extrapolated stage
    by stage to the full workload (blocks are independent, so each stage's
    time is linear in the rows it covers)."""
    import numpy as np

    import oracle
    import synth

    N, K = W_cpu.shape
    M = X_cpu.shape[0]
    nt = oracle.max_threads()
    Wb = synth.bits(W_cpu)
    Xb = synth.bits(X_cpu)
    xr_h = 2048          # rows of X for hdiag
    xr_o = 4             # rows of X for the output error
    Ws = Wb[:rows]
    t = time.perf_counter()
    h = oracle.hdiag(Xb[:xr_h])
    t_hdiag = (time.perf_counter() - t) * (M / xr_h)
    h_full = h  # the sample's h weights the sample's search; the cost does not depend on its values
    total = t_hdiag
    for B in blocks:
        for _, m in methods:
            t = time.perf_counter()
            c, s, _ = oracle.quantize(m, fmt, B, Ws, h=h_full if m == oracle.H_OPT else None)
            t_q = time.perf_counter() - t
            t = time.perf_counter()
            Wq = oracle.dequantize(fmt, B, c, s, rows, K)
            oracle.weight_error(Ws, Wq)
            t_d = time.perf_counter() - t
            t = time.perf_counter()
            oracle.output_error(Xb[:xr_o], Ws, Wq)
            t_o = time.perf_counter() - t
            total += (t_q + t_d) * (N / rows) + t_o * (M / xr_o) * (N / rows)
    value = len(blocks) * len(methods) * N * K / total / 1e9
    return {"value": value, "unit": "Gweights/s", "cores": nt, "kind": "oracle",
            "sample": "oracle (C, fp64, OpenMP %d threads) on W rows 0..%d, X rows 0..%d for hdiag and 0..%d "
                      "for the output error, every stage of the step, extrapolated linearly to the full "
                      "2560x9728 / 16384-row workload: %.1f s per step" % (nt, rows - 1, xr_h - 1, xr_o - 1, total),
            "gpu_over_cpu": gpu_value / value}


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the block-scale quantiser hot path on one MI355X.

Workload (one "step"): the INT8 / E4M3-scale case on the qwantize "Results"
page's layer shape -- W 2560 x 9728 bf16 (a seeded Student-t(4) x 0.02 stand-in
with per-row lognormal gain for the down_proj weight) and calibration X
16384 x 9728 bf16 (N(0,1), 8 outlier channels x 50):
    hdiag(X), output_gram(X) (G = X^T X, stored as float16 correlations) and
    output_reference_gram (||X W^T||^2 from G), then for B in
    {32, 64, 128, 256} and each of Naive, SSE-Optimal, H-Optimal:
    quantize_blocks (scale choice + encode), dequantize_weight_error (the
    dequantised weights and the weight error in one pass) and output error
    (output_error_gram_batch after the loop: sum_n d_n^T G d_n for D = Wq - W
    of all 12 quantisations, one MFMA walk of 12 N x K x K over G's upper
    block triangle).
    --output-route direct measures the output error with X instead:
    output_reference (Y = X W^T) once and output_error_codes (X Wq^T - Y, one
    M x N x K MFMA product) per quantisation.
value = 12 quantisations x 2560 x 9728 weights / step time, in Gweights/s.
Inputs are resident in HBM before timing starts.  The step is timed twice:
as individual launches (per-call GPU times from HIP events recorded on the
stream the kernels run on: the per-stage figures and the roofline) and as
replays of the same step captured once in a HIP graph (no host launch gaps;
a replay must first reproduce the eager step's errors bit for bit), which
gives ms_per_step and value unless --eager is given.  The replayed step runs
on two streams (--streams 2, the default; Gram route): after hdiag, the
G = X^T X product and the reference on a second stream, beside the
quantise / dequantize-and-weight-error chain of the 12 quantisations on the
first (the two branches share no buffer; the first stream waits for the
second before the output-error batch); the per-stage times come from the
one-stream launches, and a one-stream replay is timed as well.

Prints one JSON line (the metric, per-stage figures, the roofline of the
dominant kernel and the CPU oracle timed on a bounded sample).
"""
import argparse
import contextlib
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
_NOT_IN_STEP = {"alt_f16.hip", "probe.hip", "gptq.hip", "tscale.hip", "search_e2m1_elems.hip", "search_e4m3_elems.hip",
                "abi.cpp", "kernels.hpp"}


def _code_only(text):
    """C / C++ source without its comments and with runs of white space
    collapsed (string literals kept as they are): what the compiler sees."""
    import re
    tok = re.compile(r'"(?:\\.|[^"\\\n])*"|//[^\n]*|/\*.*?\*/', re.S)
    out = tok.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", text)
    return " ".join(out.split())


def source_hash():
    """Hash of the HIP sources the step's kernels are built from (every file of
    csrc/ but those listed above), comments and layout left out; counter-derived
    traffic is valid only for the kernels it was measured on."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "block_scaled_precision_hdiag_amd", "csrc", "*"))):
        if os.path.basename(f) in _NOT_IN_STEP:
            continue
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
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
    ap.add_argument("--suite", choices=["headline", "formats", "gptq", "sigma", "gemm", "hbm", "config3", "config5"],
                    default="headline",
                    help="headline: the step above (one JSON line, the default); formats: every element / "
                         "scale format x B in {16, 32} x scale choice on the same W and h (one JSON line)")
    ap.add_argument("--eager", action="store_true",
                    help="time the step as individual launches instead of replays of one captured HIP graph")
    ap.add_argument("--streams", type=int, choices=[1, 2], default=2,
                    help="streams of the replayed step (2: G = X^T X and the reference beside the quantisation "
                         "chain; Gram route only)")
    ap.add_argument("--output-route", choices=["gram", "direct"], default="gram",
                    help="output error through G = X^T X (gram) or through X W^T (direct)")
    ap.add_argument("--summarize-profile", metavar="DIR", default=None,
                    help="no GPU: write the step's profile summaries under profiles/ from rocprofv3 csv output in "
                         "DIR/{trace,valu,fetch,write} (the runs made with --copy-probe-mb 1024)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="before timing, run one device copy of this many MB (a known-size kernel that "
                         "calibrates HBM byte counters)")
    return ap.parse_args()


PROFILE_CMDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof/trace -o step -- python3 bench.py "
             "--steps 2 --warmup 1 --no-cpu --eager --copy-probe-mb 1024",
    "valu": "rocprofv3 --pmc SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_WAVE_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE "
            "SQ_INSTS_SALU SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA --output-format csv -d gpurun_out/prof/valu -o step "
            "-- python3 bench.py --steps 1 --warmup 0 --no-cpu --eager --copy-probe-mb 1024",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/prof/fetch -o step -- python3 bench.py "
             "--steps 1 --warmup 0 --no-cpu --eager --copy-probe-mb 1024",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/prof/write -o step -- python3 bench.py "
             "--steps 1 --warmup 0 --no-cpu --eager --copy-probe-mb 1024",
}


def main():
    args = parse()
    if args.summarize_profile:
        return summarize_profile(args.summarize_profile, 1024, PROFILE_CMDS)
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
    if args.suite in ("config3", "config5"):
        return layer_suite(args, dev, int(args.suite[-1]))

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
        osums = torch.empty((len(blocks) * len(methods), 3), dtype=torch.float64, device=dev)
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

    # (weight, candidate) pairs the searches evaluate per launch: one
    # instrumented call per (B, method) outside the timed region, before the
    # copy probe that opens the profiled part
    evals = {"search_sse": [], "search_h": []}
    hd.hdiag(X, out=h, workspace=ws_h)  # the H search's weights (the step recomputes them)
    for B in blocks:
        for mname, m in methods:
            if m == hd.NAIVE:
                continue
            ev = torch.zeros(1, dtype=torch.int64, device=dev)
            hd.quantize_blocks_instrumented(m, fmt, B, W, ev, h=h if m == hd.H_OPT else None)
            evals["search_" + mname].append(ev)
    torch.cuda.synchronize()
    evals = {k: sum(e.item() for e in v) / len(v) for k, v in evals.items()}

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

    side = torch.cuda.Stream(device=dev)  # default priority

    def step(rec, streams=1):
        timed("hdiag", 0, lambda: hd.hdiag(X, out=h, workspace=ws_h), rec)
        two = gram_route and streams == 2
        if two:
            # G and the reference on the second stream, after hdiag
            side.wait_stream(torch.cuda.current_stream())
        if gram_route:
            with torch.cuda.stream(side) if two else contextlib.nullcontext():
                timed("output_gram", 0, lambda: hd.output_gram(X, h=h, gram=gram, workspace=ws_g), rec)
                timed("output_reference", 0, lambda: hd.output_reference_gram(W, gram, workspace=ws_o, out=ysq),
                      rec)
        else:
            timed("output_reference", 0, lambda: hd.output_reference(X, W, ref=ref), rec)
        for bi, B in enumerate(blocks):
            for mi, (mname, m) in enumerate(methods):
                stage = "naive" if m == hd.NAIVE else "search_" + mname
                cb, sb = codes[(B, m)], scales[(B, m)]
                timed(stage, B, lambda: hd.quantize_blocks(m, fmt, B, W, h=h, codes=cb, scales=sb), rec)
                # the dequantised weights and the weight error in one pass
                timed("dequantize_weight_error", B,
                      lambda: hd.dequantize_weight_error(fmt, B, cb, sb, W, out=Wq, err=werr[bi, mi:mi + 1],
                                                         workspace=ws_w), rec)
                if not gram_route:
                    timed("output_error", B,
                          lambda: hd.output_error_codes(fmt, B, X, cb, sb, ref, N, K, workspace=ws_o,
                                                        out=oerr[bi, mi:mi + 1]), rec)
        if gram_route:
            if two:
                torch.cuda.current_stream().wait_stream(side)
            # the 12 output errors in one call (one MFMA walk over their stacked operand)
            items = [(fmt, B, codes[(B, m)], scales[(B, m)]) for B in blocks for _, m in methods]
            timed("output_error", 0,
                  lambda: hd.output_error_gram_batch(items, W, gram, ysq, sums=osums, workspace=ws_o,
                                                     out=oerr.view(-1)), rec)


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
    ms_graph = {}
    if not args.eager:
        # the same step captured once as a HIP graph (every launch of the step,
        # same buffers) on one stream and, with --streams 2, on two; each is
        # replayed, and a replay must reproduce the eager errors bit for bit
        # before its time is used
        eager_w, eager_o = werr.clone(), oerr.clone()
        for ns in sorted({1, args.streams if gram_route else 1}):
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step(False, ns)
            werr.zero_()
            oerr.zero_()
            graph.replay()
            torch.cuda.synchronize()
            if not (torch.equal(werr, eager_w) and torch.equal(oerr, eager_o)):
                raise SystemExit("graph replay (%d streams) does not reproduce the eager step" % ns)
            for _ in range(args.warmup):
                graph.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                graph.replay()
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            ms_graph[ns] = (t1 - t0) * 1e3 / args.steps
            del graph
        ns = max(ms_graph)
        ms_per_step, launch = ms_graph[ns], "hip_graph, %d stream%s" % (ns, "s" if ns > 1 else "")
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
        # codes and scales read, W read, float32 Wq written
        "dequantize_weight_error": ("hbm", sum(N * K + N * K // B + bytes_w + N * K * 4 for B in blocks) / len(blocks)),
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
        c = counters.get(stage)
        if bound == "alu":
            # the search: its work is the (weight, candidate) pairs it evaluated
            # (counted by the instrumented call); what a pair costs in VALU
            # lane-instructions comes from the counters, so `achieved` is the
            # executed VALU lane-op rate against the non-packed FP32 peak
            pairs = evals[stage]
            r = {"bound": "alu", "unit": "Tops/s", "peak": round(VALU_PEAK_TOPS, 3), "avg_ms": round(avg[stage], 4),
                 "evaluated_pairs_per_launch": int(pairs), "candidates_per_weight": round(pairs / (N * K), 3),
                 "gpairs_per_s": round(pairs / t / 1e9, 2),
                 "full_grid_equivalent_tops": round(units / t / 1e12, 3)}
            if c:
                lane_ops = c["SQ_INSTS_VALU"] * 64
                r["achieved"] = round(lane_ops / t / 1e12, 3)
                r["frac"] = round(lane_ops / t / 1e12 / VALU_PEAK_TOPS, 4)
                r["valu_lane_ops_per_pair"] = round(lane_ops / pairs, 2)
                r["valu_busy"] = round(c["valu_busy"], 4)
                r["clock_ghz"] = round(c["clock_ghz"], 3)
            else:
                r["achieved"] = r["frac"] = None
            return r
        if bound == "hbm":
            ach, peak, unit = units / t / 1e9, HBM_PEAK_GBS, "GB/s"
        else:
            ach, peak, unit = units / t / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
        r = {"bound": bound, "achieved": round(ach, 3), "peak": round(peak, 3), "unit": unit,
             "frac": round(ach / peak, 4), "avg_ms": round(avg[stage], 4)}
        if bound == "mfma" and c:
            r["mfma_util"] = round(c["mfma_util"], 4)
            r["clock_ghz"] = round(c["clock_ghz"], 3)
        return r

    stages = {s: roof(s) for s in avg}
    dominant = max(per_step, key=per_step.get)
    roofline = dict(stages[dominant])
    roofline["kernel"] = dominant
    tr = measured_traffic().get(dominant)
    roofline["traffic"] = round(tr["read_bytes"] + tr["write_bytes"]) if tr else None
    roofline["traffic_unit"] = ("bytes per call between the L2s and the memory fabric (rocprofv3 FETCH_SIZE + "
                                "WRITE_SIZE, calibrated on a device copy; Infinity Cache hits included)")
    roofline.pop("avg_ms")

    search_gwps = {s: round(N * K / (avg[s] * 1e-3) / 1e9, 3) for s in avg if s.startswith("search") or s == "naive"}

    errs = {}
    we, oe = werr.cpu().numpy(), oerr.cpu().numpy()
    for bi, B in enumerate(blocks):
        for mi, (mname, _) in enumerate(methods):
            errs["B%d_%s" % (B, mname)] = {"weight_error": round(float(we[bi, mi]), 6),
                                           "output_error": round(float(oe[bi, mi]), 6)}

    if gram_route:
        # b / t of each quantisation (the diagonal part over the total): the
        # Gram route meets the 1e-4 bar for b / t <= 2
        sm = osums.cpu().numpy()
        errs["gram_max_diag_over_total"] = round(float(np.max(sm[:, 2] / sm[:, 0])), 4)

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "Gweights/s", "n_gpus": 1,
        "profiles_source_hash": source_hash(),
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3),
        "launch": launch, "ms_per_step_eager": round(ms_eager, 3),
        "ms_per_step_graph_one_stream": round(ms_graph[1], 3) if ms_graph else None,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "INT8 (E4M3 scales) on W 2560x9728 bf16, h from X 16384x9728 bf16; "
                               "B in {32,64,128,256}; Naive + SSE-Optimal + H-Optimal; hdiag, "
                               + ("X^T X Gram matrix and ||X W^T||^2 from it, " if gram_route else
                                  "X W^T reference, ")
                               + "quantize, dequantize with the weight error, output error per step",
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
        out["cpu_baseline"] = cpu_baseline(W_cpu, X_cpu, blocks, methods, fmt, value, search_gwps)
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


# relative tolerance under which two per-block objectives count as equal:
# block_obj values are float64 sums rounded once to float32 (2^-24), so a
# pair of B = 8 objectives and one B = 16 objective of the same elements
# agree to a few 2^-24 when both blocks took the same codes
BLOCK_TIE = 2.0 ** -20


def block_pair_comparison(obj8, obj16):
    """Per 16-weight block: the B = 8 error (its two 8-blocks' objectives
    added) against the B = 16 error, both from quantize_blocks' block_obj
    ("Is Finer Better?" §3.2, Fig. 2(a): the same tensor quantised at both
    block sizes, MSE taken over the larger block).  Returns the fractions of
    blocks above the diagonal (B = 8 worse), on it (within BLOCK_TIE) and
    below.  Works on torch tensors [N, K/8] and [N, K/16] on any device."""
    import torch
    e8 = obj8.double().reshape(obj16.shape[0], -1, 2).sum(-1)
    e16 = obj16.double()
    tol = BLOCK_TIE * torch.maximum(e8, e16)
    above = (e8 - e16 > tol).double().mean().item()
    below = (e16 - e8 > tol).double().mean().item()
    return {"above": above, "equal": 1.0 - above - below, "below": below}


def mse_decomposition(W, Wq, scale_zero, B):
    """The three parts of the per-tensor MSE that "Is Finer Better?" App. F
    (Fig. 12) separates, from one quantisation: blocks whose scale is zero
    (every element rounded to zero), the maximum-magnitude element of every
    other block (the first one on ties), and the remaining elements.  W, Wq:
    [N, K] tensors; scale_zero: bool [N, K/B].  Returns the three sums of
    squared errors divided by N K (they add up to the MSE), in float64."""
    import torch
    N, K = W.shape
    d2 = (Wq.double() - W.double()) ** 2
    d2b = d2.reshape(N, K // B, B)
    zero = scale_zero.reshape(N, K // B)
    imax = W.abs().reshape(N, K // B, B).argmax(dim=-1, keepdim=True)
    at_max = torch.gather(d2b, 2, imax).squeeze(-1)
    total_b = d2b.sum(-1)
    n = float(N * K)
    s0 = total_b[zero].sum().item() / n
    smax = at_max[~zero].sum().item() / n
    srest = (total_b[~zero] - at_max[~zero]).sum().item() / n
    return {"s_zero": s0, "x_max": smax, "x_other": srest}


def sigma_suite(args, dev):
    """Block size against tensor width ("Is Finer Better?" §3.2 and Fig. 2,
    §4.3, App. F, §5.2): a seeded N(0, 1) tensor of 4096 x 4096 is scaled by
    sigma (40 values, 1e-4 .. 1) and quantised with E2M1 elements and Naive
    scales on the UE4M3 (E4M3), UE4M4, UE5M3 and binary16 grids and UE4M3
    under a per-tensor scale (UE4M3-S, §5.1) at B = 4 .. 64.  Reported:
      - the per-tensor MSE (from weight_error's sums) as MSE / sigma^2, with
        the sigma where B = 8 and B = 16 cross for each grid;
      - per 16-weight block, the B = 8 against the B = 16 error (Fig. 2(a)):
        the fractions of blocks above, on and below the diagonal, for every
        sigma and grid and for the config-4 weights (4096 x 4096 Laplace,
        std 0.02, per-row lognormal gain);
      - for UE4M3 at B = 4, 8, 16, 32, the three parts of the MSE App. F
        separates (zero-scale blocks, block maxima, other elements)."""
    import numpy as np
    import torch

    import block_scaled_precision_hdiag_amd as hd
    import synth

    N = K = 4096
    Z = synth.weights("normal", N, K, std=1.0, seed=61, dtype=torch.float32).to(dev)
    sigmas = [float(x) for x in np.geomspace(1e-4, 1.0, 40)]
    fmts = (hd.NVFP4, hd.NVFP4_UE4M4, hd.NVFP4_UE5M3, hd.FP4_F16)
    TS = -1  # marker: NVFP4 with a per-tensor scale (UE4M3-S)
    blocks = (4, 8, 16, 32, 64)
    names = {v: k for k, v in hd.FORMATS.items()}
    names[TS] = "NVFP4_TENSOR_SCALED"
    Wq = torch.empty((N, K), dtype=torch.float32, device=dev)
    rows, pairs, decomp = [], [], []
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    ws_t = torch.empty(hd.quantize_blocks_tensor_scaled_workspace_size(N, K), dtype=torch.uint8, device=dev)
    for sg in sigmas:
        W = (Z * sg).contiguous()  # the synthetic input at this width
        for fmt in fmts + (TS,):
            objs = {}
            for B in blocks:
                if fmt == TS:  # UE4M3 block scales under a per-tensor scale
                    c, sc, ts, obj = hd.quantize_blocks_tensor_scaled(hd.NAIVE, hd.NVFP4, B, W, block_obj=True,
                                                                      workspace=ws_t)
                    hd.dequantize_tensor_scaled(hd.NVFP4, B, c, sc, ts, N, K, out=Wq)
                else:
                    c, sc, obj = hd.quantize_blocks(hd.NAIVE, fmt, B, W, block_obj=True)
                    hd.dequantize(fmt, B, c, sc, N, K, out=Wq)
                objs[B] = obj
                _, sums = hd.weight_error(W, Wq, sums=True)
                rows.append((sg, fmt, B, sums))
                if fmt == hd.NVFP4 and B <= 32:
                    decomp.append((sg, B, mse_decomposition(W, Wq, sc == 0, B)))
            # (tensor-scaled objectives refer to W / s_T: the same comparison in other units)
            pairs.append((sg, fmt, block_pair_comparison(objs[8], objs[16])))
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
    # the config-4 weights (the MX block-size sweep's tensor) at B = 8 / 16
    W4 = synth.config_inputs(4)[0].to(dev)
    cfg4 = {}
    for fmt in fmts:
        o8 = hd.quantize_blocks(hd.NAIVE, fmt, 8, W4, block_obj=True)[2]
        o16 = hd.quantize_blocks(hd.NAIVE, fmt, 16, W4, block_obj=True)[2]
        cfg4[names[fmt]] = block_pair_comparison(o8, o16)
    print(json.dumps({"suite": "sigma", "config": {"workload": "N(0, sigma^2) 4096x4096 fp32 (one seeded draw scaled), "
                                                               "E2M1 elements, Naive scales", "sigmas": len(sigmas),
                                                   "blocks": list(blocks)},
                      "data": "synthetic", "quantizations": len(rows), "total_ms": round(t0.elapsed_time(t1), 3),
                      "b8_b16_crossing_sigma": crossings,
                      "b8_vs_b16_per_block": [{"sigma": round(sg, 8), "format": names[f], **p} for sg, f, p in pairs],
                      "b8_vs_b16_per_block_config4": cfg4,
                      "ue4m3_mse_parts": [{"sigma": round(sg, 8), "B": B, **p} for sg, B, p in decomp],
                      "rows": out}), flush=True)


def _roof(bound, units, ms):
    """Roofline figures of one stage from its algorithmic work per launch."""
    t = ms * 1e-3
    if bound == "hbm":
        ach, peak, unit = units / t / 1e9, HBM_PEAK_GBS, "GB/s"
    elif bound == "mfma":
        ach, peak, unit = units / t / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        ach, peak, unit = units / t / 1e12, VALU_PEAK_TOPS, "Tops/s"
    return {"bound": bound, "achieved": round(ach, 3), "peak": round(peak, 3), "unit": unit,
            "frac": round(ach / peak, 4), "avg_ms": round(ms, 4)}


def layer_suite(args, dev, ci):
    """Configuration 3 (NVFP4 on the down_proj stand-in W 2560x9728 with the
    pages' full calibration X 244449x9728) or 5 (W 8192x28672, X
    65536x28672): one pass of the hot path over the full X - hdiag, the scale
    choices (config 3: NVFP4 B = 16, 32 x Naive / SSE / H-Optimal; config 5:
    NVFP4 B = 16 and INT8 B = 128, Naive and H-Optimal), dequantize with the
    weight error in one pass, and the output error of every quantisation through G = X^T X
    (output_gram, output_reference_gram, one output_error_gram_batch) and,
    timed separately, through X W^T (output_reference, then one
    output_error_codes per quantisation).  X is streamed to the GPU in row
    chunks; per-stage GPU times are HIP-event averages over `steps` passes
    after one warm-up."""
    import numpy as np
    import torch

    import block_scaled_precision_hdiag_amd as hd
    import synth

    cfg = synth.CONFIGS[ci]
    W = synth.config_inputs(ci, x_rows=0)[0].to(dev)
    N, K = W.shape
    xc = cfg["X"]
    M = xc["M"]
    X = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    r0 = 0
    for ch in synth.activation_chunks(M, K, xc["seed"], xc["n_out"], xc["out_gain"], xc["idx_seed"]):
        X[r0:r0 + ch.shape[0]].copy_(ch)
        r0 += ch.shape[0]
    torch.cuda.synchronize()
    print("config %d: X %dx%d on the GPU" % (ci, M, K), file=sys.stderr, flush=True)
    if ci == 3:
        quants = [(hd.NVFP4, B, m) for B in (16, 32) for m in (hd.NAIVE, hd.SSE_OPT, hd.H_OPT)]
    else:
        quants = [(f, B, m) for f, B in ((hd.NVFP4, 16), (hd.INT8_E4M3, 128)) for m in (hd.NAIVE, hd.H_OPT)]
    mname = {hd.NAIVE: "naive", hd.SSE_OPT: "sse", hd.H_OPT: "h"}
    fname = {v: k for k, v in hd.FORMATS.items()}
    nq = len(quants)
    qstage = ["%s_%s_b%d" % ("naive" if m == hd.NAIVE else "search_" + mname[m], fname[f], B) for f, B, m in quants]
    qmeta = {qstage[q]: quants[q] for q in range(nq)}
    h = torch.empty(K, dtype=torch.float32, device=dev)
    ws_h = torch.empty(hd.hdiag_workspace_size(M, K), dtype=torch.uint8, device=dev)
    gram = torch.empty(hd.output_gram_size(K), dtype=torch.uint8, device=dev)
    ws_g = torch.empty(hd.output_gram_workspace_size(M, K), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(hd.output_error_gram_batch_workspace_size(nq, N, K), dtype=torch.uint8, device=dev)
    ysq = torch.empty(1, dtype=torch.float64, device=dev)
    osums = torch.empty((nq, 3), dtype=torch.float64, device=dev)
    codes = [torch.empty(hd.codes_shape(f, N, K), dtype=torch.uint8, device=dev) for f, _, _ in quants]
    scales = [torch.empty((N, K // B), dtype=torch.uint8, device=dev) for _, B, _ in quants]
    Wq = torch.empty((N, K), dtype=torch.float32, device=dev)
    ws_w = torch.empty(hd.weight_error_workspace_size(N, K), dtype=torch.uint8, device=dev)
    werr = torch.empty(nq, dtype=torch.float64, device=dev)
    oerr = torch.empty(nq, dtype=torch.float64, device=dev)
    events = []

    def timed(stage, fn, rec):
        if not rec:
            return fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        events.append((stage, a, b))

    def gram_pass(rec):
        timed("hdiag", lambda: hd.hdiag(X, out=h, workspace=ws_h), rec)
        timed("output_gram", lambda: hd.output_gram(X, h=h, gram=gram, workspace=ws_g), rec)
        timed("output_reference_gram", lambda: hd.output_reference_gram(W, gram, workspace=ws_b, out=ysq), rec)
        for q, (f, B, m) in enumerate(quants):
            timed(qstage[q], lambda: hd.quantize_blocks(m, f, B, W, h=h, codes=codes[q], scales=scales[q]), rec)
            timed("dequantize_weight_error",
                  lambda: hd.dequantize_weight_error(f, B, codes[q], scales[q], W, out=Wq, err=werr[q:q + 1],
                                                     workspace=ws_w), rec)
        items = [(f, B, codes[q], scales[q]) for q, (f, B, _) in enumerate(quants)]
        timed("output_error_gram_batch",
              lambda: hd.output_error_gram_batch(items, W, gram, ysq, sums=osums, workspace=ws_b, out=oerr), rec)

    gram_pass(False)
    torch.cuda.synchronize()
    print("config %d: warm-up pass done" % ci, file=sys.stderr, flush=True)
    # (weight, candidate) pairs each search evaluates (h is the warm-up's)
    pairs = {}
    for q, (f, B, m) in enumerate(quants):
        if m != hd.NAIVE:
            ev = torch.zeros(1, dtype=torch.int64, device=dev)
            hd.quantize_blocks_instrumented(m, f, B, W, ev, h=h if m == hd.H_OPT else None)
            pairs[qstage[q]] = ev
    torch.cuda.synchronize()
    pairs = {k: v.item() for k, v in pairs.items()}
    t0 = time.perf_counter()
    for _ in range(args.steps):
        gram_pass(True)
    torch.cuda.synchronize()
    pass_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    print("config %d: %d timed passes, %.2f ms each" % (ci, args.steps, pass_ms), file=sys.stderr, flush=True)
    o_gram = oerr.cpu().numpy().copy()
    w_err = werr.cpu().numpy().copy()
    ratios = (osums[:, 2] / osums[:, 0]).cpu().numpy()

    # the direct route: Y = X W^T stored once, then X Wq^T - Y per quantisation
    ref = torch.empty(hd.output_reference_size(M, N, K), dtype=torch.uint8, device=dev)
    ws_c = torch.empty(hd.output_error_codes_workspace_size(M, N, K), dtype=torch.uint8, device=dev)
    o_dir = torch.empty(nq, dtype=torch.float64, device=dev)

    def direct_pass(rec):
        timed("output_reference", lambda: hd.output_reference(X, W, ref=ref), rec)
        for q, (f, B, _) in enumerate(quants):
            timed("output_error_codes", lambda: hd.output_error_codes(f, B, X, codes[q], scales[q], ref, N, K,
                                                                      workspace=ws_c, out=o_dir[q:q + 1]), rec)

    direct_pass(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        direct_pass(True)
    torch.cuda.synchronize()
    direct_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    o_direct = o_dir.cpu().numpy()

    per = {}
    for st, a, b in events:
        per.setdefault(st, []).append(a.elapsed_time(b))
    avg = {k: sum(v) / len(v) for k, v in per.items()}
    nw = N * K
    work = {"hdiag": ("hbm", M * K * 2 + K * 4), "output_gram": ("mfma", 1.0 * M * K * (K + 1)),
            "output_reference_gram": ("mfma", 1.0 * N * K * K),
            # codes (0.5 or 1 B) and scales read, bf16 W read, float32 Wq written; averaged over the quantisations
            "dequantize_weight_error": ("hbm", sum(nw * ((0.5 if f in hd.FOUR_BIT else 1.0) + 2 + 4) + nw // B
                                                   for f, B, _ in quants) / nq),
            "output_error_gram_batch": ("mfma", nq * 1.0 * N * K * K),
            "output_reference": ("mfma", 2.0 * M * N * K), "output_error_codes": ("mfma", 2.0 * M * N * K)}
    stages = {}
    for st, ms in avg.items():
        if st in qmeta and qmeta[st][2] == hd.NAIVE:
            f, B, _ = qmeta[st]
            cb = 0.5 if f in hd.FOUR_BIT else 1.0
            stages[st] = _roof("hbm", nw * (2 + cb) + nw // B, ms)
        elif st in qmeta:
            # the search: its work is the pairs it evaluated; the executed VALU
            # rate (and so the fraction of peak) needs counters, which this
            # suite does not take
            f, B, m = qmeta[st]
            nc = hd.hdiag_format_info(f, 16)[2]
            t = ms * 1e-3
            stages[st] = {"bound": "alu", "unit": "Tops/s", "peak": round(VALU_PEAK_TOPS, 3), "avg_ms": round(ms, 4),
                          "gweights_per_s": round(nw / t / 1e9, 2),
                          "evaluated_pairs_per_launch": int(pairs[st]),
                          "candidates_per_weight": round(pairs[st] / nw, 3),
                          "gpairs_per_s": round(pairs[st] / t / 1e9, 2),
                          "full_grid_equivalent_tops": round(nw * nc * SEARCH_OPS[mname[m]] / t / 1e12, 3),
                          "achieved": None, "frac": None}
        else:
            bound, units = work[st]
            stages[st] = _roof(bound, units, ms)
    errors = {}
    for q, (f, B, m) in enumerate(quants):
        errors["%s_b%d_%s" % (fname[f], B, mname[m])] = {
            "weight_error": round(float(w_err[q]), 6), "output_error_gram": round(float(o_gram[q]), 6),
            "output_error_direct": round(float(o_direct[q]), 6),
            "gram_diag_over_total": round(float(ratios[q]), 4),
            "gram_vs_direct_rel": float(abs(o_gram[q] - o_direct[q]) / o_direct[q])}
    print(json.dumps({"suite": "config%d" % ci, "unit": "Gweights/s",
                      "config": {"workload": "%s: W %dx%d bf16, X %dx%d bf16 (seeded synthetic stand-ins); %d "
                                             "quantisations, hdiag, scale choice, dequantize with the weight error, and "
                                             "output error per pass" % (cfg["name"], N, K, M, K, nq),
                                 "W": [N, K], "X": [M, K]},
                      "data": "synthetic", "steps": args.steps, "pass_ms_gram_route": round(pass_ms, 3),
                      "direct_route_ms": round(direct_ms, 3),
                      "value": round(nq * nw / (pass_ms * 1e-3) / 1e9, 3),
                      "stages": stages, "errors": errors}), flush=True)


def hbm_suite(args, dev):
    """The HBM-bound stages at the large layer's size (W 8192x28672 bf16,
    470 MB; X 65536x28672 bf16, 3.76 GB), each timed launch preceded by a
    512 MB scratch write so the 256 MB Infinity Cache holds none of its input:
    hdiag, Naive quantize (NVFP4 B = 16, INT8 B = 128), dequantize (to float32
    and to bfloat16) and the weight error; median of 10 launches (HIP events
    around the launch alone), algorithmic bytes / time against 8 TB/s, beside
    a 4 GiB device-to-device copy, torch kernels with the stages' byte mixes
    and the library's streaming probes (the stages' loads and stores with
    next to no arithmetic) as references."""
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
    # torch's own kernels with the byte mixes of the stages, as references:
    # a read of W alone (sum), 2 bytes read for 0.5 written per weight (a sum
    # over groups of 4: the NVFP4 encode's code bytes) and 0.5 read for 2
    # written (a broadcast of a quarter-size bf16 tensor: the dequantize to
    # bfloat16)
    N0, K0 = W.shape
    o4 = torch.empty((N0, K0 // 4), dtype=torch.bfloat16, device=dev)
    o1 = torch.empty((), dtype=torch.bfloat16, device=dev)
    put("torch_sum_read_W", timed(lambda: torch.sum(W.view(-1), dim=0, out=o1)), W.numel() * 2)
    put("torch_reduce4_W", timed(lambda: torch.sum(W.view(N0, K0 // 4, 4), dim=-1, out=o4)), W.numel() * 2.5)
    wb = torch.empty_like(W)
    put("torch_expand4_W", timed(lambda: wb.view(N0, K0 // 4, 4).copy_(o4.unsqueeze(-1).expand(N0, K0 // 4, 4))),
        W.numel() * 2.5)
    # the library's streaming probes: the same loads and stores as the encode
    # (NVFP4 B = 16) and the dequantize to bfloat16, and a pure read and a
    # pure write, with next to no arithmetic
    nW = W.numel()
    pc = torch.empty(nW // 2, dtype=torch.uint8, device=dev)
    ps = torch.empty(nW // 16, dtype=torch.uint8, device=dev)
    pr = torch.empty(nW // 8192, dtype=torch.int32, device=dev)
    put("probe_read_W", timed(lambda: hd.hdiag_stream_probe(hd.PROBE_READ, nW, in0=W, out0=pr)), nW * 2)
    put("probe_encode_W", timed(lambda: hd.hdiag_stream_probe(hd.PROBE_ENCODE, nW, in0=W, out0=pc, out1=ps)),
        nW * 2 + nW // 2 + nW // 16)
    put("probe_write_W", timed(lambda: hd.hdiag_stream_probe(hd.PROBE_WRITE, nW, out0=wb)), nW * 2)
    put("probe_dequant_W", timed(lambda: hd.hdiag_stream_probe(hd.PROBE_DEQUANT, nW, in0=pc, in1=ps, out0=wb)),
        nW // 2 + nW // 16 + nW * 2)
    del o4, o1, wb, pc, ps, pr
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
    matmul of the same bf16 product (the vendor library) for comparison; then
    the Gram route's products: output_gram (G = X^T X, M K (K + 1) flop) and
    output_error_gram_batch over the step's 12 INT8 quantisations (12 N K^2
    flop, its operand and final kernels included).  Median of 9 timed calls
    after 2 warm-ups, HIP events on torch's stream."""
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
    fl = {k: flops for k in res}
    h = hd.hdiag(X)
    gram = torch.empty(hd.output_gram_size(K), dtype=torch.uint8, device=dev)
    ws_g = torch.empty(hd.output_gram_workspace_size(M, K), dtype=torch.uint8, device=dev)
    res["output_gram"] = timed(lambda: hd.output_gram(X, h=h, gram=gram, workspace=ws_g))
    fl["output_gram"] = 1.0 * M * K * (K + 1)
    ysq = hd.output_reference_gram(W, gram)
    items = []
    for B in (32, 64, 128, 256):
        for m in (hd.NAIVE, hd.SSE_OPT, hd.H_OPT):
            c, sc, _ = hd.quantize_blocks(m, hd.INT8_E4M3, B, W, h=h)
            items.append((hd.INT8_E4M3, B, c, sc))
    ws_b = torch.empty(hd.output_error_gram_batch_workspace_size(len(items), N, K), dtype=torch.uint8, device=dev)
    ob = torch.empty(len(items), dtype=torch.float64, device=dev)
    res["output_error_gram_batch_12"] = timed(lambda: hd.output_error_gram_batch(items, W, gram, ysq, workspace=ws_b,
                                                                                 out=ob))
    fl["output_error_gram_batch_12"] = len(items) * 1.0 * N * K * K
    out = {k: {"ms": round(v, 4), "tflops": round(fl[k] / v / 1e9, 1),
               "frac": round(fl[k] / v / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4)} for k, v in res.items()}
    print(json.dumps({"suite": "gemm", "config": {"workload": "X W^T products and the Gram route (X^T X, the batch of 12), X 16384x9728 bf16, W 2560x9728 bf16",
                                                  "M": M, "N": N, "K": K}, "data": "synthetic",
                      "peak_tflops": MFMA_BF16_PEAK_TFLOPS, "results": out}), flush=True)


# ------------------------------------------------------------------------
# Profile summaries: rocprofv3 CSV output of the headline step -> the
# committed summaries under profiles/ (no GPU needed).

def _stage_of(name, state):
    """Step stage of one dispatch from its kernel name; state carries which
    operand kernel ran last, which tells the C E^T walk of the reference
    (||X W^T||^2) from the walk of the quantisations' batch."""
    n = name.split("(")[0]
    if "hdiag_vec" in n or "hdiag_col" in n or "hdiag_final" in n:
        return "hdiag"
    if "gram_prep_kernel" in n or "xt_transpose_kernel" in n or "gemm_err_kernel<false, 2," in n:
        return "output_gram"
    if "gram_operand_kernel" in n:
        state["walk"] = "output_reference"
        return "output_reference"
    if "gram_operand_multi_kernel" in n:
        state["walk"] = "output_error"
        return "output_error"
    if "gemm_err_kernel<true, 3," in n or "gram_zero_f64" in n or "gram_final" in n:
        return state.get("walk", "output_error")
    if "encode_kernel" in n:
        return "naive"
    if "search_kernel" in n:
        return "search_h" if n.rstrip().endswith("true>") else "search_sse"
    if "dqwe_partial" in n:
        state["ratio"] = "dequantize_weight_error"
        return "dequantize_weight_error"
    if "dequant_kernel" in n:
        return "dequantize"
    if "werr_partial" in n:
        state["ratio"] = "weight_error"
        return "weight_error"
    if "ratio_final" in n:
        return state.get("ratio", "weight_error")
    if "__amd_rocclr_copyBuffer" in n:
        return "copy"
    return "other"


def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(d, suffix):
    import glob
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise SystemExit("no *%s under %s" % (suffix, d))
    return hits[0]


def _dispatches(rows, with_counters):
    """Per dispatch (in dispatch order): kernel name, stage, duration (ns) and
    counters.  The copy probe is the largest __amd_rocclr_copyBuffer."""
    by = {}
    for r in rows:
        k = int(r["Dispatch_Id"])
        e = by.setdefault(k, {"name": r["Kernel_Name"], "t": int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),
                              "c": {}})
        if with_counters:
            e["c"][r["Counter_Name"]] = float(r["Counter_Value"])
    state = {}
    out = []
    for k in sorted(by):
        e = by[k]
        e["stage"] = _stage_of(e["name"], state)
        out.append(e)
    copies = [i for i, e in enumerate(out) if e["stage"] == "copy"]
    probe = max(copies, key=lambda i: out[i]["t"]) if copies else -1
    if probe >= 0:
        out[probe]["stage"] = "copy_probe"
    # set-up work (the instrumented search calls and their hdiag among it):
    # every dispatch before the first hdiag that follows the copy probe
    started = False
    for i, e in enumerate(out):
        started = started or (i > probe and e["stage"] == "hdiag")
        if not started and e["stage"] not in ("copy", "copy_probe"):
            e["stage"] = "setup"
    return out


STAGE_ORDER = ["hdiag", "output_gram", "output_reference", "naive", "search_sse", "search_h", "dequantize",
               "weight_error", "dequantize_weight_error", "output_error"]
# calls of each stage in one step (a call may launch several kernels)
STAGE_CALLS = {"hdiag": 1, "output_gram": 1, "output_reference": 1, "naive": 4, "search_sse": 4, "search_h": 4,
               "dequantize": 12, "weight_error": 12, "dequantize_weight_error": 12, "output_error": 1}


def summarize_profile(d, probe_mb, cmds):
    """Write the kernel-stats, counters and traffic summaries of the step from
    rocprofv3 output under d (trace/, valu/, fetch/, write/ subdirectories)
    into profiles/."""
    sh = source_hash()
    tr = _dispatches(_read_csv(_find(os.path.join(d, "trace"), "kernel_trace.csv")), False)
    steps = sum(1 for e in tr if "hdiag_final" in e["name"] and e["stage"] == "hdiag")
    # kernel statistics, one row per (kernel, stage)
    agg = {}
    for e in tr:
        if e["stage"] in ("other", "copy", "copy_probe", "setup"):
            continue
        key = (e["name"].split("(")[0], e["stage"])
        agg.setdefault(key, []).append(e["t"] / 1e3)
    tot = sum(sum(v) for v in agg.values())
    per_stage = {}
    for e in tr:
        if e["stage"] in STAGE_ORDER:
            per_stage.setdefault(e["stage"], 0.0)
            per_stage[e["stage"]] += e["t"] / 1e3
    lines = ["# Kernel statistics: the bench.py step (INT8 / E4M3 scales, W 2560x9728 bf16, X 16384x9728 bf16)", "",
             "One MI355X (gfx950).  Command, from the repository root:", "", "    " + cmds["trace"], "",
             "%d steps ran (warm-up included).  Rows are split by the step stage a dispatch belongs to: the C E^T "
             "walk `gemm_err_kernel<true, 3, ...>` serves output_reference_gram (one E, the reference ||X W^T||^2) "
             "and the output errors of the quantisations (output_error_gram_batch, in walks of two "
             "quantisations); `gemm_err_kernel<false, 2, ...>` is the X^T X product of output_gram.  Summary made "
             "by `python bench.py --summarize-profile DIR`; step sources' hash (bench.py source_hash): %s." % (steps, sh),
             "", "| kernel | stage | calls | avg (us) | min (us) | max (us) | % time |", "|---|---|---:|---:|---:|---:|---:|"]
    for (k, st), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        lines.append("| `%s` | %s | %d | %.1f | %.1f | %.1f | %.2f |" % (k[:90], st, len(v), sum(v) / len(v), min(v),
                                                                        max(v), 100 * sum(v) / tot))
    lines += ["", "Per stage (all kernels of the stage, per step):", "", "| stage | us per step |", "|---|---:|"]
    for st in STAGE_ORDER:
        if st in per_stage:
            lines.append("| %s | %.1f |" % (st, per_stage[st] / steps))
    with open(os.path.join(ROOT, "profiles", "int8_down_proj_2560x9728_kernel_stats.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    # counters: executed VALU / MFMA work per stage, clocks from GRBM_GUI_ACTIVE
    va = _dispatches(_read_csv(_find(os.path.join(d, "valu"), "counter_collection.csv")), True)
    cs = {}
    for e in va:
        if e["stage"] not in STAGE_ORDER:
            continue
        c = cs.setdefault(e["stage"], {"launches": 0, "ns": 0.0})
        c["launches"] += 1
        c["ns"] += e["t"]
        for k, v in e["c"].items():
            c[k] = c.get(k, 0.0) + v
    csteps = sum(1 for e in va if "hdiag_final" in e["name"] and e["stage"] == "hdiag")
    rec = {}
    lines = ["# Executed VALU / MFMA work per call: the bench.py step (INT8 / E4M3 scales, W 2560x9728, X 16384x9728)",
             "", "One MI355X (gfx950).  One counter pass, from the repository root:", "", "    " + cmds["valu"], "",
             "Per stage: summed over all kernels of its calls in the step and divided by the calls (the search and "
             "Naive stages are one kernel per call; output_error is the batch call with its operand, walk and final "
             "kernels).  GRBM_GUI_ACTIVE is reported summed over the 8 XCDs, so GRBM_GUI_ACTIVE / 8 / duration is "
             "the shader clock during the call's kernels (meaningful for calls of 100 us and more; for shorter ones "
             "the counter's activity window exceeds the kernels' run time).  VALUBusy = "
             "SQ_ACTIVE_INST_VALU / CU_NUM / (GRBM_GUI_ACTIVE / 8) and MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES / "
             "(SIMD_NUM x GRBM_GUI_ACTIVE / 8) are the vendor's derived metrics (rocprofv3 -L), here with CU_NUM = "
             "256 and SIMD_NUM = 1024; both are taken against the cycles the clock actually ran.  SQ_ACTIVE_INST_VALU "
             "counts one quad-cycle per wave64 VALU instruction (it equals SQ_INSTS_VALU here), so VALUBusy assumes "
             "four shader cycles per instruction; readings above 1 mean the SIMDs issue more than one VALU "
             "instruction per four cycles on average (gfx950 finishes some VALU instructions in fewer than four), "
             "i.e. the VALU issue port is saturated.  Durations are those of this counter pass.",
             "", "| stage | calls | kernels | us per call | clock GHz | VALU instr / call | VALUBusy | MFMA instr / call | MfmaUtil |",
             "|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for st in STAGE_ORDER:
        if st not in cs:
            continue
        c = cs[st]
        n = STAGE_CALLS[st] * max(csteps, 1)
        grbm = c.get("GRBM_GUI_ACTIVE", 0.0) / 8.0
        clk = grbm / (c["ns"] * 1e-9) / 1e9 if c["ns"] else 0.0
        vb = c.get("SQ_ACTIVE_INST_VALU", 0.0) / 256.0 / grbm if grbm else 0.0
        mu = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (1024.0 * grbm) if grbm else 0.0
        rec[st] = {"calls": n, "kernels": c["launches"], "avg_us": c["ns"] / n / 1e3, "clock_ghz": clk,
                   "valu_busy": vb, "mfma_util": mu,
                   "SQ_INSTS_VALU": c.get("SQ_INSTS_VALU", 0.0) / n, "SQ_INSTS_MFMA": c.get("SQ_INSTS_MFMA", 0.0) / n,
                   "SQ_VALU_MFMA_BUSY_CYCLES": c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / n,
                   "GRBM_GUI_ACTIVE": c.get("GRBM_GUI_ACTIVE", 0.0) / n}
        lines.append("| %s | %d | %d | %.1f | %.2f | %.4g | %.3f | %.4g | %.3f |" % (
            st, n, c["launches"], c["ns"] / n / 1e3, clk, rec[st]["SQ_INSTS_VALU"], vb, rec[st]["SQ_INSTS_MFMA"], mu))
    lines += ["", "Machine-readable record read by bench.py (used only while the step's sources in csrc/ still hash "
                  "to source_hash):", "", "counters-json: " + json.dumps({"source_hash": sh, "stages": rec})]
    with open(os.path.join(ROOT, "profiles", "int8_down_proj_2560x9728_counters.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    # HBM traffic: FETCH_SIZE / WRITE_SIZE (KiB per dispatch), calibrated on the
    # copy probe of probe_mb MiB (it reads and writes probe_mb MiB)
    rd = _dispatches(_read_csv(_find(os.path.join(d, "fetch"), "counter_collection.csv")), True)
    wr = _dispatches(_read_csv(_find(os.path.join(d, "write"), "counter_collection.csv")), True)
    probe = float(probe_mb) * (1 << 20)
    fr = [e for e in rd if e["stage"] == "copy_probe"][0]["c"]["FETCH_SIZE"] * 1024.0
    fw = [e for e in wr if e["stage"] == "copy_probe"][0]["c"]["WRITE_SIZE"] * 1024.0
    kr, kw = probe / fr, probe / fw
    tr_rec = {}
    for lst, key, fac, col in ((rd, "FETCH_SIZE", kr, "read_bytes"), (wr, "WRITE_SIZE", kw, "write_bytes")):
        n = {}
        for e in lst:
            if e["stage"] in STAGE_ORDER:
                t = tr_rec.setdefault(e["stage"], {"read_bytes": 0.0, "write_bytes": 0.0, "launches": 0})
                t[col] += e["c"].get(key, 0.0) * 1024.0 * fac
                n[e["stage"]] = n.get(e["stage"], 0) + 1
        for st, cnt in n.items():
            tr_rec[st]["launches"] = cnt
    launches = STAGE_CALLS
    lines = ["# HBM traffic per launch: the bench.py step (INT8 / E4M3 scales, W 2560x9728, X 16384x9728)", "",
             "One MI355X (gfx950).  Two counter passes, from the repository root:", "", "    " + cmds["fetch"],
             "    " + cmds["write"], "",
             "FETCH_SIZE and WRITE_SIZE (KiB per dispatch) summed over each stage's kernels in one step and divided "
             "by the stage's calls per step (output_error is one output_error_gram_batch call: its operand, walk "
             "and final kernels for all 12 quantisations).  Both counters are taken where the L2 caches meet the "
             "memory fabric: they count every L2 miss and write-back, whether the Infinity Cache or HBM serves it, "
             "so they bound the HBM bytes from above.  Calibration: the same passes count a device copy of "
             "%d MiB (the copy probe, which reads and writes %d MiB) as %.0f MiB fetched and %.0f MiB written, so "
             "reads are scaled by %.3f and writes by %.3f." % (probe_mb, probe_mb, fr / (1 << 20), fw / (1 << 20), kr, kw),
             "", "| stage | calls per step | read GB per call | write GB per call |", "|---|---:|---:|---:|"]
    for st in STAGE_ORDER:
        if st in tr_rec:
            t = tr_rec[st]
            L = launches[st]
            t["read_bytes"] /= L
            t["write_bytes"] /= L
            lines.append("| %s | %d | %.4f | %.4f |" % (st, L, t["read_bytes"] / 1e9, t["write_bytes"] / 1e9))
    lines += ["", "Machine-readable record read by bench.py (used only while the step's sources in csrc/ still hash "
                  "to source_hash):", "", "traffic-json: " + json.dumps({"source_hash": sh, "read_scale": kr,
                                                                         "write_scale": kw, "stages": tr_rec})]
    with open(os.path.join(ROOT, "profiles", "int8_down_proj_2560x9728_hbm_traffic.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote profiles/int8_down_proj_2560x9728_{kernel_stats,counters,hbm_traffic}.md (source hash %s)" % sh)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(W_cpu, X_cpu, blocks, methods, fmt, gpu_value, gpu_search):
    """The CPU oracle on bounded samples of the same step, each stage timed at
    two sample sizes and extrapolated from the slope (so a call's fixed cost is
    not multiplied up): hdiag over rows of X, the scale choice, dequantize and
    weight error over rows of W, and the output error over rows of X for a
    fixed block of W rows (its cost is rows of X x rows of W).  Every sample has
    at least as many rows as the oracle has threads, so all of them work.  Run
    with all threads and with one."""
    import numpy as np

    import oracle
    import synth

    N, K = W_cpu.shape
    M = X_cpu.shape[0]
    Wb = synth.bits(W_cpu)
    Xb = synth.bits(X_cpu)

    def clock(f):
        t = time.perf_counter()
        f()
        return time.perf_counter() - t

    def fit(t1, n1, t2, n2):
        b = max((t2 - t1) / (n2 - n1), 0.0)
        return b, max(t1 - b * n1, 0.0)  # per-unit cost, fixed cost

    def run(nt):
        w1, w2 = 4 * nt, 16 * nt       # rows of W
        x1, x2 = 16 * nt, 64 * nt      # rows of X (output error, with w2 rows of W)
        h1, h2 = 256 * nt, 1024 * nt   # rows of X (hdiag)
        st = {}
        b, a = fit(clock(lambda: oracle.hdiag(Xb[:h1], nthreads=nt)), h1,
                   clock(lambda: oracle.hdiag(Xb[:h2], nthreads=nt)), h2)
        st["hdiag"] = a + b * M
        h = oracle.hdiag(Xb[:h2], nthreads=nt)
        st["quantize"], st["dequantize_weight_error"], st["output_error"] = 0.0, 0.0, 0.0
        search = {"sse": 0.0, "h": 0.0}
        for B in blocks:
            for mname, m in methods:
                tq, td = [], []
                for r in (w1, w2):
                    t = time.perf_counter()
                    c, s, _ = oracle.quantize(m, fmt, B, Wb[:r], h=h if m == oracle.H_OPT else None, nthreads=nt)
                    tq.append(time.perf_counter() - t)
                    t = time.perf_counter()
                    Wq = oracle.dequantize(fmt, B, c, s, r, K, nthreads=nt)
                    oracle.weight_error(Wb[:r], Wq, nthreads=nt)
                    td.append(time.perf_counter() - t)
                b, a = fit(tq[0], w1, tq[1], w2)
                st["quantize"] += a + b * N
                if mname in search:
                    search[mname] += (a + b * N) / len(blocks)
                b, a = fit(td[0], w1, td[1], w2)
                st["dequantize_weight_error"] += a + b * N
                t1 = clock(lambda: oracle.output_error(Xb[:x1], Wb[:w2], Wq, nthreads=nt))
                t2 = clock(lambda: oracle.output_error(Xb[:x2], Wb[:w2], Wq, nthreads=nt))
                b, a = fit(t1, x1, t2, x2)
                st["output_error"] += a + b * M * (N / w2)
        return st, search

    nt = oracle.max_threads()
    t0 = time.perf_counter()
    st_all, se_all = run(nt)
    st_one, se_one = run(1)
    wall = time.perf_counter() - t0
    q = len(blocks) * len(methods)
    tot_all, tot_one = sum(st_all.values()), sum(st_one.values())
    value = q * N * K / tot_all / 1e9
    return {"value": value, "unit": "Gweights/s", "cores": nt, "kind": "oracle",
            "sample": "oracle (C, fp64, OpenMP) on the step's own inputs, with t threads: W rows 0..4t-1 and "
                      "0..16t-1 for the scale choice, dequantize and weight error, X rows 0..16t-1 and 0..64t-1 (with "
                      "W rows 0..16t-1) for the output error, X rows 0..256t-1 and 0..1024t-1 for hdiag; each stage "
                      "extrapolated from the slope between its two sample sizes to the full 2560x9728 / 16384-row "
                      "step: %.1f s per step with t = %d, %.1f s with t = 1; %.1f s of host time in all"
                      % (tot_all, nt, tot_one, wall),
            "cpu_model": _cpu_model(), "nproc": os.cpu_count(),
            "stage_seconds_per_step": {k: round(v, 3) for k, v in st_all.items()},
            "stage_seconds_per_step_1thread": {k: round(v, 3) for k, v in st_one.items()},
            "value_1thread": q * N * K / tot_one / 1e9,
            "search_gweights_per_s": {k: round(N * K / v / 1e9, 5) for k, v in se_all.items()},
            "search_gweights_per_s_1thread": {k: round(N * K / v / 1e9, 5) for k, v in se_one.items()},
            "gpu_search_gweights_per_s": gpu_search,
            "gpu_over_cpu": gpu_value / value}


if __name__ == "__main__":
    main()

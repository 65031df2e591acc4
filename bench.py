"""Benchmark of the GuidedQuant Fisher + LNQ hot path on one MI355X.

One step = the whole path on one synthetic layer with inputs resident in HBM:
grouped Fisher accumulation from (X, G), then LNQ (init + `iters` x (codebook
step, assignment pass) + objective trace) on every output row.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--path lnq|grid|ganq|lut|stream] [--no-cpu-baseline]

--path grid replaces LNQ by the fixed-grid backend (uniform min-max grid per
row, `iters` assignment passes, no codebook step) and reports that path's own
metric.  --path ganq replaces LNQ's assignment pass by the GANQ-style
back-substitution over the Cholesky factor of F' (factor included in the step).
--path lut times the lookup-table product y = W_hat x of the packed
(C, P) format instead (default layer 28672 -> 8192, 4-bit, one bfloat16
activation vector): a step is --lut-reps back-to-back products.  --path stream
times the Fisher alone with X and G in pinned host memory, streamed to the GPU
in chunks of --chunk-tokens tokens (PCIe-bound).

Prints one JSON line.  `value` is rows quantized per second for the whole
layer (Fisher included); the Fisher TFLOP/s, the LNQ-only rows/s and the
per-stage times are extra fields.  The per-stage times come from the last
warmup step, run with every stage bracketed by HIP events on the library's
stream; the timed steps carry events around the dominant stage only, and
`roofline` is computed for that stage from those events.  The
`cpu_baseline` leg times the fp64 oracle on a bounded sample of the same
workload on the host cores.
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

PEAK_BF16_MFMA = 2500e12      # dense bf16 matrix-core FLOP/s
# fp32 vector arithmetic: 256 compute units x 4 SIMDs x 16 lanes at 2.4 GHz = 39.3e12 lane
# operations/s.  An FMA is 2 flops, so 78.6e12 FLOP/s with one FMA per lane per cycle, the
# rate this build issues (its device code is compiled without packed fp32 instructions);
# packed fp32 (two per lane per cycle) doubles it to the published 157.3e12.
PEAK_FP32_VALU = 78.6e12      # fp32 vector FLOP/s this build can issue (unpacked FMA)
PEAK_FP32_VALU_PACKED = 157.3e12
PEAK_HBM = 8e12               # bytes/s
PEAK_FP32_ADD = 78.6e12       # fp32 vector adds/s of the chip (packed: two adds per lane per cycle)
PEAK_FP64_VALU = 78.6e12      # fp64 vector FLOP/s (FMA = 2 flops)
PEAK_PCIE = 63.0e9            # host-to-device bytes/s, PCIe 5.0 x16 (32 GT/s x 16, 128b/130b)


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=None,
                    help="llama2_7b_attn by default; llama2_70b_down for --path lut")
    ap.add_argument("--path", choices=("lnq", "grid", "ganq", "lut", "stream"), default="lnq")
    ap.add_argument("--chunk-tokens", type=int, default=16384)
    ap.add_argument("--lut-reps", type=int, default=100)
    ap.add_argument("--lut-batch", type=int, default=1)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (calibrates "
                         "the HBM byte counters against a kernel of known traffic)")
    ap.add_argument("--cpu-rows", type=int, default=64,
                    help="rows of the CPU baseline's LNQ sample (spread over the host cores)")
    ap.add_argument("--cpu-tokens", type=int, default=16384,
                    help="tokens of the CPU baseline's Fisher sample")
    ap.add_argument("--block", type=int, default=512,
                    help="assignment block B (64, 128, 256 or 512; the result is the same up "
                         "to float32 summation order)")
    return ap.parse_args()


# HBM bytes per launch of a stage's kernel, from rocprofv3 FETCH_SIZE and WRITE_SIZE passes
# over the 4096 x 4096 layer, scaled by what the counters read for a plain 1 GiB copy
# (fetch x 2.0, write x 1.0).  Each entry holds a digest of the kernel's source file and
# the headers it includes at the time the counters were taken; once the source changes the
# figure no longer describes the kernel and is reported as null.
_CSRC = os.path.join(ROOT, "post_weight_quantization_gq_amd", "csrc")
_TRAFFIC = {
    # stage: (workload, source file, digest, bytes read, bytes written) of its main kernel,
    # averaged over the launches that do the work
    "lnq_gram": ("llama2_7b_attn", "gq_lnq_mm.hip", "80dc741c80ab9adb", 267339818, 16777216),
    "fisher_mfma": ("llama2_7b_attn", "gq_fisher.hip", "cddf0c6a79bd9111", 7052849959, 1384120320),
    "lnq_sweep": ("llama2_7b_attn", "gq_lnq.hip", "683fbfa5a52f52ca", 710898895, 270519898),
    "lnq_resid": ("llama2_7b_attn", "gq_lnq_mm.hip", "80dc741c80ab9adb", 403082224, 67108864),
    "lnq_delta": ("llama2_7b_attn", "gq_lnq.hip", "683fbfa5a52f52ca", 1879248210, 85692275),
    "ganq_pass": ("llama2_7b_attn", "gq_ganq.hip", "dc6ee64370d8c958", 731559625, 259311091),
    "lut_gemv": ("llama2_70b_down", "gq_lut.hip", "623cb61e64e42808", 118509837, 42933),
}


def _source_digest(fname):
    import hashlib
    h = hashlib.sha256()
    for f in (fname, "gq_common.h", "gq_internal.h"):
        with open(os.path.join(_CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(stage, wl):
    t = _TRAFFIC.get(stage)
    if t is None or t[0] != wl.name or _source_digest(t[1]) != t[2]:
        return None
    return t[3] + t[4]


def _incremental_iters(wl, nchg):
    """Iterations whose codebook step updates A and the residual from the previous
    pass's changed coordinates (the library's switch: at most d_out d_in (m + 3) 17 / 10000
    changes), given the per-pass change counts."""
    lim = wl.d_out * wl.d_in * (wl.m + 3) * 17 // 10000
    return [t for t in range(2, wl.iters + 1) if nchg[t - 2] <= lim]


def _grid_roofline(wl, nchg, ms_step):
    """Composite lower bound on one layer with the fixed-grid backend:
      group scale and Fisher as for LNQ;
      per pass           4 G d_in^2 (F' read once) + d_out d_in (codes) bytes at the HBM peak
                         + (3 m d_in per row for the candidate changes + 2 d_in per changed
                         coordinate) fp32 flops at the fp32 vector peak.
    frac = t_roof / t_measured."""
    n, d, d_out, G, m, it = wl.n, wl.d_in, wl.d_out, wl.groups, wl.m, wl.iters
    t_scale = (2 * n * d_out + 4 * G * n) / PEAK_HBM
    t_fisher = n * d * (d + 1) * G / PEAK_BF16_MFMA
    t_bytes = it * (4 * G * d * d + d_out * d) / PEAK_HBM
    t_alu = (it * d_out * 3 * m * d + 2 * d * float(np.sum(nchg))) / PEAK_FP32_VALU_PACKED
    t_roof = t_scale + t_fisher + t_bytes + t_alu
    return {"t_roof_ms": t_roof * 1e3, "t_measured_ms": ms_step, "frac": t_roof * 1e3 / ms_step,
            "terms_ms": {"group_scale": t_scale * 1e3, "fisher": t_fisher * 1e3,
                         "passes_bytes": t_bytes * 1e3, "passes_alu": t_alu * 1e3}}


def _ganq_roofline(wl, nchg, ms_step):
    """Composite lower bound on one layer with the GANQ-style alternation: group scale and
    Fisher as for LNQ; the float64 Cholesky of every group (G d_in^3 / 3 FMAs at the fp64
    vector peak); per iteration the codebook systems as for LNQ and the back-substitution's
    matrix-core product (3 bf16 products over the triangle, d_out d_in^2 flops each).
    frac = t_roof / t_measured."""
    n, d, d_out, G, m, it = wl.n, wl.d_in, wl.d_out, wl.groups, wl.m, wl.iters
    t_scale = (2 * n * d_out + 4 * G * n) / PEAK_HBM
    t_fisher = n * d * (d + 1) * G / PEAK_BF16_MFMA
    t_chol = 2 * G * d ** 3 / 3 / PEAK_FP64_VALU
    t_gram = it * max(d_out * d * d / PEAK_FP32_ADD, (4 * G * d * d + d_out * d) / PEAK_HBM)
    t_back = it * 3 * d_out * d * d / PEAK_BF16_MFMA
    t_roof = t_scale + t_fisher + t_chol + t_gram + t_back
    return {"t_roof_ms": t_roof * 1e3, "t_measured_ms": ms_step, "frac": t_roof * 1e3 / ms_step,
            "terms_ms": {"group_scale": t_scale * 1e3, "fisher": t_fisher * 1e3,
                         "cholesky": t_chol * 1e3, "codebook_systems": t_gram * 1e3,
                         "back_substitution": t_back * 1e3}}


def _layer_roofline(wl, nchg, ms_step):
    """Composite lower bound on the time of one layer (Fisher + LNQ), term by term:
      group scale        bytes 2 n d_out + 4 G n at the HBM peak;
      Fisher             n d_in (d_in + 1) G flops (unique entries) at the bf16 MFMA peak;
      per iteration      max(d_out d_in^2 adds at the fp32 add peak (the gather-reduce of
                         P^T F' P), 4 G d_in^2 + d_out d_in bytes at the HBM peak)
                         + (2 d_in m per row for the residual refresh + 2 d_in per changed
                         coordinate) fp32 flops at the fp32 vector peak.
    frac = t_roof / t_measured."""
    n, d, d_out, G, m, it = wl.n, wl.d_in, wl.d_out, wl.groups, wl.m, wl.iters
    t_scale = (2 * n * d_out + 4 * G * n) / PEAK_HBM
    t_fisher = n * d * (d + 1) * G / PEAK_BF16_MFMA
    t_gram = it * max(d_out * d * d / PEAK_FP32_ADD, (4 * G * d * d + d_out * d) / PEAK_HBM)
    t_upd = (it * d_out * 2 * d * m + 2 * d * float(np.sum(nchg))) / PEAK_FP32_VALU_PACKED
    t_roof = t_scale + t_fisher + t_gram + t_upd
    return {"t_roof_ms": t_roof * 1e3, "t_measured_ms": ms_step, "frac": t_roof * 1e3 / ms_step,
            "terms_ms": {"group_scale": t_scale * 1e3, "fisher": t_fisher * 1e3,
                         "codebook_systems": t_gram * 1e3, "residual_and_moves": t_upd * 1e3}}


def _stage_units(stage, wl, nchg, grid=False, ganq=False):
    """Algorithmic work of a stage in one step: (bound, amount, peak, unit, launches).

    The contractions count the flops of the bf16 products the method runs: F' and the
    error E enter as bf16 hi + lo pairs to reach float32-level accuracy, so the
    residual is three bf16 products and the codebook Gram two (its one-hot operand
    is exact in bf16), over the upper triangle of 256-wide tiles of F'.  `launches` is
    the number of launches per step that do the work (a step after a pass with few
    changes skips the Gram and the residual before it; those launches return at
    once), or None when every launch does.
    """
    n, d, d_out, G, m, it = wl.n, wl.d_in, wl.d_out, wl.groups, wl.m, wl.iters
    incr = [] if (grid or ganq) else _incremental_iters(wl, nchg)
    dense = 0 if grid else it - len(incr)
    if stage == "fisher_mfma":
        # unique entries of the symmetric F_g: n d (d + 1) flops per group
        return "mfma", n * d * (d + 1) * G, PEAK_BF16_MFMA, "TFLOP/s", None
    if stage == "lnq_gram":
        ntile = (d + 255) // 256
        tri = sum(min(256, d - 256 * t) * (d - 256 * t) for t in range(ntile))
        return "mfma", dense * 2 * 2 * tri * d_out * m, PEAK_BF16_MFMA, "TFLOP/s", dense
    if stage == "ganq_chol":
        # float64 Cholesky of every group's F': d^3 / 3 FMAs per group
        return "alu", 2 * G * d ** 3 / 3, PEAK_FP64_VALU, "TFLOP/s", None
    if stage == "ganq_pass":
        # the matrix-core part of the back-substitution: E U^T over the strict upper
        # triangle of U = L^T as three bf16 products
        return "mfma", it * 3 * 2 * d_out * d * d / 2, PEAK_BF16_MFMA, "TFLOP/s", None
    if stage == "lnq_resid":
        # before each recomputed codebook step, before each pass, and the final objective;
        # each E F' per group as three bf16 products (the fixed-grid path: before each
        # pass and the final objective; GANQ: in each codebook step, after it, and the
        # final objective)
        calls = dense + it + 1
        return "mfma", calls * 3 * 2 * d_out * d * d, PEAK_BF16_MFMA, "TFLOP/s", calls
    if stage == "lnq_delta":
        # per updated step: one float32 row of F per changed coordinate, old and new codes,
        # the residual read and written, the per-slice shares of A written
        nsl = (d + 511) // 512
        amount = sum(4 * d * float(nchg[t - 2]) + d_out * d * (1 + 1 + 4 + 4) +
                     d_out * nsl * m * m * 4 for t in incr)
        return "hbm", amount, PEAK_HBM, "GB/s", len(incr)
    if stage == "lnq_sweep":
        # m candidate changes (3 flops each) per coordinate, 2 d flops per move
        return ("alu", it * d_out * d * 3 * m + 2 * d * float(np.sum(nchg)), PEAK_FP32_VALU,
                "TFLOP/s", None)
    if stage == "lnq_solve":
        # per call: read R, P, W and the Gram partials (the fixed-grid path: the final
        # objective only)
        ntile = (d + 255) // 256
        if grid:
            return "hbm", d_out * d * (4 + 1 + 2), PEAK_HBM, "GB/s", None
        return ("hbm", (it + 1) * d_out * (d * (4 + 1 + 2) + ntile * m * m * 4), PEAK_HBM,
                "GB/s", None)
    if stage == "group_scale":
        return "hbm", 2 * n * d_out + 4 * G * n, PEAK_HBM, "GB/s", None
    if stage == "fisher_pack":
        # read X, write XT (bf16)
        return "hbm", 2 * n * d + 2 * n * d, PEAK_HBM, "GB/s", None
    return None


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path has no "
              "multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch
    import post_weight_quantization_gq_amd as gq
    from post_weight_quantization_gq_amd import synth

    dev = torch.device("cuda:0")
    if args.copy_probe:
        nbytes = 1 << 30
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": nbytes, "copy_probe_bytes_written": nbytes,
                          "copies": 3}), flush=True)
        return
    if args.path == "lut":
        run_lut(args)
        return
    if args.path == "stream":
        run_stream(args)
        return
    wl = synth.workload(args.workload or "llama2_7b_attn")
    print(f"[bench] workload {wl.name}: d_in={wl.d_in} d_out={wl.d_out} n={wl.n} "
          f"groups={wl.groups} bits={wl.bits} iters={wl.iters}",
          file=sys.stderr, flush=True)
    t0 = time.time()
    inp = synth.make_inputs(wl, seed=args.seed)

    def dv(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    X, G, W = dv(inp["X"]), dv(inp["G"]), dv(inp["W"])
    print(f"[bench] inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    F = torch.empty((wl.groups, wl.d_in, wl.d_in), dtype=torch.float32, device=dev)
    ws_f = torch.empty(max(1, gq.fisher_workspace_size(wl.n, wl.d_in, wl.d_out, wl.groups)),
                       dtype=torch.uint8, device=dev)
    ganq = args.path == "ganq"
    ws_size = (gq.ganq_workspace_size if ganq else gq.lnq_workspace_size)(
        wl.d_out, wl.d_in, wl.groups, wl.bits)
    ws_l = torch.empty(max(1, ws_size), dtype=torch.uint8, device=dev)
    C = torch.empty((wl.d_out, wl.m), dtype=torch.float32, device=dev)
    P = torch.empty((wl.d_out, wl.d_in), dtype=torch.uint8, device=dev)

    grid = args.path == "grid"

    def step():
        gq.gq_fisher_accumulate(X, G, wl.groups, F=F, ws=ws_f)
        if grid:
            return gq.grid_quantize(W, F, wl.bits, wl.iters, block=args.block, ridge_rel=1e-6,
                                    C=C, P=P, init=gq.GQ_INIT_UNIFORM, ws=ws_l)
        if ganq:
            return gq.ganq_quantize(W, F, wl.bits, wl.iters, ridge_rel=1e-6, C=C, P=P,
                                    init=gq.GQ_INIT_QUANTILE, ws=ws_l)
        return gq.lnq_quantize(W, F, wl.bits, wl.iters, block=args.block, ridge_rel=1e-6, C=C,
                               P=P, init=gq.GQ_INIT_QUANTILE, ws=ws_l)

    warm = max(1, args.warmup)
    for i in range(warm):
        if i == warm - 1:
            # the last warmup step records every stage with HIP events: that is the
            # per-stage breakdown; the timed steps below carry events for one stage only
            gq.gq_timing_read()
            gq.gq_timing_enable(True)
        step()
        torch.cuda.synchronize()
        print(f"[bench] warmup {i + 1}/{warm} done", file=sys.stderr, flush=True)
    gq.gq_timing_enable(False)
    breakdown = gq.gq_timing_read()
    per_step = {k: v[0] for k, v in breakdown.items() if v[1]}
    launches = {k: v[1] for k, v in breakdown.items() if v[1]}
    dom = max(per_step, key=per_step.get)

    # timed region: events only around the dominant stage's launches, on the stream
    # the library launches them on (the caller's current stream)
    gq.gq_timing_enable([dom])
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    outs = None
    for _ in range(args.steps):
        outs = step()
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    gq.gq_timing_enable(False)
    timed = gq.gq_timing_read()
    ms_step = (t_end - t_start) * 1e3 / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_step:.2f} ms/step", file=sys.stderr, flush=True)

    trace = outs[2].cpu().numpy()
    nchg = outs[3].cpu().numpy()
    fisher_stages = ("group_scale", "fisher_pack", "fisher_mfma", "fisher_finalize",
                     "fisher_plain")
    fisher_ms = sum(per_step.get(k, 0) for k in fisher_stages)
    lnq_ms = sum(v for k, v in per_step.items() if k.startswith("lnq"))
    sym_flops = wl.n * wl.d_in * (wl.d_in + 1) * wl.groups

    # roofline of the stage with the largest share of the step, from the events of
    # the timed region
    roof = None
    spec = _stage_units(dom, wl, nchg, grid, ganq)
    if spec is not None and timed[dom][1]:
        bound, amount, peak, unit, working = spec
        n_launch = timed[dom][1] / args.steps if working is None else working
        avg_ms = timed[dom][0] / args.steps / n_launch
        per_launch = amount / n_launch
        achieved = per_launch / (avg_ms * 1e-3)
        scale = 1e9 if unit == "GB/s" else 1e12
        roof = {"kernel": dom, "bound": bound, "achieved": achieved / scale, "peak": peak / scale,
                "unit": unit, "frac": achieved / peak, "traffic": _traffic(dom, wl),
                "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                "copy-calibrated)",
                "avg_launch_ms": avg_ms, "units_per_launch": per_launch,
                "launches_per_step": n_launch}
        if bound == "alu":
            roof["peak_note"] = ("fp32 vector: 256 CUs x 64 lanes x 2.4 GHz x 2 (FMA) = 78.6 "
                                 "TFLOP/s, the rate this build issues (packed fp32 off); the "
                                 "published packed peak is 157.3")
            roof["frac_of_packed_peak"] = achieved / PEAK_FP32_VALU_PACKED

    # every stage's fraction of its own bound, from the warm-up step's per-stage times
    stage_roof = {}
    for k, ms in per_step.items():
        sp = _stage_units(k, wl, nchg, grid, ganq)
        if sp is None or ms <= 0:
            continue
        bound, amount, peak, unit, _ = sp
        ach = amount / (ms * 1e-3)
        scale = 1e9 if unit == "GB/s" else 1e12
        stage_roof[k] = {"bound": bound, "achieved": round(ach / scale, 2), "peak": peak / scale,
                         "unit": unit, "frac": round(ach / peak, 4)}

    metric = ("Fixed-grid GuidedQuant rows quantized/s (Fisher + uniform grid + assignment "
              f"passes) at {wl.d_in}x{wl.d_out}, {wl.bits}-bit, 1 MI355X" if grid else
              "GANQ-style rows quantized/s (Fisher + Cholesky + codebook / back-substitution "
              f"alternation) at {wl.d_in}x{wl.d_out}, {wl.bits}-bit, 1 MI355X" if ganq else
              "LNQ rows quantized/s + Fisher TFLOP/s at 4096x4096, 3-bit, 1 MI355X")
    result = {
        "metric": metric,
        "value": wl.d_out / (ms_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "path": args.path, "d_in": wl.d_in, "d_out": wl.d_out,
                   "n_tokens": wl.n, "groups": wl.groups, "bits": wl.bits, "iters": wl.iters,
                   "block": args.block},
        "fisher_ms": fisher_ms,
        "fisher_ms_stages": list(k for k in fisher_stages if k in per_step),
        "fisher_tflops": sym_flops / (fisher_ms * 1e-3) / 1e12 if fisher_ms else None,
        "fisher_tflops_gemm_convention": (2 * wl.n * wl.d_in ** 2 * wl.groups) /
        (fisher_ms * 1e-3) / 1e12 if fisher_ms else None,
        "fisher_contraction_only_tflops": sym_flops / (per_step["fisher_mfma"] * 1e-3) / 1e12
        if per_step.get("fisher_mfma") else None,
        "lnq_rows_per_s": wl.d_out / (lnq_ms * 1e-3) if lnq_ms else None,
        "s_per_layer": ms_step * 1e-3,
        "stage_ms_per_step": {k: round(v, 4) for k, v in per_step.items()},
        "stage_launches_per_step": launches,
        "stage_breakdown_from": "last warmup step, every stage bracketed by HIP events",
        "changed_per_sweep": [int(x) for x in nchg],
        "codebook_steps_from_changes": [] if (grid or ganq) else _incremental_iters(wl, nchg),
        "objective_trace": [float(x) for x in trace],
        "monotone": bool(np.all(trace[1:] <= trace[:-1] * (1 + 1e-6))),
        "layer_roofline": (_grid_roofline if grid else _ganq_roofline if ganq else
                           _layer_roofline)(wl, nchg, ms_step),
        "roofline": roof,
        "stage_rooflines": stage_roof,
        "stage_rooflines_from": "last warmup step (per-stage HIP events); each stage's "
                                "algorithmic work over its time against its own bound",
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, inp, F, args)
    print(json.dumps(result), flush=True)


def run_lut(args):
    """The lookup-table product on one layer's shape: seeded random codes (uniform over
    the 2^bits entries), sorted N(0, 0.02^2) codebooks, N(0, 1) bfloat16 activations."""
    import torch
    import post_weight_quantization_gq_amd as gq
    from post_weight_quantization_gq_amd import synth
    dev = torch.device("cuda:0")
    wl = synth.workload(args.workload or "llama2_70b_down")
    B = args.lut_batch
    rng = np.random.default_rng(args.seed)
    P_np = rng.integers(0, wl.m, size=(wl.d_out, wl.d_in), dtype=np.uint8)
    C_np = np.sort(rng.standard_normal((wl.d_out, wl.m)).astype(np.float32) * np.float32(0.02),
                   axis=1)
    x_bits = synth.f32_to_bf16_bits(rng.standard_normal((B, wl.d_in)).astype(np.float32))
    P = torch.from_numpy(P_np).to(dev)
    C = torch.from_numpy(C_np).to(dev)
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    Q = gq.lut_pack_codes(P, wl.bits)
    y = torch.empty((B, wl.d_out), dtype=torch.float32, device=dev)
    R = args.lut_reps
    print(f"[bench] lut product {wl.d_in} -> {wl.d_out}, {wl.bits}-bit, batch {B}, "
          f"{R} products per step", file=sys.stderr, flush=True)

    def step():
        for _ in range(R):
            gq.lut_gemv(Q, C, x, wl.bits, y=y)

    for i in range(max(1, args.warmup)):
        step()
        torch.cuda.synchronize()
    gq.gq_timing_read()
    gq.gq_timing_enable(["lut_gemv"])
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    gq.gq_timing_enable(False)
    timed = gq.gq_timing_read()
    ms_step = (t_end - t_start) * 1e3 / args.steps
    n_launch = timed["lut_gemv"][1]
    avg_ms = timed["lut_gemv"][0] / n_launch
    packed = Q.numel() * 4
    # algorithmic bytes of one product: packed codes, codebooks, activations, outputs
    alg = packed + wl.d_out * wl.m * 4 + B * wl.d_in * 2 + B * wl.d_out * 4
    achieved = alg / (avg_ms * 1e-3)
    result = {
        "metric": f"LUT dequant GEMV packed-weight GB/s at {wl.d_in}->{wl.d_out}, {wl.bits}-bit, "
                  f"batch {B}, 1 MI355X",
        "value": packed * R / (ms_step * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "path": "lut", "d_in": wl.d_in, "d_out": wl.d_out,
                   "bits": wl.bits, "batch": B, "products_per_step": R},
        "us_per_product_wall": ms_step * 1e3 / R,
        "us_per_product_events": avg_ms * 1e3,
        "roofline": {"kernel": "lut_gemv", "bound": "hbm", "achieved": achieved / 1e9,
                     "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": achieved / PEAK_HBM,
                     "traffic": _traffic("lut_gemv", wl) if B == 1 else None,
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                     "copy-calibrated)",
                     "avg_launch_ms": avg_ms, "units_per_launch": alg,
                     "launches_per_step": n_launch / args.steps},
    }
    if not args.no_cpu_baseline:
        import oracle as O
        rows = min(wl.d_out, 512)
        x64 = synth.bf16_bits_to_f32(x_bits).astype(np.float64)
        t0 = time.perf_counter()
        O.lut_gemv(C_np[:rows], P_np[:rows], x64, True)
        t = (time.perf_counter() - t0) * wl.d_out / rows
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:  # pragma: no cover
            cores = 1
        result["cpu_baseline"] = {"value": packed / t / 1e9, "unit": "GB/s", "cores": cores,
                                  "kind": "oracle",
                                  "sample": f"oracle product on the first {rows} of {wl.d_out} "
                                            f"rows ({t * rows / wl.d_out:.2f}s measured, "
                                            f"scaled to the layer)"}
    print(json.dumps(result), flush=True)


def run_stream(args):
    """The Fisher of one layer's calibration data held in pinned host memory."""
    import torch
    import post_weight_quantization_gq_amd as gq
    from post_weight_quantization_gq_amd import synth
    dev = torch.device("cuda:0")
    wl = synth.workload(args.workload or "llama2_7b_attn")
    t0 = time.time()
    inp = synth.make_inputs(wl, seed=args.seed, want=("X", "G"))

    def host(a):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 \
            else torch.from_numpy(a)
        return t.pin_memory()

    X, G = host(inp["X"]), host(inp["G"])
    del inp
    print(f"[bench] pinned host inputs ready in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)
    T = args.chunk_tokens
    F = torch.empty((wl.groups, wl.d_in, wl.d_in), dtype=torch.float32, device=dev)
    ws = torch.empty(gq.fisher_stream_workspace_size(min(T, wl.n), wl.d_in, wl.d_out, wl.groups),
                     dtype=torch.uint8, device=dev)

    def step():
        gq.gq_fisher_accumulate_host(X, G, wl.groups, F=F, chunk_tokens=T, ws=ws)

    warm = max(1, args.warmup)
    for i in range(warm):
        if i == warm - 1:
            gq.gq_timing_read()
            gq.gq_timing_enable(True)
        step()
        torch.cuda.synchronize()
    gq.gq_timing_enable(False)
    per_step = {k: v[0] for k, v in gq.gq_timing_read().items() if v[1]}
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t_start) * 1e3 / args.steps
    host_bytes = X.numel() * X.element_size() + G.numel() * G.element_size()
    achieved = host_bytes / (ms_step * 1e-3)
    result = {
        "metric": f"Host-streamed Fisher tokens/s at {wl.d_in}x{wl.d_out}, {wl.n} tokens "
                  f"(X, G in pinned host memory), 1 MI355X",
        "value": wl.n / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "path": "stream", "d_in": wl.d_in, "d_out": wl.d_out,
                   "n_tokens": wl.n, "groups": wl.groups, "chunk_tokens": T},
        "stage_ms_per_step": {k: round(v, 4) for k, v in per_step.items()},
        "stage_breakdown_from": "last warmup step; fisher_h2d is timed on the copy stream",
        "roofline": {"kernel": "host-to-device copies", "bound": "pcie",
                     "achieved": achieved / 1e9, "peak": PEAK_PCIE / 1e9, "unit": "GB/s",
                     "frac": achieved / PEAK_PCIE, "traffic": None,
                     "units_per_launch": host_bytes, "launches_per_step": 1},
    }
    print(json.dumps(result), flush=True)


def _cpu_info():
    info = {"os_cpu_count": os.cpu_count()}
    try:
        info["affinity"] = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        info["affinity"] = info["os_cpu_count"]
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return info


def _oracle_row_worker(args):
    """One row of the oracle in a worker process (spawned, single-threaded BLAS; F'
    memory-mapped from the file the parent wrote).  Returns the row's seconds."""
    path, w, m, iters, kind = args
    import oracle as O
    Fp = np.load(path, mmap_mode="r")
    fn = {"grid": O.grid_row, "ganq": O.ganq_row}.get(kind, O.lnq_row)
    t0 = time.perf_counter()
    fn(Fp, w, m, iters)
    return time.perf_counter() - t0


def cpu_baseline(wl, inp, F, args):
    """Time the fp64 oracle on a bounded sample of the same layer, scaled to rows/s.

    Fisher leg: the oracle's float64 Fisher of the first --cpu-tokens tokens (numpy's
    matmul on the host's BLAS threads), scaled to all tokens (the Fisher is a sum over
    tokens).  LNQ leg: --cpu-rows rows of group 0 (rows are independent given F'_g),
    one row per worker process at a time over min(16, host cores) spawned workers, each
    on one BLAS thread; the sample's wall time is scaled to all rows."""
    import multiprocessing as mp
    import shutil
    import tempfile
    import oracle as O
    from post_weight_quantization_gq_amd import synth
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    info = _cpu_info()
    workers = max(1, min(16, info["affinity"]))
    print("[bench] cpu baseline: oracle Fisher on a token sample", file=sys.stderr, flush=True)
    nt = min(args.cpu_tokens, wl.n)
    Xs = synth.decode(inp["X"][:nt])
    Gs = synth.decode(inp["G"][:nt])
    t0 = time.perf_counter()
    O.fisher(Xs, Gs, wl.groups)
    t_f_meas = time.perf_counter() - t0
    t_f = t_f_meas * (wl.n / nt)
    del Xs, Gs
    rows = min(args.cpu_rows, wl.d_out // wl.groups)
    print(f"[bench] cpu baseline: oracle {args.path} on {rows} rows over {workers} worker "
          f"processes", file=sys.stderr, flush=True)
    Fp = O.damped(F[0].cpu().double().numpy(), 1e-6)
    base = "/dev/shm" if os.path.isdir("/dev/shm") and \
        shutil.disk_usage("/dev/shm").free > 2 * Fp.nbytes + (64 << 20) else None
    tmp = tempfile.mkdtemp(prefix="gq_bench_", dir=base)
    try:
        path = os.path.join(tmp, "Fp.npy")
        np.save(path, Fp)
        del Fp
        w = synth.decode(inp["W"][:rows])
        saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS")}
        for k in saved:
            os.environ[k] = "1"
        try:
            pool = mp.get_context("spawn").Pool(workers)
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
        with pool:
            pool.map(_oracle_row_worker, [(path, w[0], wl.m, 0, args.path)] * workers)  # warm
            t0 = time.perf_counter()
            per_row = pool.map(_oracle_row_worker,
                               [(path, w[j], wl.m, wl.iters, args.path) for j in range(rows)])
            t_rows = time.perf_counter() - t0
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    t_lnq = t_rows * wl.d_out / rows
    t_layer = t_f + t_lnq
    return {"value": wl.d_out / t_layer, "unit": "rows/s", "cores": max(workers, blas_threads),
            "kind": "oracle",
            "sample": f"Fisher on the first {nt} of {wl.n} tokens ({t_f_meas:.1f}s measured on "
                      f"{blas_threads} BLAS threads, scaled x{wl.n / nt:g}) + {args.path} on "
                      f"{rows} rows of group 0 ({t_rows:.1f}s wall over {workers} worker "
                      f"processes, {float(np.mean(per_row)):.2f}s per row on one core, scaled "
                      f"to {wl.d_out} rows)",
            "fisher_cores": blas_threads, "lnq_workers": workers, "lnq_rows": rows,
            "fisher_s_est": t_f, "lnq_s_est": t_lnq, "lnq_s_per_row_one_core":
            float(np.mean(per_row)), **info}


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the GEMM hot path on one MI355X.

A step is one pass of the hot path over the two headline workloads, with all
inputs resident in HBM before timing starts:
  * gemm_f32          M = N = K = 4096, A, B ~ normal(0, 1)      (seed 1005)
  * gemm_f16_f32acc   M = N = K = 8192, A, B ~ uniform[-1, 1) -> binary16 (seed 1006)
Throughput is 2MNK per step over the step time, in TFLOP/s.  Each kernel is
also timed on its own, with HIP events recorded on the stream it runs on,
and compared with the matrix peak of its input type.

Prints ONE JSON line (rank 0; this benchmark runs on one GPU only).

  python bench.py [--steps K] [--warmup W] [--only f32|f16|bf16|e4m3|e5m2|i8]
                  [--ladder | --no-ladder] [--no-cpu-baseline] [--copy-calibration]

--only times one workload instead of the two-kernel step: the two headline
ones, or the 8192^3 workloads of the BF16, FP8 (E4M3, E5M2) and INT8 entry
points (2MNK integer operations per second for INT8).

Unless --no-all-workloads is given, every named workload (the BF16, FP8 and
INT8 entry points included) is then timed on its own under "all_workloads",
every input format at 2048^3 under "mid_sizes", the convolution workloads
under "conv_workloads", and every kernel variant
(rung) at 1024^3 and 4096^3 FP32 and 8192^3 FP16 under "ladder" (a few
seconds; --no-ladder skips it, --ladder adds it to any run); --conv-only
times just the convolutions.
--copy-calibration runs a plain device-to-device copy of known size first;
used only by the hardware-counter runs that calibrate HBM byte counts.

After the timed region each headline kernel (and the whole step) is also run
back to back for a couple of seconds ("sustained") while a child process
samples the GPU's clock and socket power through the amdsmi library; the
medians go into "sustained" (the clock a power-capped kernel settles at is
what its throughput follows).  With the FP16 kernel in the step, the
matrix-core ceiling is measured the same way: a calibration kernel (its own
library) that issues the FP16 tile's MFMA stream on the workload's operand
values held in registers, with no memory traffic; "f16_frac_of_mfma_ceiling"
is the GEMM's sustained rate over it.  --no-sustained skips all of this.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s (2MNK/t) at FP32 4096³ and FP16-in 8192³; % of matrix peak"
# MI355X dense matrix peaks (TFLOP/s, TOP/s for INT8): 1024 SIMDs at 2.4 GHz
# doing 64 FP32, 1024 16-bit or 2048 8-bit multiply-adds' worth of flops a clock
PEAK_TFLOPS = {"f32": 157.3, "f16": 2516.6, "bf16": 2516.6, "e4m3": 5033.2, "e5m2": 5033.2, "i8": 5033.2}
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
_COMMON = ["dense_gemm_optimisation_row_amd/csrc/common.h", "dense_gemm_optimisation_row_amd/csrc/lds_dma.h"]
KERNEL_SOURCES = {
    "f32": ["dense_gemm_optimisation_row_amd/csrc/mfma_f32.hip"] + _COMMON,
    "f16": ["dense_gemm_optimisation_row_amd/csrc/mfma_f16.hip"] + _COMMON,
    "bf16": ["dense_gemm_optimisation_row_amd/csrc/mfma_f16.hip"] + _COMMON,
    "e4m3": ["dense_gemm_optimisation_row_amd/csrc/mfma_8bit.hip"] + _COMMON,
    "e5m2": ["dense_gemm_optimisation_row_amd/csrc/mfma_8bit.hip"] + _COMMON,
    "i8": ["dense_gemm_optimisation_row_amd/csrc/mfma_8bit.hip"] + _COMMON,
}
# the workload each format is timed on
KIND_WORKLOAD = {"f32": "f32_4096", "f16": "f16_8192", "bf16": "bf16_8192", "e4m3": "e4m3_8192",
                 "e5m2": "e5m2_8192", "i8": "i8_8192"}
KIND_DTYPE = {"f32": "f32", "f16": "f16-in/f32-acc", "bf16": "bf16-in/f32-acc", "e4m3": "fp8e4m3-in/f32-acc",
              "e5m2": "fp8e5m2-in/f32-acc", "i8": "i8-in/i32-acc"}
KIND_LABEL = {"f32": "FP32 GEMM 4096x4096x4096 row-major",
              "f16": "FP16-in/FP32-acc GEMM 8192x8192x8192 row-major",
              "bf16": "BF16-in/FP32-acc GEMM 8192x8192x8192 row-major",
              "e4m3": "FP8 E4M3-in/FP32-acc GEMM 8192x8192x8192 row-major",
              "e5m2": "FP8 E5M2-in/FP32-acc GEMM 8192x8192x8192 row-major",
              "i8": "INT8-in/INT32-acc GEMM 8192x8192x8192 row-major"}


def entry_point(dg, kind):
    return {"f32": dg.gemm_f32, "f16": dg.gemm_f16_f32acc, "bf16": dg.gemm_bf16_f32acc,
            "e4m3": dg.gemm_e4m3_f32acc, "e5m2": dg.gemm_e5m2_f32acc, "i8": dg.gemm_i8_i32acc}[kind]


def to_device(torch, np, A, kind, dev):
    """numpy operand of a format -> device tensor of the entry point's dtype."""
    if kind == "bf16":      # uint16 bit patterns
        return torch.from_numpy(A.view(np.int16)).view(torch.bfloat16).to(dev)
    if kind in ("e4m3", "e5m2"):   # uint8 codes
        return torch.from_numpy(A).to(dev).view(torch.float8_e4m3fn if kind == "e4m3" else torch.float8_e5m2)
    return torch.from_numpy(A).to(dev)


def kernel_source_hash(kind: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kind: str, launches_per_kernel: int = 1):
    """HBM bytes per launch from the committed counter summary, or None when
    it is missing or was taken on a different kernel source."""
    path = os.path.join(PROFILES, f"traffic_{kind}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        m = re.match(r"\s*([a-z_0-9]+)\s*[:=]\s*(\S+)", line)
        if m:
            vals[m.group(1)] = m.group(2)
    if vals.get("kernel_source_sha256_16") != kernel_source_hash(kind):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"]) * launches_per_kernel
    except (KeyError, ValueError):
        return None


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", choices=["all", "f32", "f16", "bf16", "e4m3", "e5m2", "i8"], default="all")
    ap.add_argument("--ladder", action="store_true", help="time every rung even without the all-workloads leg")
    ap.add_argument("--no-ladder", action="store_true", help="skip timing every rung after the all-workloads leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target host time of the CPU-baseline sample")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-all-workloads", action="store_true",
                    help="skip timing the smaller parity workloads after the main run")
    ap.add_argument("--conv-only", action="store_true",
                    help="time only the convolution workloads (for kernel traces of the im2col path)")
    ap.add_argument("--no-sustained", action="store_true",
                    help="skip the sustained runs with clock and power sampling")
    ap.add_argument("--sustained-seconds", type=float, default=2.0)
    ap.add_argument("--smi-sampler", type=float, default=0.0, help=argparse.SUPPRESS)
    args = ap.parse_args()

    if args.smi_sampler > 0:
        return smi_sampler(args.smi_sampler)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the GEMM path here is single-GPU "
              "(no collectives); run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import dense_gemm_optimisation_row_amd as dg
    from dense_gemm_optimisation_row_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dg.binding.load()   # fail loudly if the HIP library is missing
    stream = torch.cuda.current_stream(dev)

    if args.conv_only:
        print(json.dumps({"conv_workloads": conv_workloads(dg, inputs, torch, dev, stream)}), flush=True)
        return 0

    if args.copy_calibration:
        # plain copy of known size, for scaling HBM byte counters
        src = torch.empty(256 * 2 ** 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    kinds = ["f32", "f16"] if args.only == "all" else [args.only]
    wl = {k: inputs.WORKLOADS[KIND_WORKLOAD[k]] for k in kinds}
    dev_in = {}
    for k in kinds:
        A, B = inputs.workload_matrices(wl[k])
        a = to_device(torch, np, A, k, dev)
        b = to_device(torch, np, B, k, dev)
        c = torch.empty((wl[k].M, wl[k].N), dtype=torch.int32 if k == "i8" else torch.float32, device=dev)
        dev_in[k] = (a, b, c)
        del A, B
    torch.cuda.synchronize()

    def call(k):
        a, b, c = dev_in[k]
        entry_point(dg, k)(a, b, c, stream=stream)

    for _ in range(args.warmup):
        for k in kinds:
            call(k)
    torch.cuda.synchronize()

    # timed region: K whole steps, each kernel bracketed by events on its stream
    ev = {k: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)] for k in kinds}
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(args.steps):
        for k in kinds:
            ev[k][s][0].record(stream)
            call(k)
            ev[k][s][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    flops_step = sum(wl[k].flops for k in kinds)
    value = flops_step / (ms_per_step * 1e-3) / 1e12

    per = {}
    for k in kinds:
        ms = [a.elapsed_time(b) for a, b in ev[k]]
        avg = float(np.mean(ms))
        tf = wl[k].flops / (avg * 1e-3) / 1e12
        a, b, c = dev_in[k]
        in_bytes = (a.numel() + b.numel()) * a.element_size()
        per[k] = {
            "workload": wl[k].name, "M": wl[k].M, "N": wl[k].N, "K": wl[k].K,
            "kernel": dg.variant_name(dg.plan(k, wl[k].M, wl[k].N, wl[k].K)["variant"]),
            "avg_ms": round(avg, 5), "min_ms": round(float(np.min(ms)), 5),
            "tflops": round(tf, 2), "peak_tflops": PEAK_TFLOPS[k],
            "frac_of_peak": round(tf / PEAK_TFLOPS[k], 4),
            "algorithmic_bytes": in_bytes + c.numel() * 4,
        }

    dom = max(kinds, key=lambda k: per[k]["avg_ms"])
    roofline = {
        "kernel": per[dom]["kernel"], "workload": per[dom]["workload"],
        "bound": "mfma", "achieved": per[dom]["tflops"], "peak": PEAK_TFLOPS[dom],
        "unit": "TOP/s" if dom == "i8" else "TFLOP/s", "frac": per[dom]["frac_of_peak"],
        "traffic": read_traffic(dom),
        "algorithmic_flops": wl[dom].flops, "algorithmic_bytes": per[dom]["algorithmic_bytes"],
    }
    others = [
        {"kernel": per[k]["kernel"], "workload": per[k]["workload"], "bound": "mfma",
         "achieved": per[k]["tflops"], "peak": PEAK_TFLOPS[k], "unit": "TFLOP/s",
         "frac": per[k]["frac_of_peak"], "traffic": read_traffic(k)}
        for k in kinds if k != dom]

    unit = "TOP/s" if kinds == ["i8"] else "TFLOP/s"
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "+".join(KIND_DTYPE[k] for k in kinds),
        "data": "synthetic (seeded numpy PCG64: normal(0,1) f32 4096^3; uniform[-1,1) "
                "rounded to the input format, 8192^3)",
        "config": {"workload": " + ".join(KIND_LABEL[k] for k in kinds),
            "per_step": [wl[k].name for k in kinds]},
        "per_workload": per,
        "roofline": roofline,
        "roofline_other": others,
        "device": torch.cuda.get_device_name(dev),
    }

    if not args.no_all_workloads:
        out["all_workloads"] = all_workloads(dg, inputs, torch, dev, stream, dev_in, wl)
        out["mid_sizes"] = mid_sizes(dg, inputs, torch, dev, stream)
        out["conv_workloads"] = conv_workloads(dg, inputs, torch, dev, stream)

    if not args.no_sustained:
        calls, flops = {}, {}
        for k in kinds:
            calls[k], flops[k] = (lambda k=k: call(k)), wl[k].flops
            if k == "f16":
                # the matrix-core ceiling of the same tile stream on the same
                # inputs (calibration kernel: MFMAs only, operands held in
                # registers), right after the GEMM, under the same power limit
                ceil_fn = mfma_f16_ceiling_call(dev_in["f16"], wl["f16"], torch, stream)
                if ceil_fn is not None:
                    calls["f16_mfma_ceiling"], flops["f16_mfma_ceiling"] = ceil_fn, wl[k].flops
        if len(kinds) > 1:
            calls["step"], flops["step"] = (lambda: [call(k) for k in kinds]), flops_step
        out["sustained"] = sustained(calls, flops, torch, args.sustained_seconds)
        if "f16_mfma_ceiling" in out["sustained"] and "f16" in out["sustained"]:
            g, c = out["sustained"]["f16"], out["sustained"]["f16_mfma_ceiling"]
            if "tflops" in g and "tflops" in c:
                out["sustained"]["f16_frac_of_mfma_ceiling"] = round(g["tflops"] / c["tflops"], 4)

    if args.ladder or not (args.no_ladder or args.no_all_workloads):
        out["ladder"] = ladder(dg, inputs, torch, dev, stream)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(kinds, wl, args.cpu_seconds)

    print(json.dumps(out), flush=True)
    return 0


def _time_calls(fn, torch, stream, reps):
    fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _settled_time(fn, torch, stream, budget_ms=100.0, max_reps=5000):
    """Milliseconds per call of ``fn``, back to back, after about 30 ms of
    untimed calls: a short call that follows host-side work (input
    generation) otherwise starts on a clock still rising from idle, and a
    few milliseconds of timed calls would include the ramp."""
    est = _time_calls(fn, torch, stream, 3)
    _time_calls(fn, torch, stream, max(1, min(max_reps, int(30.0 / max(est, 1e-3)))))
    reps = max(3, min(max_reps, int(budget_ms / max(est, 1e-3))))
    return _time_calls(fn, torch, stream, reps)


def _time_cold(fn, torch, stream, flush, reps):
    """Milliseconds per call of ``fn`` with the caches cold: before each call
    a fill of ``flush`` (larger than the memory-side cache and every L2
    together) evicts the operands, and only the call itself lies between the
    events."""
    total = 0.0
    for i in range(reps):
        with torch.cuda.stream(stream):
            flush.fill_(i & 0xff)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        total += e0.elapsed_time(e1)
    return total / reps


def all_workloads(dg, inputs, torch, dev, stream, dev_in, wl):
    """2MNK/t and fraction of the matrix peak for every workload, each timed
    on its own after the main timed region (the headline ones reuse their
    resident inputs).  Calls of at least 0.1 ms are also timed with the
    caches cold (their operands, 128 to 384 MiB, are about the size of the
    256 MB memory-side cache, so warm back-to-back calls may be served from
    it)."""
    import numpy as np

    res = {}
    flush = None
    for name, w in inputs.WORKLOADS.items():
        kind = w.dtype
        if wl.get(kind) is not None and wl[kind].name == name and kind in dev_in:
            a, b, c = dev_in[kind]
        else:
            A, B = inputs.workload_matrices(w)
            a, b = to_device(torch, np, A, kind, dev), to_device(torch, np, B, kind, dev)
            c = torch.empty((w.M, w.N), dtype=torch.int32 if kind == "i8" else torch.float32, device=dev)
            del A, B
        f = entry_point(dg, kind)
        ms = _settled_time(lambda: f(a, b, c, stream), torch, stream)
        tf = w.flops / (ms * 1e-3) / 1e12
        p = dg.plan(kind, w.M, w.N, w.K)
        # algorithmic bytes: each input read once, C (4-byte elements) written once
        nbytes = (w.M * w.K + w.K * w.N) * a.element_size() + 4 * w.M * w.N
        gbs = nbytes / (ms * 1e-3) / 1e9
        # the roofline's bound: HBM when the arithmetic intensity is below the ridge
        bound = "hbm" if w.flops / nbytes < PEAK_TFLOPS[kind] * 1e12 / (HBM_PEAK_GBS * 1e9) else "mfma"
        res[name] = {"M": w.M, "N": w.N, "K": w.K, "dtype": w.dtype, "ms": round(ms, 5),
                     "tflops": round(tf, 3), "frac_of_peak": round(tf / PEAK_TFLOPS[kind], 4),
                     "algorithmic_bytes": nbytes, "achieved_gbs": round(gbs, 1),
                     "frac_of_hbm": round(gbs / HBM_PEAK_GBS, 4), "bound": bound,
                     "kernel": dg.variant_name(p["variant"]), "tile": [p["tile_m"], p["tile_n"]]}
        if ms >= 0.1:
            if flush is None:
                flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)   # 1 GiB
            cms = _time_cold(lambda: f(a, b, c, stream), torch, stream, flush, 10)
            ctf = w.flops / (cms * 1e-3) / 1e12
            res[name].update({"ms_cold": round(cms, 5), "tflops_cold": round(ctf, 3),
                              "frac_of_peak_cold": round(ctf / PEAK_TFLOPS[kind], 4)})
        if ms < 0.1:
            # short calls: also timed as a replayed HIP graph of back-to-back
            # calls, which takes the host's per-call launch cost out
            g = graph_time(lambda: f(a, b, c), torch, c)
            if g is not None:
                gms, same = g
                gtf = w.flops / (gms * 1e-3) / 1e12
                ggbs = nbytes / (gms * 1e-3) / 1e9
                res[name].update({"ms_graph": round(gms, 5), "tflops_graph": round(gtf, 3),
                                  "frac_of_peak_graph": round(gtf / PEAK_TFLOPS[kind], 4),
                                  "achieved_gbs_graph": round(ggbs, 1),
                                  "frac_of_hbm_graph": round(ggbs / HBM_PEAK_GBS, 4),
                                  "graph_matches_eager": same})
    del flush
    return res


# mid-size products, where the tile choice sets how many compute units work:
# every input format at 2048^3 (64 tiles of 256^2, 256 of 128^2)
MID_SIZES = [(2048, 2048, 2048)]


def mid_sizes(dg, inputs, torch, dev, stream):
    """2MNK/t, fraction of the matrix peak and the planned tile of every
    input format at the MID_SIZES shapes (uniform[-1, 1) inputs rounded to the
    format, seed 3000), calls timed back to back."""
    import numpy as np

    res = {}
    for M, N, K in MID_SIZES:
        for kind in ("f32", "f16", "bf16", "e4m3", "e5m2", "i8"):
            A, B = inputs.matrices(M, N, K, 3000, "uniform", kind)
            a, b = to_device(torch, np, A, kind, dev), to_device(torch, np, B, kind, dev)
            c = torch.empty((M, N), dtype=torch.int32 if kind == "i8" else torch.float32, device=dev)
            f = entry_point(dg, kind)
            ms = _settled_time(lambda: f(a, b, c, stream), torch, stream, budget_ms=50.0)
            tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
            p = dg.plan(kind, M, N, K)
            res[f"{kind}_{M}x{N}x{K}"] = {"ms": round(ms, 5), "tflops": round(tf, 3),
                                          "frac_of_peak": round(tf / PEAK_TFLOPS[kind], 4),
                                          "kernel": dg.variant_name(p["variant"]),
                                          "tile": [p["tile_m"], p["tile_n"]]}
            del a, b, c
    return res


def graph_time(fn, torch, out, calls=20, replays=20):
    """Milliseconds per call of ``fn`` captured ``calls`` times in one HIP
    graph and replayed ``replays`` times (after one warm-up replay), and
    whether ``out`` after the replays equals ``out`` after an eager call
    (every replay is compared, with eager calls between them).  None when
    the capture fails."""
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        ref = out.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(calls):
                fn()
        same = True
        for _ in range(3):
            out.zero_()
            g.replay()
            torch.cuda.synchronize()
            same = same and bool(torch.equal(out, ref))
            fn()
            torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        g.replay()
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        same = same and bool(torch.equal(out, ref))
        ms = e0.elapsed_time(e1) / (replays * calls)
        del g
        return ms, same
    except Exception as e:   # report no graph figure rather than fail the run
        print(f"# graph timing skipped: {e}", file=sys.stderr, flush=True)
        torch.cuda.synchronize()
        return None


def conv_workloads(dg, inputs, torch, dev, stream):
    """Convolutions (im2col + GEMM, or for 16-bit layers with enough tiles an
    implicit GEMM: on a channels-last copy of x when C is a multiple of 32,
    else gathering from x): 2 N K P Q C R S per call over the whole call,
    workspace allocated once."""
    import numpy as np

    res = {}
    for name, w in inputs.CONV_WORKLOADS.items():
        x, wt = inputs.conv_tensors(w)
        xd, wd = to_device(torch, np, x, w.dtype, dev), to_device(torch, np, wt, w.dtype, dev)
        P, Q = w.out_hw
        y = torch.empty((w.N, w.K, P, Q), dtype=torch.float32, device=dev)
        prm = dg.conv_params(w.N, w.C, w.H, w.W, w.K, w.R, w.S, (w.stride, w.stride), (w.pad, w.pad))
        ws = torch.empty(dg.conv2d_workspace(prm, xd.element_size()), dtype=torch.uint8, device=dev)
        f = lambda: dg.conv2d(w.dtype, xd, wd, (w.stride, w.stride), (w.pad, w.pad), y=y, workspace=ws,
                              stream=stream)
        ms = _settled_time(f, torch, stream)
        tf = w.flops / (ms * 1e-3) / 1e12
        alg = dg.conv2d_algorithm(prm, xd.element_size())
        if alg == dg.CONV_IMPLICIT_NHWC:
            name_alg, tile = "implicit_gemm_channels_last", [64, 256] if w.K <= 64 else [128, 64]
        elif alg == dg.CONV_IMPLICIT:
            name_alg, tile = "implicit_gemm", [128 if w.K > 64 else 64, 256]
        else:
            gp = dg.plan(w.dtype, w.K, -(-w.N * P * Q // 8) * 8, -(-w.C * w.R * w.S // 8) * 8)
            name_alg, tile = "im2col_gemm", [gp["tile_m"], gp["tile_n"]]
        res[name] = {"N": w.N, "C": w.C, "H": w.H, "W": w.W, "K": w.K, "R": w.R, "S": w.S,
                     "stride": w.stride, "pad": w.pad, "dtype": w.dtype, "ms": round(ms, 5),
                     "tflops": round(tf, 3), "frac_of_peak": round(tf / PEAK_TFLOPS[w.dtype], 4),
                     "gemm": [w.K, w.N * P * Q, w.C * w.R * w.S],
                     "algorithm": name_alg, "gemm_tile": tile,
                     "workspace_bytes": int(ws.numel())}
        del xd, wd, y, ws
    return res


def ladder(dg, inputs, torch, dev, stream):
    """Time every rung on the workloads (same inputs as the step)."""
    res = []
    for name, variants in (("f32_1024", dg.F32_VARIANTS), ("f32_4096", dg.F32_VARIANTS),
                           ("f16_8192", dg.F16_VARIANTS)):
        w = inputs.WORKLOADS[name]
        A, B = inputs.workload_matrices(w)
        a, b = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
        c = torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
        half = w.dtype == "f16"
        for v in variants:
            f = dg.gemm_f16_f32acc_variant if half else dg.gemm_f32_variant
            est = _time_calls(lambda: f(v, a, b, c, stream), torch, stream, 1)
            reps = max(1, min(50, int(200.0 / max(est, 1e-3))))
            ms = _time_calls(lambda: f(v, a, b, c, stream), torch, stream, reps)
            tf = w.flops / (ms * 1e-3) / 1e12
            res.append({"workload": name, "variant": dg.variant_name(v), "ms": round(ms, 4),
                        "tflops": round(tf, 3),
                        "frac_of_peak": round(tf / PEAK_TFLOPS["f16" if half else "f32"], 4)})
            print(f"# ladder {name} {dg.variant_name(v)}: {ms:.3f} ms {tf:.2f} TFLOP/s",
                  file=sys.stderr, flush=True)
        del a, b, c
    return res


def mfma_f16_ceiling_call(dev_in, w, torch, stream):
    """A callable that runs the matrix-core rate calibration kernel (its own
    library, libdgor_calibrate.so) on the FP16 workload's inputs, or None if
    that library was not built."""
    import ctypes

    path = os.path.join(ROOT, "dense_gemm_optimisation_row_amd", "libdgor_calibrate.so")
    if not os.path.exists(path):
        print(f"# {path} missing: no matrix-core ceiling", file=sys.stderr, flush=True)
        return None
    lib = ctypes.CDLL(path)
    f = lib.dgor_calibrate_mfma_f16
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 3 + [ctypes.c_void_p]
    f.restype = ctypes.c_int
    a, b, _ = dev_in
    c = torch.empty((w.M, w.N), dtype=torch.float32, device=a.device)
    h = int(stream.cuda_stream)

    def run():
        rc = f(a.data_ptr(), b.data_ptr(), c.data_ptr(), w.M, w.N, w.K, h)
        if rc != 0:
            raise RuntimeError(f"calibration kernel launch failed ({rc})")
    return run


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(kinds, wl, seconds):
    """The oracle as it stands, on the host's cores: every workload of the
    step in full when that fits about ``seconds`` of host time (it does for
    the default step: about 1.5 s for FP32 4096^3 and 10 s for FP16-in
    8192^3 on 16 threads), else on a leading block of rows; plus one thread
    on FP32 1024^3 for a per-core figure."""
    import numpy as np

    import oracle
    from dense_gemm_optimisation_row_amd import inputs

    threads = oracle.threads(0)
    fns = {"f32": oracle.gemm_f32, "f16": oracle.gemm_f16, "bf16": oracle.gemm_bf16,
           "e4m3": oracle.gemm_e4m3, "e5m2": oracle.gemm_e5m2, "i8": oracle.gemm_i8}
    rates = {}
    samples = []
    full_s = {}
    budget = 2.5 * seconds / len(kinds)
    for k in kinds:
        w = wl[k]
        A, B = inputs.workload_matrices(w)
        fn = fns[k]
        rows = max(threads, 8)
        t0 = time.perf_counter()
        fn(A[:rows], B)
        dt = time.perf_counter() - t0
        rows2 = w.M if dt * w.M / rows <= budget else int(max(rows, rows * budget / max(dt, 1e-3)))
        t0 = time.perf_counter()
        fn(A[:rows2], B)
        dt = time.perf_counter() - t0
        rates[k] = 2.0 * rows2 * w.N * w.K / dt        # flop/s
        if rows2 == w.M:
            full_s[w.name] = round(dt, 3)
            samples.append(f"all {w.M} rows of {w.name} ({dt:.1f} s)")
        else:
            samples.append(f"{rows2} of {w.M} rows of {w.name} ({dt:.1f} s)")
        del A, B
    # per core: one thread on the pages' size (FP32 1024^3)
    w1 = inputs.WORKLOADS["f32_1024"]
    A, B = inputs.workload_matrices(w1)
    t0 = time.perf_counter()
    oracle.gemm_f32(A, B, nthreads=1)
    dt1 = time.perf_counter() - t0
    step_flops = sum(wl[k].flops for k in kinds)
    step_seconds = sum(wl[k].flops / rates[k] for k in kinds)
    return {"value": round(step_flops / step_seconds / 1e12, 6), "unit": "TFLOP/s",
            "cores": threads, "kind": "oracle",
            "sample": "; ".join(samples) + " (FP64-accumulating C loop nest, OpenMP over rows)",
            "cpu_model": cpu_model(),
            "step_seconds": round(step_seconds, 3),
            "full_seconds": full_s,
            "per_workload_gflops": {wl[k].name: round(rates[k] / 1e9, 3) for k in kinds},
            "one_thread_f32_1024": {"seconds": round(dt1, 3), "gflops_per_core": round(w1.flops / dt1 / 1e9, 3)}}


def smi_sampler(period: float) -> int:
    """Child-process loop: one JSON line of GPU 0's clocks and power every
    ``period`` seconds, read through the amdsmi library, until killed."""
    import amdsmi

    amdsmi.amdsmi_init()
    h = amdsmi.amdsmi_get_processor_handles()[0]

    def num(v):
        return v if isinstance(v, (int, float)) else None

    while True:
        rec = {"t": time.time()}
        try:
            m = amdsmi.amdsmi_get_gpu_metrics_info(h)
            clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and 0 < c < 10000]
            rec["sclk_mhz"] = sum(clks) / len(clks) if clks else num(m.get("current_gfxclk"))
            rec["power_w"] = num(m.get("current_socket_power"))
            rec["energy"] = num(m.get("energy_accumulator"))
            rec["ppt_acc"] = num(m.get("ppt_residency_acc"))
            rec["acc_counter"] = num(m.get("accumulation_counter"))
            rec["hotspot_c"] = num(m.get("temperature_hotspot"))
        except Exception as e:   # report, keep sampling
            rec["error"] = str(e)[:200]
        print(json.dumps(rec), flush=True)
        time.sleep(period)


def sustained(calls, flops, torch, seconds):
    """Each call run back to back for ``seconds`` while a child process samples
    the GPU clock and socket power; returns per call the mean time per call
    and the medians of the samples taken in the second half of the run (after
    the clock has settled), plus the fraction of that time the power limit
    was holding the clock down (the firmware's PPT residency counter)."""
    import statistics
    import subprocess
    import threading

    proc = subprocess.Popen([sys.executable, os.path.abspath(__file__), "--smi-sampler", "0.02"],
                            stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
    lines = []
    first = threading.Event()

    def reader():
        for ln in proc.stdout:
            try:
                lines.append(json.loads(ln))
            except ValueError:
                continue
            first.set()

    th = threading.Thread(target=reader, daemon=True)
    th.start()
    res = {}
    try:
        if not first.wait(30.0):
            return {"error": "amdsmi sampler produced no sample"}
        for name, fn in calls.items():
            fn()
            torch.cuda.synchronize()
            t_begin = time.time()
            n = 0
            t_half = None
            while time.time() - t_begin < seconds:
                for _ in range(10):
                    fn()
                n += 10
                torch.cuda.synchronize()
                if t_half is None and time.time() - t_begin >= seconds / 2:
                    t_half = (time.time(), n)
            t_end = time.time()
            ms = (t_end - t_half[0]) / max(1, n - t_half[1]) * 1e3
            win = [r for r in lines if t_half[0] <= r["t"] <= t_end and "error" not in r]
            rec = {"ms_per_call": round(ms, 5), "tflops": round(flops[name] / (ms * 1e-3) / 1e12, 2),
                   "samples": len(win)}
            vals = lambda key: [r[key] for r in win if r.get(key) is not None]
            if vals("sclk_mhz"):
                rec["sclk_mhz"] = round(statistics.median(vals("sclk_mhz")), 1)
            if vals("power_w"):
                rec["socket_power_w"] = round(statistics.median(vals("power_w")), 1)
            ok = [r for r in win if r.get("ppt_acc") is not None and r.get("acc_counter") is not None]
            if len(ok) >= 2 and ok[-1]["acc_counter"] > ok[0]["acc_counter"]:
                rec["power_limited_frac"] = round((ok[-1]["ppt_acc"] - ok[0]["ppt_acc"]) /
                                                  (ok[-1]["acc_counter"] - ok[0]["acc_counter"]), 3)
            hs = vals("hotspot_c")
            if hs:
                rec["hotspot_c"] = max(hs)
            res[name] = rec
    finally:
        proc.kill()
        proc.wait()
    return res


if __name__ == "__main__":
    sys.exit(main())

"""Benchmark of the stage-pipelined fp16 TN GEMM on one MI355X.

One step = one D = A @ B^T call (the whole hot path: prologue, pipelined
mainloop and epilogue in one kernel) on inputs already resident in HBM.

Prints ONE JSON line (rank 0):
  value        whole-job TFLOP/s = 2 M N K * steps / timed wall time
  roofline     the GEMM kernel against the dense fp16 MFMA peak: achieved =
               2 M N K per launch / mean launch duration (one pair of HIP
               events around the back-to-back timed launches, on the stream
               they are launched on; when the host enqueues launches no
               faster than they run, the steps are captured once as a HIP
               graph that the timed region replays); traffic = bytes per
               launch that leave L2 (FETCH_SIZE and WRITE_SIZE, scaled by a
               plain copy of known size) from the committed rocprofv3
               summary, or null if the kernel source changed since it was
               taken.  Requests leaving L2 may still hit the memory-side
               Infinity Cache, so this bounds the HBM bytes from above
  cpu_baseline the CPU oracle timed on a bounded row sample of the same
               workload, on this host's cores
  per_config   every other workload of the measurement plan (256^3, 4096^3,
               the attention-score shape, the ragged shape, the tall-skinny
               shape and the M = N = 2048 stage sweep), each with its own
               roofline and CPU baseline; the sweep also per stage count

Other modes: variants, ksweep (every compiled variant), attention (the
fused forward), calibrate_copy (the copy the traffic counters are scaled
by), stage_model (T_copy and T_compute of the stage-count formula),
lds_patterns (epilogue staging access patterns, for the LDS counters), and
host-only summaries of rocprofv3 runs of this script: trace_summary,
profile_summary, ksweep_summary, lds_summary.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fp16 GEMM TFLOP/s at M=N=K=4096/8192 and % of MI355X fp16 MFMA peak"
PEAK_TFLOPS = 2516.6          # MI355X dense fp16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


# the device code of the GEMM kernels (the attention forward, the launcher's
# host code and the measurement probe are separate sources; which kernel a
# workload runs is checked through the variant recorded with the traffic)
GEMM_SOURCES = ("gemm_kernel.hpp", "persistent_kernel.hpp", "shortk_kernel.hpp", "onewave_mainloop.inc",
                "onewave_b3_mainloop.inc", "onewave_b3h_mainloop.inc", "onewave128_mainloop.inc")


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "stage_pipelined_mainloop_amd", "csrc")
    for name in GEMM_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, variant: str | None = None):
    """Bytes leaving L2 per launch from profiles/traffic_<workload>.json when
    it was measured on the current kernel source and (if given) on the same
    variant; otherwise None."""
    p = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    if variant is not None and t.get("variant") != variant:
        return None
    return t.get("hbm_bytes_per_launch")


def mfma_ceiling(a, b, target_ms: float = 20.0, shape16: bool = False):
    """TFLOP/s of pure fp16 MFMAs on fragments of the workload's own inputs
    (libsgprobe.so): the power-limited ceiling for this operand data, with
    32x32x16 MFMAs (or 16x16x32 with shape16)."""
    import ctypes

    import torch
    so = os.path.join(ROOT, "stage_pipelined_mainloop_amd", "libsgprobe.so")
    L = ctypes.CDLL(so)
    L.sg_probe_mfma_ceiling.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p,
                                        ctypes.c_longlong, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_void_p]
    L.sg_probe_mfma_ceiling.restype = ctypes.c_int
    L.sg_probe_mfma_ceiling_shape.argtypes = [ctypes.c_int] + L.sg_probe_mfma_ceiling.argtypes
    L.sg_probe_mfma_ceiling_shape.restype = ctypes.c_int
    L.sg_probe_mfma_ceiling_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    L.sg_probe_mfma_ceiling_flops.restype = ctypes.c_double
    blocks = 1024
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=a.device)
    stream = torch.cuda.current_stream(a.device)

    def run(iters):
        rc = L.sg_probe_mfma_ceiling_shape(int(shape16), a.data_ptr(), a.numel(), b.data_ptr(),
                                           b.numel(), blocks, iters, sink.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"mfma ceiling probe failed to launch ({rc})")

    run(50)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    run(50)
    e1.record(stream)
    torch.cuda.synchronize()
    iters = max(50, int(50 * target_ms / max(e0.elapsed_time(e1), 1e-3)))
    e0.record(stream)
    run(iters)
    e1.record(stream)
    torch.cuda.synchronize()
    return L.sg_probe_mfma_ceiling_flops(blocks, iters) / (e0.elapsed_time(e1) / 1e3) / 1e12


def cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(A, B, target_s: float):
    import oracle
    M, K = A.shape
    N = B.shape[0]
    # calibrate on a few rows, then size the sample to about target_s
    t0 = time.perf_counter()
    oracle.gemm_tn_f64_rows(A, B, 0, 2)
    dt = max(time.perf_counter() - t0, 1e-6)
    rows = int(max(2, min(M, 2 * target_s / dt)))
    t0 = time.perf_counter()
    oracle.gemm_tn_f64_rows(A, B, 0, rows)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * N * K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"rows 0..{rows - 1} of D ({rows} x {N} outputs, K={K}), fp64 accumulation, "
                      f"{dt:.1f} s wall"}


def time_launches(fn, steps: int, warmup: int):
    """Launch `fn` (one launch on the current stream) `warmup` times, then
    `steps` times back to back between one pair of HIP events; returns the
    mean milliseconds per launch.  No events sit between the launches: an
    event pair around every launch adds about 2.5 us to each reading, which
    is a fifth of a 12 us kernel."""
    import torch
    for _ in range(warmup):
        fn()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def launch_spread(fn, steps: int, flush=None):
    """Median and minimum of per-launch event timings (each includes the
    event overhead); with `flush`, it runs before every launch, outside the
    events, to measure with cold caches."""
    import torch
    stream = torch.cuda.current_stream()
    ms = []
    for _ in range(steps):
        if flush is not None:
            flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
    ms.sort()
    return ms[len(ms) // 2], ms[0]


def takes(cfg, K: int) -> bool:
    """Whether a compiled variant takes this K: the short-K schedule (4)
    holds the whole K extent in its ring."""
    return cfg.schedule != 4 or K <= cfg.tile_k * cfg.stages


def variant_info(cfg):
    import stage_pipelined_mainloop_amd as sg
    st, info = sg.sg_query_config(cfg)
    d = info.as_dict()
    d["query_status"] = st
    return d


def mode_variants(args) -> int:
    """Time every compiled variant on one workload; one JSON line each."""
    import numpy as np
    import torch

    import stage_pipelined_mainloop_amd as sg
    from stage_pipelined_mainloop_amd import inputs
    M, N, K, dist, seed = inputs.WORKLOADS[args.workload]
    A, B = inputs.workload(args.workload)
    alpha = float(np.float32(1.0 / math.sqrt(K))) if args.workload == "attn_scores" else None
    a = torch.from_numpy(A).cuda()
    b = torch.from_numpy(B).cuda()
    d = torch.empty((M, N), dtype=torch.float16, device="cuda")
    for c in sg.configs():
        if not takes(c, K):
            continue
        mean = time_launches(lambda: sg.gemm(a, b, out=d, alpha=alpha, config=c),
                             args.steps, args.warmup)
        t = 2.0 * M * N * K / (mean / 1e3) / 1e12
        print(json.dumps({"mode": "variants", "workload": args.workload,
                          "variant": c.as_tuple(), "ms_mean": round(mean, 4),
                          "tflops": round(t, 1),
                          "pct_peak": round(100 * t / PEAK_TFLOPS, 2),
                          "launches": args.warmup + args.steps, "warmup": args.warmup,
                          "info": variant_info(c)}), flush=True)
    return 0


def mode_vendor_blas(args) -> int:
    """Reference point, not part of the library: this GEMM against the ROCm
    BLAS that torch.matmul dispatches to (hipBLASLt) on the same operands and
    stream, interleaved (7 alternating rounds of --steps launches after
    --warmup of each).  One JSON line per workload: median microseconds and
    TFLOP/s of each, their ratio, and the largest |difference| of the two
    fp16 results (different summation orders)."""
    import statistics

    import torch

    import stage_pipelined_mainloop_amd as sg
    from stage_pipelined_mainloop_amd import inputs
    for w in args.workload.split(","):
        M, N, K, dist, seed = inputs.WORKLOADS[w]
        A, B = inputs.workload(w)
        a = torch.from_numpy(A).cuda()
        b = torch.from_numpy(B).cuda()
        bt = b.t()
        d_sg = torch.empty((M, N), dtype=torch.float16, device="cuda")
        calls = {"stagegemm": lambda: sg.gemm(a, b, out=d_sg),
                 "rocm_blas": lambda: torch.matmul(a, bt)}
        st = torch.cuda.current_stream()
        for f in calls.values():
            for _ in range(args.warmup):
                f()
        res = {n: [] for n in calls}
        for rnd in range(7):
            order = list(calls) if rnd % 2 == 0 else list(calls)[::-1]
            for n in order:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record(st)
                for _ in range(args.steps):
                    calls[n]()
                e1.record(st)
                torch.cuda.synchronize()
                res[n].append(e0.elapsed_time(e1) * 1e3 / args.steps)
        us = {n: statistics.median(v) for n, v in res.items()}
        tf = {n: 2.0 * M * N * K / (u * 1e-6) / 1e12 for n, u in us.items()}
        diff = float((calls["stagegemm"]().float() - calls["rocm_blas"]().float()).abs().max())
        print(json.dumps({"mode": "vendor_blas", "workload": w, "shape": [M, N, K],
                          "us": {n: round(u, 2) for n, u in us.items()},
                          "tflops": {n: round(t, 1) for n, t in tf.items()},
                          "stagegemm_over_rocm_blas": round(tf["stagegemm"] / tf["rocm_blas"], 4),
                          "max_abs_diff": diff, "rounds": 7, "launches_per_round": args.steps}),
              flush=True)
    return 0


FORMS_SHAPES = [(6144, 6144, 4096), (4352, 4352, 4096), (81920, 256, 4096), (65536, 256, 2048),
                (4352, 4104, 1088), (2048, 2048, 8192), (2048, 2048, 16384), (8192, 8192, 8200),
                (4096, 4096, 128), (2048, 2048, 2048), (2048, 2048, 512), (2048, 2048, 128),
                (81920, 256, 256), (256, 256, 256)]


def mode_vendor_summary(args) -> int:
    """profiles/vendor_blas_square8192.md from `python bench.py --mode
    vendor_blas --workload square8192,square4096` (its output in
    --bench-log) and, in --prof-dir, a kernel trace (vendor/**) and two
    counter passes (vendor_fetch, vendor_sq) of `python bench.py --mode
    vendor_blas --workload square8192 --steps 3 --warmup 1`.  Host-only."""
    import csv
    import statistics
    with open(args.bench_log) as f:
        lines = [json.loads(ln) for ln in f if ln.startswith("{") and '"vendor_blas"' in ln]
    pdir = args.prof_dir
    sq_names = ["SQ_INSTS_LDS", "SQ_LDS_IDX_ACTIVE", "SQ_BUSY_CU_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES",
                "GRBM_GUI_ACTIVE", "SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_SALU"]
    P = "python bench.py --mode vendor_blas --workload square8192 --steps 3 --warmup 1"

    def side(name):
        return "stagegemm" if "_ZN2sg" in name else "blas"
    # the GEMM kernels of each side: the most time-consuming kernel of each
    trace = _glob1(f"{pdir}/vendor/**/*kernel_trace.csv")
    kern = {}
    with open(trace) as f:
        for r in csv.DictReader(f):
            n = r["Kernel_Name"]
            if "_ZN2sg" not in n and "Cijk" not in n:
                continue
            k = kern.setdefault(n, {"durs": [], "row": r})
            k["durs"].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    hot = {}
    for n, k in kern.items():
        sd = side(n)
        if sd not in hot or sum(k["durs"]) > sum(kern[hot[sd]]["durs"]):
            hot[sd] = n
    counters = {sd: {} for sd in hot}
    for key in ("vendor_fetch", "vendor_sq"):
        with open(_glob1(f"{pdir}/**/{key}_counter_collection.csv")) as f:
            per = {}
            for r in csv.DictReader(f):
                for sd, n in hot.items():
                    if r["Kernel_Name"] == n:
                        d = per.setdefault((sd, int(r["Dispatch_Id"])), {})
                        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        for (sd, _), d in per.items():
            for c, v in d.items():
                counters[sd].setdefault(c, []).append(v)
    med = {sd: {c: statistics.median(v) for c, v in cs.items()} for sd, cs in counters.items()}
    ndisp = {sd: len(counters[sd].get("FETCH_SIZE", [])) for sd in hot}

    out = ["# This GEMM beside the ROCm BLAS GEMM on square8192 (M = N = K = 8192, uniform [-1, 1] fp16)", "",
           "A reference point, not part of the library: `torch.matmul(A, B.t())` on the same device tensors "
           "dispatches to hipBLASLt.", "",
           "## Interleaved timing (one process, one box)", "",
           "Command: `python bench.py --mode vendor_blas --workload square8192,square4096` (7 alternating rounds "
           "of 50 launches after 30 warm-up launches of each); summarised with `python bench.py --mode "
           "vendor_summary --prof-dir <dir> --bench-log <that run's output>`.", "",
           "| Workload | stagegemm us | hipBLASLt us | stagegemm TFLOP/s | hipBLASLt TFLOP/s | ratio | "
           "max abs difference of the fp16 results |", "|---|---|---|---|---|---|---|"]
    for ln in lines:
        out.append(f"| {ln['workload']} | {ln['us']['stagegemm']:.2f} | {ln['us']['rocm_blas']:.2f} | "
                   f"{ln['tflops']['stagegemm']:.1f} | {ln['tflops']['rocm_blas']:.1f} | "
                   f"{ln['stagegemm_over_rocm_blas']:.3f} | {ln['max_abs_diff']:g} |")
    out += ["", f"## Kernels and counters (square8192, per launch, median over the dispatches of each: "
                f"{ndisp.get('stagegemm', 0)} and {ndisp.get('blas', 0)})", "",
            f"Commands: `rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/vendor -o vendor -- {P}`, "
            f"`rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o vendor_fetch -- {P}` and "
            f"`rocprofv3 --pmc {' '.join(sq_names)} --output-format csv -d <dir> -o vendor_sq -- {P}`.", "",
            "| | stagegemm | hipBLASLt |", "|---|---|---|"]

    def cell(sd, fmt):
        return fmt(sd) if sd in hot else "-"
    rows = [("kernel", lambda sd: f"`{hot[sd][:110]}`"),
            ("workgroup, grid", lambda sd: f"{kern[hot[sd]]['row']['Workgroup_Size_X']} threads, "
                                           f"{int(kern[hot[sd]]['row']['Grid_Size_X']) // int(kern[hot[sd]]['row']['Workgroup_Size_X'])} workgroups"),
            ("LDS per workgroup", lambda sd: f"{kern[hot[sd]]['row']['LDS_Block_Size']} B"),
            ("registers (VGPR + AGPR)", lambda sd: f"{kern[hot[sd]]['row']['VGPR_Count']} + "
                                                   f"{kern[hot[sd]]['row']['Accum_VGPR_Count']}"),
            ("kernel trace, median us", lambda sd: f"{statistics.median(kern[hot[sd]]['durs']) / 1e3:.1f}"),
            ("FETCH_SIZE (raw KiB)", lambda sd: f"{med[sd].get('FETCH_SIZE', float('nan')):.0f}")]
    for c in sq_names:
        big = c not in ("SQ_WAVES",)
        rows.append((c, (lambda c, big: lambda sd: (f"{med[sd].get(c, float('nan')) / 1e6:.2f} M" if big
                                                   else f"{med[sd].get(c, float('nan')):.0f}"))(c, big)))
    for label, fmt in rows:
        out.append(f"| {label} | {cell('stagegemm', fmt)} | {cell('blas', fmt)} |")
    fn = os.path.join(PROFILES, "vendor_blas_square8192.md")
    with open(fn, "w") as f:
        f.write("\n".join(out) + "\n")
    print(json.dumps({"summary": fn, "kernels": hot}))
    return 0


ATTN_C1 = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_ANY "
           "SQ_WAVE_CYCLES SQ_BUSY_CU_CYCLES SQ_WAIT_INST_ANY SQ_WAIT_ANY GRBM_GUI_ACTIVE")
ATTN_C2 = ("SQ_WAIT_INST_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_ACTIVE_INST_LDS SQ_INSTS_VALU "
           "SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_VALU_TRANS_F32")


def mode_attention_summary(args) -> int:
    """profiles/attention_fwd_4096x4096x128.md from a kernel trace of `python
    bench.py --mode attention --heads 16 --steps 20 --warmup 30` (--prof-dir
    /attn, its output in --bench-log) and four counter passes of the same
    program with --steps 5 --warmup 2 (attn_c1, attn_c2, attn_fetch,
    attn_write in --prof-dir, beside the copy calibration).  Host-only."""
    import csv
    import statistics
    pdir = args.prof_dir
    scale = _copy_scales(pdir)
    with open(args.bench_log) as f:
        lines = [json.loads(ln) for ln in f if ln.startswith("{") and '"attention"' in ln]
    trace = _glob1(f"{pdir}/attn/**/*kernel_trace.csv")
    groups = {}
    with open(trace) as f:
        for r in csv.DictReader(f):
            n = r["Kernel_Name"]
            kind = "forward" if "attention_fwd_kernel" in n else "merge" if "attention_combine" in n else None
            if kind is None:
                continue
            wgs = int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"])
            groups.setdefault((kind, wgs, int(r["Workgroup_Size_X"])), []).append(
                int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    run = "python bench.py --mode attention --heads 16"
    out = ["# attention_fwd_kernel on 4096 x 4096 x 128 (d = 128), fp16, N(0,1) inputs", "",
           "Fused O = softmax(alpha Q K^T) V, alpha = fp32(1/sqrt(128)); `bench.py --mode attention` "
           "(one head with the library's split count, then 16 heads).", "",
           "## Kernel trace (rocprofv3 --kernel-trace --stats)", "",
           f"Command: `rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/attn -o attn -- {run} "
           "--steps 20 --warmup 30`; summarised with `python bench.py --mode attention_summary --prof-dir <dir> "
           "--bench-log <that run's output>`.", "",
           "| Kernel | Workgroups x threads | Calls | Average (us) | Median (us) | Min (us) |",
           "|---|---|---|---|---|---|"]
    for (kind, wgs, thr), d in sorted(groups.items()):
        out.append(f"| {kind} | {wgs} x {thr} | {len(d)} | {statistics.mean(d) / 1e3:.1f} | "
                   f"{statistics.median(d) / 1e3:.1f} | {min(d) / 1e3:.1f} |")
    out += ["", "The trace includes the warm-up launches. The bench lines printed under the tracer: " +
            "; ".join(f"{ln['heads']} head(s), {ln['splits']} split(s): {ln['ms'] * 1e3:.1f} us"
                      for ln in lines) + ".", ""]
    # counter passes: the 16-head forward launches (the largest grid)
    fwd, fwd_thr = max(((wgs, thr) for (kind, wgs, thr) in groups if kind == "forward"),
                       key=lambda x: x[0] * x[1])
    vals, durs = {}, []
    for key in ("attn_c1", "attn_c2", "attn_fetch", "attn_write"):
        per = {}
        with open(_glob1(f"{pdir}/**/{key}_counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                if "attention_fwd_kernel" not in r["Kernel_Name"]:
                    continue
                if (int(r["Grid_Size"]) // int(r["Workgroup_Size"]), int(r["Workgroup_Size"])) != (fwd, fwd_thr):
                    continue
                wave_per_wg = int(r["Workgroup_Size"]) // 64
                d = per.setdefault(int(r["Dispatch_Id"]), [{}, 0])
                d[0][r["Counter_Name"]] = d[0].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
                if r.get("End_Timestamp"):
                    d[1] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        for c_, dur in per.values():
            for k, v in c_.items():
                vals.setdefault(k, []).append(v)
            if key == "attn_c1" and dur > 0:
                durs.append(dur)
    c = {k: statistics.median(v) for k, v in vals.items()}
    P = f"{run} --steps 5 --warmup 2"
    out += ["## Counters, 16 heads (one --pmc pass each; median over the 16-head forward launches)", "",
            f"Commands: `rocprofv3 --pmc {ATTN_C1} --output-format csv -d <dir> -o attn_c1 -- {P}`, "
            f"`rocprofv3 --pmc {ATTN_C2} --output-format csv -d <dir> -o attn_c2 -- (same)`, then "
            "`--pmc FETCH_SIZE` (-o attn_fetch) and `--pmc WRITE_SIZE` (-o attn_write), and both on "
            "`python bench.py --mode calibrate_copy --steps 3 --warmup 1`.", "",
            "| Counter | Per launch |", "|---|---|"]
    for k in sorted(c):
        out.append(f"| {k} | {c[k]:.4g} |")
    H, M, N, d = 16, 4096, 4096, 128
    waves = fwd * wave_per_wg
    tiles = waves * (N // 64)                       # 64-key tiles, every wave all of them
    dur = statistics.median(durs) if durs else float("nan")
    fetched = c["FETCH_SIZE"] * 1024 * scale["FETCH_SIZE"]
    written = c["WRITE_SIZE"] * 1024 * scale["WRITE_SIZE"]
    comp = 2.0 * H * (2 * M + 2 * N) * d
    out += ["", "Derived:",
            f"- shader clock: GRBM_GUI_ACTIVE / 8 XCDs / median duration in the same pass ({dur / 1e3:.1f} us) = "
            f"{c['GRBM_GUI_ACTIVE'] / 8 / dur:.2f} GHz",
            f"- MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs over SQ_BUSY_CU_CYCLES / 256 CUs = "
            f"{100 * (c['SQ_VALU_MFMA_BUSY_CYCLES'] / 1024) / (c['SQ_BUSY_CU_CYCLES'] / 256):.1f} %",
            f"- VALU co-issued with MFMA: SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES = "
            f"{100 * c['SQ_VALU_MFMA_COEXEC_CYCLES'] / c['SQ_VALU_MFMA_BUSY_CYCLES']:.1f} %",
            f"- LDS bank conflicts: {c['SQ_LDS_BANK_CONFLICT']:.0f}",
            f"- per wave and 64-key tile: {c['SQ_INSTS_MFMA'] / tiles:.0f} MFMA, {c['SQ_INSTS_LDS'] / tiles:.0f} LDS, "
            f"{c['SQ_INSTS_VALU_TRANS_F32'] / tiles:.1f} transcendental, {c['SQ_INSTS_VALU'] / tiles:.0f} VALU "
            "instructions (MFMA included)",
            f"- bytes leaving L2 (copy-scaled, FETCH x{scale['FETCH_SIZE']:.3f}, WRITE x{scale['WRITE_SIZE']:.3f}): "
            f"fetched {fetched / 1e6:.1f} MB + written {written / 1e6:.1f} MB = {(fetched + written) / 1e6:.1f} MB; "
            f"compulsory 2 H (2M + 2N) d = {comp / 1e6:.1f} MB, ratio {(fetched + written) / comp:.2f}"]
    fn = os.path.join(PROFILES, "attention_fwd_4096x4096x128.md")
    with open(fn, "w") as f:
        f.write("\n".join(out) + "\n")
    print(json.dumps({"summary": fn, "forward_wgs": fwd, "dispatches": len(durs)}))
    return 0


def mode_forms(args) -> int:
    """The call forms the library chooses between, interleaved on the same
    uniform [-1, 1] operands: each form's --steps launches captured in one
    HIP graph (so host launch costs do not count, for the library and the
    vendor alike), --warmup eager launches first, then 7 alternating rounds
    of one replay each: the library's plain call (the remainder form where it
    applies), the split-K call with the split count given in each line
    (the library's own when it splits, else 4), the 256x256 tiled kernel
    alone (schedule 10, or 12 when K % 64 != 0 or the grid has at most two
    tile rows or columns), and torch.matmul (hipBLASLt)
    as a reference point.  One JSON line per shape: median microseconds,
    TFLOP/s, the plan (splits, remainder quarters), and whether the plain
    call and the tiled kernel agree bit for bit."""
    import statistics

    import torch

    import stage_pipelined_mainloop_amd as sg
    for M, N, K in FORMS_SHAPES:
        g = torch.Generator(device="cuda")
        g.manual_seed(M + N + K)
        a = (torch.rand((M, K), generator=g, device="cuda") * 2 - 1).half()
        b = (torch.rand((N, K), generator=g, device="cuda") * 2 - 1).half()
        bt = b.t()
        lib_splits = sg.gemm_fp16_tn_splitk_splits(M, N, K)
        splits = lib_splits if lib_splits > 1 else 4
        need = sg.gemm_fp16_tn_splitk_workspace_bytes(M, N, K, splits)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        outs = {n: torch.empty((M, N), dtype=torch.float16, device="cuda")
                for n in ("plain", "split", "tiled256")}
        def stream():
            # the stream current at each call: inside graph capture, the capture stream
            return torch.cuda.current_stream().cuda_stream
        streaming = min((M + 255) // 256, (N + 255) // 256) <= 2
        tiled = (256, 256, 64, 2, 4, 10) if K % 64 == 0 and not streaming else (256, 256, 64, 3, 4, 12)
        calls = {
            "plain": lambda: sg.gemm_fp16_tn_alpha(M, N, K, 1.0, a.data_ptr(), b.data_ptr(),
                                                   outs["plain"].data_ptr(), stream()),
            "split": lambda: sg.gemm_fp16_tn_splitk(M, N, K, 1.0, a.data_ptr(), b.data_ptr(),
                                                    outs["split"].data_ptr(), splits, ws.data_ptr(),
                                                    ws.numel(), stream()),
            "tiled256": lambda: sg.gemm_fp16_tn_cfg(M, N, K, 1.0, a.data_ptr(), b.data_ptr(),
                                                    outs["tiled256"].data_ptr(), tiled, stream()),
            "rocm_blas": lambda: torch.matmul(a, bt),
        }
        graphs = {}
        for n, f in calls.items():
            for _ in range(args.warmup):
                f()
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for _ in range(args.steps):
                    f()
            graphs[n] = gr
        res = {n: [] for n in calls}
        for rnd in range(7):
            order = list(calls) if rnd % 2 == 0 else list(calls)[::-1]
            for n in order:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record()
                graphs[n].replay()
                e1.record()
                torch.cuda.synchronize()
                res[n].append(e0.elapsed_time(e1) * 1e3 / args.steps)
        us = {n: statistics.median(v) for n, v in res.items()}
        print(json.dumps({
            "mode": "forms", "shape": [M, N, K],
            "plan": {"library_splits": lib_splits, "split_run": splits,
                     "remainder_quarters": sg.gemm_fp16_tn_remainder_quarters(M, N, K),
                     "plain_variant": variant_name(sg.sg_select_config(M, N, K)),
                     "tiled256": list(tiled)},
            "us": {n: round(u, 2) for n, u in us.items()},
            "tflops": {n: round(2.0 * M * N * K / (u * 1e-6) / 1e12, 1) for n, u in us.items()},
            "plain_equals_tiled256": bool(torch.equal(outs["plain"].view(torch.int16),
                                                      outs["tiled256"].view(torch.int16))),
            "rounds": 7, "launches_per_round": args.steps}), flush=True)
    return 0


def mode_forms_summary(args) -> int:
    """profiles/call_forms.md from `python bench.py --mode forms` (its output
    in --bench-log) and a kernel trace of the same command (stats CSV under
    --prof-dir/forms/).  Host-only."""
    import csv
    with open(args.bench_log) as f:
        lines = [json.loads(ln) for ln in f if ln.startswith("{") and '"forms"' in ln]
    names = ["plain", "split", "tiled256", "rocm_blas"]
    out = ["# Call forms: remainder form, split-K, 256x256 tiles alone, hipBLASLt", "",
           f"Command: `python bench.py --mode forms --steps {lines[0]['launches_per_round']} "
           f"--warmup {args.warmup}` (each form's launches captured in one HIP graph, 7 interleaved "
           "replays, median per launch from HIP events); "
           "kernel statistics from `rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/forms "
           "-o forms -- python bench.py --mode forms` with the same arguments; summarised with "
           "`python bench.py --mode forms_summary --prof-dir <dir> --bench-log <that run's output>`.", "",
           "`plain` is the library's call (gemm_fp16_tn_alpha: the remainder form where the plan takes "
           "it), `split` gemm_fp16_tn_splitk with the count in the plan column, `tiled256` the "
           "256x256 kernel alone (gemm_fp16_tn_cfg), `rocm_blas` torch.matmul on the same operands.", "",
           "| shape | plan | plain us | split us | tiled256 us | rocm_blas us | plain TFLOP/s | plain = tiled256 bitwise |",
           "|---|---|---|---|---|---|---|---|"]
    for ln in lines:
        p = ln["plan"]
        plan = (f"splits {p['library_splits']} (split run x{p['split_run']}), "
                f"quarters {p['remainder_quarters']}, {p['plain_variant']}")
        out.append(f"| {ln['shape'][0]}x{ln['shape'][1]}x{ln['shape'][2]} | {plan} | " +
                   " | ".join(f"{ln['us'][n]:.2f}" for n in names) +
                   f" | {ln['tflops']['plain']:.1f} | {ln['plain_equals_tiled256']} |")
    stats = _glob1(f"{args.prof_dir}/forms/**/*kernel_stats.csv")
    if stats:
        out += ["", "## Kernel statistics of the traced run", "",
                "| kernel | calls | average us |", "|---|---|---|"]
        with open(stats) as f:
            rows = sorted(csv.DictReader(f), key=lambda r: -float(r["TotalDurationNs"]))
        for r in rows[:16]:
            out.append(f"| `{r['Name'][:110]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} |")
    fn = os.path.join(PROFILES, "call_forms.md")
    with open(fn, "w") as f:
        f.write("\n".join(out) + "\n")
    print(json.dumps({"summary": fn, "shapes": len(lines)}))
    return 0


def mode_ksweep(args) -> int:
    """M = N = 2048, K in the sweep list: the library's choice (split-K when
    it picks it), then every compiled stage count of the 128x128 (4 waves)
    and 256x256 (8 waves) tiles; LDS bytes and occupancy from the library's
    query.  Each line records how many kernel dispatches it made, so a
    kernel trace or counter pass of this mode can be mapped back to it."""
    import torch

    import stage_pipelined_mainloop_amd as sg
    from stage_pipelined_mainloop_amd import inputs
    for K in inputs.KSWEEP_K:
        A, B = inputs.ksweep(K)
        a = torch.from_numpy(A).cuda()
        b = torch.from_numpy(B).cuda()
        M = N = inputs.KSWEEP_MN
        d = torch.empty((M, N), dtype=torch.float16, device="cuda")
        fn, vname, s = library_call(M, N, K, a, b, d, None)
        entries = [("library", vname, fn, 2 if s > 1 else 1, None)]
        for c in sg.configs():
            if (c.tile_m, c.tile_n, c.waves) not in ((128, 128, 4), (256, 256, 8)) or not takes(c, K):
                continue
            entries.append(("variant", variant_name(c),
                            (lambda c=c: sg.gemm(a, b, out=d, config=c)), 1, c))
        for kind, name, f, kernels, c in entries:
            mean = time_launches(f, args.steps, args.warmup)
            t = 2.0 * M * N * K / (mean / 1e3) / 1e12
            gbs = 2.0 * (M * K + N * K + M * N) / (mean / 1e3) / 1e9
            line = {"mode": "ksweep", "M": M, "N": N, "K": K, "kind": kind, "variant": name,
                    "ms_mean": round(mean, 4), "tflops": round(t, 1),
                    "pct_peak": round(100 * t / PEAK_TFLOPS, 2), "hbm_gbs_compulsory": round(gbs, 1),
                    "launches": args.warmup + args.steps, "warmup": args.warmup,
                    "kernels_per_call": kernels}
            if c is not None:
                line["config"] = c.as_tuple()
                line["info"] = variant_info(c)
            print(json.dumps(line), flush=True)
    return 0


def mode_attention(args) -> int:
    """The fused attention forward O = softmax(alpha Q K^T) V on H heads of
    the attention-score shape (M = N = 4096, d = 128, N(0,1) inputs), next to
    the unfused route on the same GPU (this library's GEMM for the scores,
    then torch's softmax and batched product) and, as a reference point,
    torch's scaled_dot_product_attention on the same tensors (one JSON line
    per head count)."""
    import numpy as np
    import torch

    import stage_pipelined_mainloop_amd as sg
    from stage_pipelined_mainloop_amd import inputs
    M, N, d = 4096, 4096, 128
    alpha = float(np.float32(1.0 / math.sqrt(d)))
    for H in (1, args.heads):
        q = torch.from_numpy(np.stack([inputs.matrix(M, d, 7000 + 3 * h, "normal") for h in range(H)])).cuda()
        k = torch.from_numpy(np.stack([inputs.matrix(N, d, 7001 + 3 * h, "normal") for h in range(H)])).cuda()
        v = torch.from_numpy(np.stack([inputs.matrix(N, d, 7002 + 3 * h, "normal") for h in range(H)])).cuda()
        o = torch.empty_like(q)
        splits = sg.attention_fp16_splits(H, M, N, d)
        ws = torch.empty(max(sg.attention_fp16_workspace_bytes(H, M, N, d, splits), 16),
                         dtype=torch.uint8, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr())

        def fused_call(sp):
            # the C entry directly: Python-side checks would cost more than
            # the kernels at one head
            return lambda: sg.attention_fp16_fwd_split(H, M, N, d, alpha, *ptrs, sp, ws.data_ptr(),
                                                       ws.numel(), stream)
        warm = max(args.warmup, 30)
        fused = time_launches(fused_call(splits), args.steps, warm)
        unsplit = time_launches(fused_call(1), args.steps, warm) if splits > 1 else fused
        s = torch.empty((H, M, N), dtype=torch.float16, device="cuda")

        def unfused():
            for h in range(H):
                sg.gemm(q[h], k[h], out=s[h], alpha=alpha)
            p = torch.softmax(s.float(), dim=-1).half()
            return torch.bmm(p, v)
        ref_ms = time_launches(unfused, max(3, args.steps // 5), 2)
        q4, k4, v4 = q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0)
        sdpa_ms = time_launches(lambda: torch.nn.functional.scaled_dot_product_attention(q4, k4, v4),
                                args.steps, warm)
        flops = 4.0 * H * M * N * d
        tf = flops / (fused / 1e3) / 1e12
        print(json.dumps({"mode": "attention", "metric": "fused attention forward TFLOP/s (4 H M N d)",
                          "heads": H, "M": M, "N": N, "d": d, "splits": splits, "ms": round(fused, 4),
                          "ms_one_split": round(unsplit, 4),
                          "tflops": round(tf, 1),
                          "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_TFLOPS,
                                       "unit": "TFLOP/s", "frac": round(tf / PEAK_TFLOPS, 4)},
                          "unfused_ms": round(ref_ms, 4),
                          "unfused": "library GEMM for S, torch softmax (fp32) and bmm",
                          "torch_sdpa_ms": round(sdpa_ms, 4)}), flush=True)
    return 0


def mode_calibrate_copy(args) -> int:
    """A plain device copy of known size, for scaling the FETCH_SIZE and
    WRITE_SIZE counters: each launch reads and writes exactly 512 MiB."""
    import torch
    n = 512 * 1024 * 1024
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    mean = time_launches(lambda: dst.copy_(src), args.steps, args.warmup)
    print(json.dumps({"mode": "calibrate_copy", "bytes_read": n, "bytes_written": n,
                      "ms_mean": round(mean, 4), "gbs": round(2 * n / (mean / 1e3) / 1e9, 1)}),
          flush=True)
    return 0


def variant_name(cfg, splits: int = 1) -> str:
    v = "x".join(str(x) for x in cfg.as_tuple()[:3]) + f" S{cfg.stages} w{cfg.waves} sched{cfg.schedule}"
    return v + (f" split-K x{splits}" if splits > 1 else "")


def library_call(M: int, N: int, K: int, a, b, d, alpha):
    """The library's choice for this shape as one launch function (split-K
    with its workspace when the library picks it), its description and the
    split count."""
    import torch

    import stage_pipelined_mainloop_amd as sg
    s = max(sg.gemm_fp16_tn_splitk_splits(M, N, K), 1)
    need = sg.gemm_fp16_tn_splitk_workspace_bytes(M, N, K, s) if s > 1 else 0
    al = 1.0 if alpha is None else float(alpha)
    ptrs = (a.data_ptr(), b.data_ptr(), d.data_ptr())

    def stream():
        # the stream current at each call: inside graph capture, the capture
        # stream, so that a captured graph holds the kernels
        return torch.cuda.current_stream().cuda_stream
    if need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=a.device)   # contents do not matter

        def fn():
            sg.gemm_fp16_tn_splitk(M, N, K, al, *ptrs, s, ws.data_ptr(), need, stream())
        fn.workspace = ws
        # the split-K pieces run schedule 10 when every row starts on a
        # 128-byte line, else schedule 12
        lines = K % 64 == 0 and (a.data_ptr() | b.data_ptr()) % 128 == 0
        cfg = sg.SgConfig(256, 256, 64, 2, 4, 10) if lines else sg.SgConfig(256, 256, 64, 3, 4, 12)
        return fn, variant_name(cfg, s), s

    def fn():
        sg.gemm_fp16_tn_alpha(M, N, K, al, *ptrs, stream())
    name = variant_name(sg.sg_select_config(M, N, K))
    quarters = sg.gemm_fp16_tn_remainder_quarters(M, N, K)
    if quarters > 0:
        name += f" + {quarters} 128x128 quarters on sched14"
    return fn, name, 1


def timed_mean_ms(fn, target_ms: float = 40.0, min_launches: int = 20):
    """Mean launch time of `fn` back to back: about target_ms of warm-up, then
    about target_ms timed between one pair of HIP events.  Calls that may be
    launch-bound (the host enqueues nearly as slowly as they run, or they run
    under 50 us, where the host's enqueue rate decides whether the GPU idles
    between launches) are also replayed from a captured HIP graph, as in the
    headline measurement, and the faster of the two counts.  Returns (ms,
    launch kind)."""
    import torch
    for _ in range(10):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(20):
        fn()
    enq = (time.perf_counter() - t0) / 20
    torch.cuda.synchronize()
    per = (time.perf_counter() - t0) / 20
    n = max(min_launches, min(5000, int(target_ms / 1e3 / max(per, 1e-6))))
    if enq > 0.9 * per or per < 50e-6:
        # a graph of 50 launches (as in the headline measurement), replayed
        # back to back about n / 50 times
        per_graph = 50
        reps = max(1, n // per_graph)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                fn()
        g.replay()
        g.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1) / (reps * per_graph)
        # a graph of kernels of a few microseconds can replay slower than
        # eager launches run: report the faster way of launching
        eager_ms = time_launches(fn, n, n)
        return (graph_ms, "graph") if graph_ms < eager_ms else (eager_ms, "eager")
    return time_launches(fn, n, n), "eager"


def roofline_of(M: int, N: int, K: int, ms: float, workload: str | None = None,
                variant: str | None = None) -> dict:
    """MFMA roofline above the ridge (about 315 flop/B), HBM below it, with
    the algorithmic work 2MNK flop or 2(MK + NK + MN) bytes per launch."""
    flops = 2.0 * M * N * K
    algo_bytes = 2.0 * (M * K + N * K + M * N)
    traffic = load_traffic(workload, variant) if workload else None
    ridge = PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if flops / algo_bytes < ridge:
        gbs = algo_bytes / (ms / 1e3) / 1e9
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic}
    tf = flops / (ms / 1e3) / 1e12
    return {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / PEAK_TFLOPS, 4), "traffic": traffic}


def cpu_baseline_full(A, B, min_s: float = 0.5):
    """The oracle on the whole (small) problem, repeated for at least min_s."""
    import oracle
    M, K = A.shape
    N = B.shape[0]
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.gemm_tn_f64(A, B)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_s:
            break
    return {"value": 2.0 * M * N * K * reps / dt / 1e12, "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle", "cpu": cpu_model(),
            "sample": f"all {M} x {N} outputs (K={K}), {reps} runs, {dt:.2f} s wall"}


def per_config(args) -> dict:
    """Every workload of the measurement plan besides the headline: the
    library's choice timed on one GPU with its roofline, next to the oracle
    timed on this host on a bounded sample of the same workload; the stage
    sweep also per stage count (LDS bytes and workgroups per CU from the
    library's query)."""
    import numpy as np
    import torch

    import stage_pipelined_mainloop_amd as sg
    from stage_pipelined_mainloop_amd import inputs
    res = {}
    cpu_s = args.config_cpu_seconds
    for name in ("square256", "square4096", "attn_scores", "ragged8000", "tall81920"):
        M, N, K, dist, seed = inputs.WORKLOADS[name]
        A, B = inputs.workload(name)
        alpha = float(np.float32(1.0 / math.sqrt(K))) if name == "attn_scores" else None
        a, b = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
        d = torch.empty((M, N), dtype=torch.float16, device="cuda")
        fn, vname, s = library_call(M, N, K, a, b, d, alpha)
        ms, kind = timed_mean_ms(fn)
        entry = {"M": M, "N": N, "K": K, "dist": dist, "variant": vname, "launch": kind,
                 "kernel_us": round(ms * 1e3, 2),
                 "tflops": round(2.0 * M * N * K / (ms / 1e3) / 1e12, 1),
                 "roofline": roofline_of(M, N, K, ms, name, vname)}
        if not args.no_cpu_baseline:
            entry["cpu_baseline"] = (cpu_baseline_full(A, B) if M * N * K <= 1 << 26
                                     else cpu_baseline(A, B, cpu_s))
        res[name] = entry
        print(f"[bench] {name}: {entry['kernel_us']} us, {entry['variant']}", file=sys.stderr,
              flush=True)
        del a, b, d, fn
    # stage sweep: M = N = 2048, every K; the library's choice and the best
    # compiled variant at each stage count of the 128x128 (4 waves) and
    # 256x256 (8 waves) families
    sweep = {"M": inputs.KSWEEP_MN, "N": inputs.KSWEEP_MN, "K": {}}
    M = N = inputs.KSWEEP_MN
    for K in inputs.KSWEEP_K:
        A, B = inputs.ksweep(K)
        a, b = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
        d = torch.empty((M, N), dtype=torch.float16, device="cuda")
        fn, vname, s = library_call(M, N, K, a, b, d, None)
        ms, kind = timed_mean_ms(fn, target_ms=20.0)
        per_k = {"library": {"variant": vname, "kernel_us": round(ms * 1e3, 2),
                             "roofline": roofline_of(M, N, K, ms)}, "by_stages": {}}
        for c in sg.configs():
            if (c.tile_m, c.tile_n, c.waves) not in ((128, 128, 4), (256, 256, 8)) or not takes(c, K):
                continue
            cms, _ = timed_mean_ms(lambda: sg.gemm(a, b, out=d, config=c), target_ms=5.0,
                                   min_launches=10)
            key = str(c.stages)
            best = per_k["by_stages"].get(key)
            if best is None or cms * 1e3 < best["kernel_us"]:
                info = variant_info(c)
                per_k["by_stages"][key] = {
                    "variant": variant_name(c), "kernel_us": round(cms * 1e3, 2),
                    "tflops": round(2.0 * M * N * K / (cms / 1e3) / 1e12, 1),
                    "frac": roofline_of(M, N, K, cms)["frac"],
                    "lds_ring_bytes": info["lds_bytes"], "lds_total_bytes": info["lds_total_bytes"],
                    "wg_per_cu": info["wg_per_cu"]}
        bs = min(per_k["by_stages"].items(), key=lambda kv: kv[1]["kernel_us"])
        per_k["best_fixed_stage_count"] = {"stages": int(bs[0]), **bs[1]}
        if not args.no_cpu_baseline:
            per_k["cpu_baseline"] = cpu_baseline(A, B, cpu_s / 2)
        sweep["K"][str(K)] = per_k
        print(f"[bench] ksweep K={K}: {per_k['library']['kernel_us']} us, {vname}", file=sys.stderr,
              flush=True)
        del a, b, d, fn
    res["ksweep"] = sweep
    return res


def mode_stage_model(args) -> int:
    """The stage-count model of "Lesson 6", section 4, evaluated for the
    256 x 256 x 64 tile of the large-shape kernel on this GPU: T_copy (one K
    tile's LDS-DMA loads, issue to completion, every CU copying at once) and
    T_compute (one K tile's MFMAs per wave) in shader clock cycles from the
    probe library, S_min = ceil(T_copy / T_compute) + 1 from the library's
    sg_minimum_stages, and the LDS footprint and workgroups per CU of every
    ring depth at this tile next to the ring the kernel uses."""
    import ctypes
    import statistics

    import numpy as np
    import torch

    import stage_pipelined_mainloop_amd as sg
    from stage_pipelined_mainloop_amd import inputs
    so = os.path.join(ROOT, "stage_pipelined_mainloop_amd", "libsgprobe.so")
    P = ctypes.CDLL(so)
    P.sg_probe_stage_timing.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p,
                                        ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    P.sg_probe_stage_timing.restype = ctypes.c_int
    M, N, K, dist, seed = inputs.WORKLOADS[args.workload]
    A, B = inputs.workload(args.workload)
    a, b = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles_m = M // 256
    blocks = min(cus, tiles_m * (N // 256))
    ntile = K // 64
    out = torch.zeros(blocks * 32, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()

    def run():
        rc = P.sg_probe_stage_timing(a.data_ptr(), M, b.data_ptr(), N, K, tiles_m, blocks, ntile,
                                     out.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"stage probe failed to launch ({rc})")
    for _ in range(3):
        run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    run()
    e1.record(stream)
    torch.cuda.synchronize()
    r = out.view(blocks, 8, 4).cpu().numpy().astype(np.float64)
    copy_w = r[:, :, 0] / r[:, :, 2]              # per wave, cycles per K tile
    comp_w = r[:, :, 1] / r[:, :, 2]
    copy = copy_w.ravel()
    comp = comp_w.ravel()
    # a workgroup's tile is ready when its last wave's loads are, and its
    # MFMAs are done when its last wave's are
    copy_wg = copy_w.max(axis=1)
    comp_wg = comp_w.max(axis=1)

    def stats(x):
        return {"median": round(float(np.median(x)), 1), "mean": round(float(x.mean()), 1),
                "p10": round(float(np.percentile(x, 10)), 1), "p90": round(float(np.percentile(x, 90)), 1)}
    t_copy = statistics.median(copy.tolist())
    t_comp = statistics.median(comp.tolist())
    s_min = sg.sg_minimum_stages(int(round(t_copy)), int(round(t_comp)))
    t_copy_wg = float(np.median(copy_wg))
    t_comp_wg = float(np.median(comp_wg))
    s_min_wg = sg.sg_minimum_stages(int(round(t_copy_wg)), int(round(t_comp_wg)))
    stage_bytes = (256 + 256) * 64 * 2
    rings = [{"stages": st, "lds_bytes": st * stage_bytes,
              "wg_per_cu_lds": (160 * 1024) // (st * stage_bytes)} for st in range(2, 6)]
    _, info = sg.sg_query_config(sg.SgConfig(256, 256, 64, 3, 4, 12))
    print(json.dumps({
        "mode": "stage_model", "workload": args.workload, "tile": "256x256x64",
        "workgroups": blocks, "k_tiles_timed": ntile, "probe_ms": round(e0.elapsed_time(e1), 3),
        "T_copy_cycles": stats(copy), "T_compute_cycles": stats(comp),
        "copy_over_compute": round(t_copy / t_comp, 3),
        "S_min": s_min, "formula": "ceil(T_copy / T_compute) + 1 (medians over waves)",
        "per_workgroup": {"T_copy_cycles": stats(copy_wg), "T_compute_cycles": stats(comp_wg),
                          "copy_over_compute": round(t_copy_wg / t_comp_wg, 3), "S_min": s_min_wg,
                          "statistic": "slowest wave of each workgroup, median over workgroups"},
        "rings_of_whole_stages": rings,
        "kernel_rings": {
            "schedule_10": {"A_slots": 2, "B_slots": 2, "lds_bytes": 2 * stage_bytes, "wg_per_cu": 1,
                            "loads_issued": "A(k+2), B(k+2) in the second half of tile k"},
            "schedule_12": {"A_slots": 2, "B_slots": 3, "lds_bytes": info.lds_bytes,
                            "wg_per_cu": info.wg_per_cu,
                            "loads_issued": "B(k+2) in the first half, A(k+2) in the second half of tile k"}}}),
          flush=True)
    return 0


def _pmc(path: str, name_filter: str = "_ZN2sg"):
    """Rows of a rocprofv3 counter CSV for this library's kernels, grouped by
    dispatch: {dispatch id: (kernel name, {counter: value}, duration ns)}."""
    import csv
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if name_filter not in r["Kernel_Name"]:
                continue
            d = out.setdefault(int(r["Dispatch_Id"]), [r["Kernel_Name"], {}, 0])
            d[1][r["Counter_Name"]] = d[1].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            if "End_Timestamp" in r and r["End_Timestamp"]:
                d[2] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return out


def _glob1(pattern: str):
    import glob
    f = sorted(glob.glob(pattern, recursive=True))
    return f[0] if f else None


def _copy_scales(prof_dir: str):
    """FETCH_SIZE / WRITE_SIZE scale factors from the calibration copy passes
    (512 MiB read and written per launch)."""
    scale = {}
    for key, counter in (("copy_fetch", "FETCH_SIZE"), ("copy_write", "WRITE_SIZE")):
        rows = _pmc(_glob1(f"{prof_dir}/**/{key}_counter_collection.csv"), "")
        vals = [c[counter] for _, (n, c, _d) in rows.items() if counter in c and "opy" in n]
        if not vals:
            vals = [max(c.get(counter, 0.0) for _, (n, c, _d) in rows.items())]
        scale[counter] = (512 * 1024 * 1024) / (max(vals) * 1024)
    return scale


SQ_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE "
               "SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_WAVES SQ_INSTS_LDS GRBM_GUI_ACTIVE")


def mode_profile_summary(args) -> int:
    """Turn one workload's profiling runs into profiles/<kernel>_<workload>.md
    and profiles/traffic_<workload>.json (which the bench line reads):
    a kernel trace of `python bench.py --workload W --no-per-config
    --no-cpu-baseline` averaged over exactly its timed dispatches, and three
    counter passes of the same command with --steps 5 --warmup 1 (FETCH_SIZE,
    WRITE_SIZE, and the SQ counters), scaled by the calibration copy's passes.
    Host-only, no GPU.  Expects in --prof-dir: trace_<W>/ (kernel trace and
    stats CSVs), trace_<W>.log (that run's output), <W>_fetch, <W>_write,
    <W>_sq, copy_fetch, copy_write counter CSVs."""
    import csv
    import statistics
    w, pdir = args.workload, args.prof_dir
    scale = _copy_scales(pdir)
    with open(f"{pdir}/trace_{w}.log") as f:
        b = json.loads([ln for ln in f if ln.startswith("{")][-1])
    M, N, K = b["config"]["M"], b["config"]["N"], b["config"]["K"]
    win = b["config"]["trace_window"]
    trace = _glob1(f"{pdir}/trace_{w}/**/*kernel_trace.csv")
    per = {}
    with open(trace) as f:
        for r in csv.DictReader(f):
            per.setdefault(r["Kernel_Name"], []).append(
                (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    ours = {k: v for k, v in per.items() if "_ZN2sg" in k}
    hot = max(ours, key=lambda k: sum(d for _, d in ours[k]))
    seq = [d for _, d in sorted(ours[hot])]
    window = seq[win["first"]:win["first"] + win["count"]]
    mean_ns = statistics.mean(window)
    pm = {}
    for key in ("fetch", "write", "sq"):
        rows = _pmc(_glob1(f"{pdir}/**/{w}_{key}_counter_collection.csv"))
        sel = [c for _, (n, c, _d) in sorted(rows.items()) if n == hot]
        durs = [d for _, (n, c, d) in sorted(rows.items()) if n == hot and d > 0]
        agg = {}
        for c in sel:
            for kk, v in c.items():
                agg.setdefault(kk, []).append(v)
        pm[key] = ({kk: statistics.mean(v) for kk, v in agg.items()},
                   statistics.mean(durs) if durs else None)
    fetch_b = pm["fetch"][0]["FETCH_SIZE"] * 1024 * scale["FETCH_SIZE"]
    write_b = pm["write"][0]["WRITE_SIZE"] * 1024 * scale["WRITE_SIZE"]
    sq, sq_dur = pm["sq"]
    flops = 2.0 * M * N * K
    algo = 2.0 * (M * K + N * K + M * N)
    roof = roofline_of(M, N, K, mean_ns / 1e6)
    # The bench's own timing of this workload: from a bench.py run made
    # without the profiler (--bench-log), else from the traced run.  (The
    # kernel tracer adds its own cost to every dispatch, which dominates the
    # replay of a graph of kernels of a few microseconds, so short
    # workloads need the former.)
    events_us, events_src = b["config"]["kernel_ms_mean"] * 1e3, "the traced run"
    if args.bench_log:
        with open(args.bench_log) as f:
            bl = json.loads([ln for ln in f if ln.startswith("{")][-1])
        if bl["config"]["workload"] == w:
            events_us, events_src = bl["config"]["kernel_ms_mean"] * 1e3, "a bench.py run without the profiler"
        elif w in bl.get("per_config", {}):
            events_us, events_src = bl["per_config"][w]["kernel_us"], "a bench.py run without the profiler"
    short = hot.split("Cfg")[1].split("EEE")[0].replace("ILi", "").replace("ELi", "_").replace("E", "")
    family = hot.split("2sg")[1].split("INS_")[0].lstrip("0123456789")
    util = sq["SQ_VALU_MFMA_BUSY_CYCLES"] / (4 * sq["SQ_BUSY_CU_CYCLES"])
    conflict = sq["SQ_LDS_BANK_CONFLICT"] / max(sq["SQ_LDS_IDX_ACTIVE"], 1)
    ghz = sq["GRBM_GUI_ACTIVE"] / 8 / sq_dur if sq_dur else float("nan")
    P = f"python bench.py --workload {w} --no-per-config --no-cpu-baseline --steps 5 --warmup 1"
    trace_cmd = (f"rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/trace_{w} -o {w} -- "
                 f"python bench.py --workload {w} --no-per-config --no-cpu-baseline")
    lines = [
        f"# {family}<{short}> on {w} (M={M}, N={N}, K={K})", "",
        f"Kernel: `{hot}`", "",
        "## Kernel trace, timed dispatches only", "",
        f"Command: `{trace_cmd}`", "",
        f"Summarised with `python bench.py --mode profile_summary --prof-dir <dir> --workload {w}`.", "",
        "| Dispatches in trace | Timed window | Mean over window (us) | Roofline at that mean | bench.py events (us) | trace / events |",
        "|---|---|---|---|---|---|",
        f"| {len(seq)} | {win['first']}..{win['first'] + win['count'] - 1} | {mean_ns / 1e3:.2f} | "
        f"{roof['achieved']} {roof['unit']}, frac {roof['frac']} | {events_us:.2f} | "
        f"{mean_ns / 1e3 / events_us:.4f} |", "",
        f"Launches: {b['config'].get('launch', 'eager')}; variant {b['config']['variant']}. "
        f"bench.py events: the mean per launch from {events_src}.", "",
        "## Bytes leaving L2 (two --pmc passes, scaled by a plain copy)", "",
        f"Commands: `rocprofv3 --pmc FETCH_SIZE --output-format csv -- {P}` and the same with `WRITE_SIZE`; "
        "calibration: `rocprofv3 --pmc FETCH_SIZE -- python bench.py --mode calibrate_copy --steps 3 --warmup 1` "
        f"(and `WRITE_SIZE`), a copy of 512 MiB each way: scales {scale['FETCH_SIZE']:.3f} and {scale['WRITE_SIZE']:.3f}.",
        "The L2's misses may still hit the memory-side Infinity Cache (no counter for its hits is exposed), "
        "so these bytes bound the HBM bytes from above.", "",
        "| Per launch | Value |", "|---|---|",
        f"| FETCH_SIZE (raw) | {pm['fetch'][0]['FETCH_SIZE']:.0f} KiB |",
        f"| WRITE_SIZE (raw) | {pm['write'][0]['WRITE_SIZE']:.0f} KiB |",
        f"| fetched (scaled) | {fetch_b / 1e6:.1f} MB |",
        f"| written (scaled) | {write_b / 1e6:.1f} MB |",
        f"| leaving L2, total | {(fetch_b + write_b) / 1e6:.1f} MB |",
        f"| algorithmic 2(MK+NK+MN) | {algo / 1e6:.1f} MB |",
        f"| leaving L2 / algorithmic | {(fetch_b + write_b) / algo:.2f} |",
        f"| GB/s at the window mean | {(fetch_b + write_b) / mean_ns:.0f} |", "",
        "## SQ counters (one --pmc pass)", "",
        f"Command: `rocprofv3 --pmc {SQ_COUNTERS} --output-format csv -- {P}`", "",
        "| Counter | Per launch |", "|---|---|"]
    lines += [f"| {c} | {v:.4g} |" for c, v in sorted(sq.items())]
    lines += ["", "Derived:",
              f"- MFMA utilisation: SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs x SQ_BUSY_CU_CYCLES) = {100 * util:.1f} %",
              f"- LDS bank-conflict rate: SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE = {conflict:.4f}"]
    if sq_dur and sq_dur >= 100e3:
        lines += [f"- shader clock in the counter pass: GRBM_GUI_ACTIVE / 8 XCDs / duration = {ghz:.2f} GHz "
                  f"(peak at that clock: {256 * 4096 * ghz / 1e3:.0f} TFLOP/s)"]
    md = "\n".join(lines) + "\n"
    fn = os.path.join(PROFILES, f"gemm_tn_{short}_{w}.md")
    with open(fn, "w") as f:
        f.write(md)
    tj = {"workload": w, "kernel": hot, "variant": b["config"]["variant"],
          "kernel_source_sha": kernel_source_sha(),
          "hbm_bytes_per_launch": round(fetch_b + write_b), "fetch_bytes": round(fetch_b),
          "write_bytes": round(write_b), "fetch_scale": round(scale["FETCH_SIZE"], 4),
          "write_scale": round(scale["WRITE_SIZE"], 4), "summary": os.path.basename(fn),
          "kind": "bytes leaving L2 (FETCH_SIZE + WRITE_SIZE, copy-scaled)"}
    with open(os.path.join(PROFILES, f"traffic_{w}.json"), "w") as f:
        json.dump(tj, f, indent=1)
    print(json.dumps({"summary": fn, "window_us": round(mean_ns / 1e3, 2), "mfma_util": round(util, 4),
                      "lds_conflict_rate": round(conflict, 4),
                      "l2_egress_mb": round((fetch_b + write_b) / 1e6, 1)}))
    return 0


def mode_ksweep_summary(args) -> int:
    """profiles/ksweep_m2048_n2048.md from a kernel trace and three counter
    passes of `python bench.py --mode ksweep` (files in --prof-dir:
    ks_trace/ and ks_trace.log from `--steps 10 --warmup 3`; ks_fetch,
    ks_write, ks_sq counter CSVs and ks_pmc.log from `--steps 1 --warmup 0`),
    plus the CPU baselines of a default bench.py run (--bench-log).  Each
    sweep line's dispatches are found by order; a split-K call's time runs
    from its first kernel's start to its reduction's end."""
    import csv
    import statistics
    pdir = args.prof_dir
    scale = _copy_scales(pdir)

    def lines_of(path):
        with open(path) as f:
            return [json.loads(ln) for ln in f if ln.startswith("{") and '"ksweep"' in ln]
    tl = lines_of(f"{pdir}/ks_trace.log")
    pl = lines_of(f"{pdir}/ks_pmc.log")
    rows = []
    with open(_glob1(f"{pdir}/ks_trace/**/*kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            if "_ZN2sg" in r["Kernel_Name"]:
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    rows.sort()
    timing, i = [], 0
    for ln in tl:
        k, n = ln["kernels_per_call"], ln["launches"]
        calls = [rows[i + j * k:i + (j + 1) * k] for j in range(n)]
        i += n * k
        timed = calls[ln["warmup"]:]
        timing.append(statistics.mean(c[-1][1] - c[0][0] for c in timed) / 1e3)
    pmc = {key: sorted(_pmc(_glob1(f"{pdir}/**/ks_{key}_counter_collection.csv")).items())
           for key in ("fetch", "write", "sq")}
    cpu = {}
    if args.bench_log:
        with open(args.bench_log) as f:
            bl = json.loads([ln for ln in f if ln.startswith("{")][-1])
        for K, e in bl["per_config"]["ksweep"]["K"].items():
            cpu[int(K)] = e.get("cpu_baseline")
    out = ["# K-sweep at M = N = 2048 (stage-count tuning)", "",
           "Commands (each run's dispatches are mapped to the sweep lines by order):",
           "- timing: `rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/ks_trace -o ksweep -- "
           "python bench.py --mode ksweep --steps 10 --warmup 3` (mean over the 10 timed calls of each line)",
           f"- counters: `rocprofv3 --pmc {SQ_COUNTERS} --output-format csv -d <dir> -o ks_sq -- "
           "python bench.py --mode ksweep --steps 1 --warmup 0`, and the same with `FETCH_SIZE` (-o ks_fetch) "
           "and `WRITE_SIZE` (-o ks_write); copy calibration as in the per-workload summaries "
           f"(scales {scale['FETCH_SIZE']:.3f} / {scale['WRITE_SIZE']:.3f})",
           "- summarised with `python bench.py --mode ksweep_summary --prof-dir <dir> --bench-log <bench.py output>`",
           "",
           "Inputs: A, B = 2048 x K fp16, uniform[-1,1] (seeds 5/6).  `us` = mean GPU time per call from the trace "
           "(a split-K call: first kernel's start to the reduction's end); `busy` = SQ_VALU_MFMA_BUSY_CYCLES / "
           "(4 x SQ_BUSY_CU_CYCLES); `conflict` = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; `L2 out` = "
           "copy-scaled FETCH_SIZE + WRITE_SIZE per call (bytes leaving L2, an upper bound on HBM bytes) and "
           "`GB/s` that over `us`; `ring` = stages x (tile_m + tile_n) x tile_k x 2 bytes, `lds` = allocated LDS, "
           "`wg/cu` = resident workgroups per CU (runtime query), `regs` = registers per lane.  The library line "
           "is the call bench.py times for this shape.", ""]
    j = 0
    for K in sorted({ln["K"] for ln in tl}):
        c = cpu.get(K)
        out += [f"## K = {K}", ""]
        if c:
            out += [f"Oracle on this host: {c['value']:.4f} TFLOP/s on {c['cores']} threads ({c['sample']}).", ""]
        out += ["| variant | S | us | TFLOP/s | frac | busy | conflict | L2 out MB | GB/s | ring B | lds B | wg/cu | regs |",
                "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
        for idx, ln in enumerate(tl):
            if ln["K"] != K:
                continue
            us = timing[idx]
            k = ln["kernels_per_call"]
            sq = {}
            fetch = write = 0.0
            for q in range(k):
                for cn, v in pmc["sq"][j + q][1][1].items():
                    sq[cn] = sq.get(cn, 0.0) + v
                fetch += pmc["fetch"][j + q][1][1].get("FETCH_SIZE", 0.0)
                write += pmc["write"][j + q][1][1].get("WRITE_SIZE", 0.0)
            j += k * pl[idx]["launches"] if idx < len(pl) else k
            l2 = (fetch * scale["FETCH_SIZE"] + write * scale["WRITE_SIZE"]) * 1024
            M = N = 2048
            tf = 2.0 * M * N * K / us / 1e6
            busy = sq.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) / max(4 * sq.get("SQ_BUSY_CU_CYCLES", 1), 1)
            conf = sq.get("SQ_LDS_BANK_CONFLICT", 0) / max(sq.get("SQ_LDS_IDX_ACTIVE", 1), 1)
            info = ln.get("info", {})
            st = ln["config"][3] if "config" in ln else "-"
            name = ("**library: " + ln["variant"] + "**") if ln["kind"] == "library" else ln["variant"]
            out.append(f"| {name} | {st} | {us:.1f} | {tf:.1f} | {tf / PEAK_TFLOPS:.3f} | {100 * busy:.1f} % | "
                       f"{conf:.3f} | {l2 / 1e6:.1f} | {l2 / us / 1e3:.0f} | {info.get('lds_bytes', '-')} | "
                       f"{info.get('lds_total_bytes', '-')} | {info.get('wg_per_cu', '-')} | {info.get('regs', '-')} |")
        out.append("")
    fn = os.path.join(PROFILES, "ksweep_m2048_n2048.md")
    with open(fn, "w") as f:
        f.write("\n".join(out) + "\n")
    print(json.dumps({"summary": fn, "lines": len(tl)}))
    return 0


LDS_PATTERNS = [
    "padded 144-byte rows, 16x16 pieces: 64-bit write (tiled epilogue before)",
    "padded 144-byte rows: 128-bit read (tiled epilogue before)",
    "128-byte rows, slot ^ ((r >> 1) & 15), 32x32 pieces: 64-bit write (persistent/short-K before)",
    "128-byte rows, slot ^ ((r >> 1) & 15): 128-bit read (persistent/short-K before)",
    "128-byte rows, slot ^ (r & 15), 32x32 pieces: 64-bit write (all epilogues now)",
    "128-byte rows, slot ^ (r & 15), 16x16 pieces: 64-bit write (all epilogues now)",
    "128-byte rows, slot ^ (r & 15): 128-bit read (all epilogues now)",
    "contiguous 64-bit write",
    "contiguous 128-bit read",
]


def mode_lds_patterns(args) -> int:
    """Run each epilogue staging access pattern of the probe library once
    (256 one-wave workgroups x 1000 repetitions of 8 accesses); meant to run
    under rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS,
    whose dispatches --mode lds_summary maps back to the patterns."""
    import ctypes

    import torch
    P = ctypes.CDLL(os.path.join(ROOT, "stage_pipelined_mainloop_amd", "libsgprobe.so"))
    P.sg_probe_lds_pattern.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p]
    P.sg_probe_lds_pattern.restype = ctypes.c_int
    sink = torch.empty(256 * 64, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for i, name in enumerate(LDS_PATTERNS):
        if P.sg_probe_lds_pattern(i, 256, 1000, sink.data_ptr(), stream) != 0:
            raise RuntimeError(f"pattern {i} failed to launch")
        torch.cuda.synchronize()
        print(json.dumps({"mode": "lds_patterns", "pattern": i, "name": name}), flush=True)
    return 0


def mode_lds_summary(args) -> int:
    """profiles/lds_epilogue_patterns.md from a counter pass of --mode
    lds_patterns (lds_counter_collection.csv in --prof-dir)."""
    rows = sorted((d, n, c) for d, (n, c, _) in
                  _pmc(_glob1(f"{args.prof_dir}/**/lds_counter_collection.csv"), "lds_pattern").items())
    out = ["# LDS bank conflicts of the epilogue staging patterns (gfx950)", "",
           "Command: `rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS GRBM_GUI_ACTIVE "
           "--output-format csv -d <dir> -o lds -- python bench.py --mode lds_patterns`; summarised with "
           "`python bench.py --mode lds_summary --prof-dir <dir>`.", "",
           "Each pattern: 256 one-wave workgroups, 1000 repetitions of 8 accesses of one staging block "
           "(32 rows of 64 fp16).  Cycles and conflict cycles per LDS instruction (the compiler may pair two "
           "64-bit writes into one instruction: then one instruction is two accesses).", "",
           "| pattern | LDS instructions | active cycles / instr | conflict cycles / instr |", "|---|---|---|---|"]
    for i, (d, n, c) in enumerate(rows):
        ins = max(c.get("SQ_INSTS_LDS", 0.0), 1.0)
        out.append(f"| {LDS_PATTERNS[i] if i < len(LDS_PATTERNS) else n} | {ins:.0f} | "
                   f"{c.get('SQ_LDS_IDX_ACTIVE', 0) / ins:.2f} | {c.get('SQ_LDS_BANK_CONFLICT', 0) / ins:.2f} |")
    fn = os.path.join(PROFILES, "lds_epilogue_patterns.md")
    with open(fn, "w") as f:
        f.write("\n".join(out) + "\n")
    print(json.dumps({"summary": fn, "patterns": len(rows)}))
    return 0


def mode_variants_summary(args) -> int:
    """profiles/variants_<workload>.md from a kernel trace of `python bench.py
    --mode variants --workload W` (trace CSV under --prof-dir/var_<W>/, that
    run's output in --bench-log): every compiled variant's mean GPU time over
    its timed dispatches, mapped by order."""
    import csv
    import statistics
    w = args.workload
    with open(args.bench_log) as f:
        lines = [json.loads(ln) for ln in f if ln.startswith("{") and '"variants"' in ln]
    rows = []
    with open(_glob1(f"{args.prof_dir}/var_{w}/**/*kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            if "_ZN2sg" in r["Kernel_Name"]:
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),
                             r["Kernel_Name"]))
    rows.sort()
    M, N, K = inputs_shape(w)
    out = [f"# Every compiled variant on {w} (M={M}, N={N}, K={K})", "",
           f"Command: `rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/var_{w} -o {w} -- "
           f"python bench.py --mode variants --workload {w} --steps {lines[0]['launches'] - lines[0]['warmup']} "
           f"--warmup {lines[0]['warmup']}`; summarised with `python bench.py --mode variants_summary "
           f"--prof-dir <dir> --bench-log <that run's output> --workload {w}`.", "",
           "`us` = mean kernel-trace duration over each variant's timed dispatches (mapped by order).  "
           "Schedules: 0 three-phase, 1 cute order, 2 ping-pong, 3 persistent, 4 short K, 5 cute order on "
           "16x16x32 MFMAs, 7 ping-pong on 16x16x32, 8 split-load ping-pong, 10 one wave per SIMD.", "",
           "| variant (tile_m, tile_n, tile_k, stages, waves, schedule) | us | TFLOP/s | frac |", "|---|---|---|---|"]
    i = 0
    res = []
    for ln in lines:
        n = ln["launches"]
        seg = rows[i:i + n]
        i += n
        us = statistics.mean(d for _, d, _ in seg[ln["warmup"]:]) / 1e3
        res.append((us, ln["variant"]))
    for us, v in sorted(res):
        tf = 2.0 * M * N * K / us / 1e6
        out.append(f"| {tuple(v)} | {us:.1f} | {tf:.1f} | {tf / PEAK_TFLOPS:.3f} |")
    fn = os.path.join(PROFILES, f"variants_{w}.md")
    with open(fn, "w") as f:
        f.write("\n".join(out) + "\n")
    print(json.dumps({"summary": fn, "variants": len(res), "fastest": res and min(res)[1]}))
    return 0


def inputs_shape(workload: str):
    from stage_pipelined_mainloop_amd import inputs
    M, N, K, _, _ = inputs.WORKLOADS[workload]
    return M, N, K


def mode_trace_summary(args) -> int:
    """Summarise a rocprofv3 kernel trace (CSV) of a bench.py run, given that
    run's JSON line: per kernel, dispatches and mean duration over all of
    them; for the step's kernel, the mean over exactly the timed dispatches
    (config.trace_window of the JSON line) and the roofline figure it gives,
    to set beside the run's own event timing.  Host-only, no GPU."""
    import csv
    import statistics
    line = None
    with open(args.bench_log) as f:
        for ln in f:
            ln = ln.strip()
            if ln.startswith("{") and '"metric"' in ln:
                line = json.loads(ln)
    if line is None:
        print(f"no bench JSON line in {args.bench_log}", file=sys.stderr)
        return 1
    cfgd = line["config"]
    M, N, K = cfgd["M"], cfgd["N"], cfgd["K"]
    win = cfgd["trace_window"]
    per = {}
    with open(args.trace) as f:
        for row in csv.DictReader(f):
            dur = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3   # us
            per.setdefault(row["Kernel_Name"], []).append((int(row["Start_Timestamp"]), dur))
    print("| kernel | dispatches | mean us (all) | median us | min us |")
    print("|---|---|---|---|---|")
    for name, v in sorted(per.items(), key=lambda kv: -sum(d for _, d in kv[1])):
        ds = [d for _, d in v]
        print(f"| `{name[:90]}` | {len(ds)} | {statistics.mean(ds):.2f} | "
              f"{statistics.median(ds):.2f} | {min(ds):.2f} |")
    hot = max(per, key=lambda k: sum(d for _, d in per[k]))
    seq = [d for _, d in sorted(per[hot])]
    window = seq[win["first"]:win["first"] + win["count"]]
    if len(window) != win["count"]:
        print(f"trace holds {len(seq)} dispatches of the step kernel; window {win} incomplete",
              file=sys.stderr)
        return 1
    mean_us = statistics.mean(window)
    roof = roofline_of(M, N, K, mean_us / 1e3)
    bench_us = cfgd["kernel_ms_mean"] * 1e3
    print()
    print(f"Timed window: dispatches {win['first']}..{win['first'] + win['count'] - 1} of `{hot[:90]}`: "
          f"mean {mean_us:.2f} us -> {roof['achieved']} {roof['unit']}, frac {roof['frac']} "
          f"(bench events: {bench_us:.2f} us, frac {line['roofline']['frac']}; "
          f"trace / events = {mean_us / bench_us:.4f})")
    return 0


def mode_dma_rate(args) -> int:
    """The copy side of the tiled kernels as a rate: bytes per shader cycle
    that one CU moves into LDS by LDS-DMA when every CU streams the 64-deep K
    tiles of its own A and B panels at once, with 1..4 tiles' loads in flight
    and nothing else running (the probe library's sg_probe_dma_rate).  Tiles
    of 128 rows per operand run on the M = N = 2048, K = 8192 sweep operands
    (a 16 x 16 grid, as the 128x128 kernels see it), tiles of 256 rows on the
    8192^3 operands, and again on the 8000 x 7936 x 8200 operands, whose rows
    start 16 bytes apart from one 128-byte line to the next, so that each
    row's 128 bytes of a K tile straddle two lines (K tiles past K / 64 are
    not streamed).  Each line also gives the MFMA-busy fraction that rate
    could feed at 4096 fp16 flop per CU and cycle (the dense peak per CU):
    2 x 128 x 128 x 64 flop per 32 KiB tile (64 flop per byte), 2 x 256 x 256
    x 64 per 64 KiB (128 flop per byte)."""
    import ctypes

    import numpy as np
    import torch

    from stage_pipelined_mainloop_amd import inputs
    so = os.path.join(ROOT, "stage_pipelined_mainloop_amd", "libsgprobe.so")
    P = ctypes.CDLL(so)
    P.sg_probe_dma_rate.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p,
                                    ctypes.c_longlong] + [ctypes.c_int] * 7 + [ctypes.c_void_p,
                                                                                ctypes.c_void_p]
    P.sg_probe_dma_rate.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    for rows, (A, B) in ((128, inputs.ksweep(8192)), (256, inputs.workload("square8192")),
                         (256, inputs.workload("ragged8000"))):
        M, K = A.shape
        N = B.shape[0]
        a, b = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
        tiles_m, tiles_n = M // rows, N // rows
        ntile = K // 64
        out = torch.zeros(cus * 16, dtype=torch.int64, device="cuda")
        fpb = 2.0 * rows * rows * 64 / (2 * rows * 128)
        for depth in (1, 2, 3, 4):
            def run():
                rc = P.sg_probe_dma_rate(a.data_ptr(), M, b.data_ptr(), N, K, rows, depth, tiles_m,
                                         tiles_n, cus, ntile, out.data_ptr(), stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"DMA rate probe failed to launch ({rc})")
            for _ in range(3):
                run()
            reps = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                run()
                e1.record(stream)
                torch.cuda.synchronize()
                r = out.view(cus, 4, 4).cpu().numpy().astype(np.float64)
                # a workgroup's tiles are in when its slowest wave's loads are
                cyc = r[:, :, 0].max(axis=1) / ntile
                reps.append((float(np.median(cyc)), e0.elapsed_time(e1)))
            cyc, ms = sorted(reps)[len(reps) // 2]
            tile_bytes = 2 * rows * 128
            rate = tile_bytes / cyc
            print(json.dumps({
                "mode": "dma_rate", "rows_per_operand": rows, "tiles_in_flight": depth,
                "operands": f"{M}x{K} and {N}x{K}", "workgroups": cus, "k_tiles": ntile,
                "cycles_per_k_tile": round(cyc, 1), "bytes_per_cycle_per_cu": round(rate, 2),
                "device_gbs": round(cus * ntile * tile_bytes / (ms / 1e3) / 1e9, 1),
                "mfma_busy_it_could_feed": round(min(1.0, rate * fpb / 4096.0), 3)}), flush=True)
        del a, b
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--mode", default="bench",
                    choices=["bench", "variants", "ksweep", "calibrate_copy", "attention",
                             "trace_summary", "stage_model", "profile_summary", "ksweep_summary",
                             "lds_patterns", "lds_summary", "variants_summary", "vendor_blas",
                             "forms", "forms_summary", "vendor_summary",
                             "attention_summary", "dma_rate"])
    ap.add_argument("--trace", default=None, help="kernel-trace CSV for --mode trace_summary")
    ap.add_argument("--bench-log", default=None, help="that run's output for --mode trace_summary")
    ap.add_argument("--prof-dir", default=None,
                    help="directory of rocprofv3 outputs for --mode profile_summary / ksweep_summary")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed launches first (default: about 100 ms of them, at least 30)")
    ap.add_argument("--workload", default="square8192")
    ap.add_argument("--config", default=None,
                    help="explicit variant tile_m,tile_n,tile_k,stages,waves,schedule")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--config-cpu-seconds", type=float, default=2.0,
                    help="oracle seconds per sampled CPU baseline of the other workloads")
    ap.add_argument("--no-per-config", action="store_true",
                    help="time only the headline workload (profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--heads", type=int, default=16, help="heads for --mode attention")
    ap.add_argument("--cold", action="store_true",
                    help="also time single launches after a 512 MiB cache flush")
    ap.add_argument("--graph", default="auto", choices=["auto", "on", "off"],
                    help="replay the timed steps as one captured HIP graph (auto: when "
                         "the host enqueues launches no faster than the GPU runs them)")
    args = ap.parse_args()
    auto_warmup = args.warmup is None
    if auto_warmup:
        args.warmup = 30

    if args.gpus != 1:
        print(f"bench.py measures one GPU (asked for {args.gpus}): the GEMM shards into "
              "independent output tiles (split M, broadcast B) with no exchange during "
              "compute, so N GPUs each run this one-GPU step on their share",
              file=sys.stderr)
        return 2
    if args.mode == "trace_summary":
        return mode_trace_summary(args)
    if args.mode == "stage_model":
        return mode_stage_model(args)
    if args.mode == "dma_rate":
        return mode_dma_rate(args)
    if args.mode == "profile_summary":
        return mode_profile_summary(args)
    if args.mode == "ksweep_summary":
        return mode_ksweep_summary(args)
    if args.mode == "lds_patterns":
        return mode_lds_patterns(args)
    if args.mode == "lds_summary":
        return mode_lds_summary(args)
    if args.mode == "variants_summary":
        return mode_variants_summary(args)
    if args.mode == "variants":
        return mode_variants(args)
    if args.mode == "vendor_blas":
        return mode_vendor_blas(args)
    if args.mode == "forms":
        return mode_forms(args)
    if args.mode == "forms_summary":
        return mode_forms_summary(args)
    if args.mode == "vendor_summary":
        return mode_vendor_summary(args)
    if args.mode == "attention_summary":
        return mode_attention_summary(args)
    if args.mode == "ksweep":
        return mode_ksweep(args)
    if args.mode == "calibrate_copy":
        return mode_calibrate_copy(args)
    if args.mode == "attention":
        return mode_attention(args)

    import numpy as np
    import torch

    import stage_pipelined_mainloop_amd as sg
    from stage_pipelined_mainloop_amd import inputs

    M, N, K, dist, seed = inputs.WORKLOADS[args.workload]
    A, B = inputs.workload(args.workload)
    alpha = float(np.float32(1.0 / math.sqrt(K))) if args.workload == "attn_scores" else None
    dev = torch.device("cuda:0")
    a = torch.from_numpy(A).to(dev)
    b = torch.from_numpy(B).to(dev)
    d = torch.empty((M, N), dtype=torch.float16, device=dev)
    cfg = tuple(int(x) for x in args.config.split(",")) if args.config else None
    if cfg:
        vname = variant_name(sg.SgConfig(*cfg))

        def step():
            sg.gemm(a, b, out=d, alpha=alpha, config=cfg)
    else:
        step, vname, _ = library_call(M, N, K, a, b, d, alpha)

    for _ in range(10):
        step()
    torch.cuda.synchronize()
    # 50 launches, so the one synchronisation at the end is a small part
    tw = time.perf_counter()
    for _ in range(50):
        step()
    enqueue = (time.perf_counter() - tw) / 50
    torch.cuda.synchronize()
    per = (time.perf_counter() - tw) / 50
    if auto_warmup:
        # about 100 ms of launches, so that the clock has settled before the
        # timed steps even for a kernel of a few microseconds
        args.warmup = max(30, min(20000, int(0.1 / max(per, 1e-6))))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # When Python and ctypes enqueue a launch no faster than the GPU runs it,
    # the GPU idles between kernels; then the K steps are captured once as a
    # HIP graph and the timed region replays it, so the events time the
    # kernels back to back.  Otherwise the launches stay eager: at 4096^3 the
    # replay measured 12 % slower than eager launches.
    graph = None
    if args.graph == "on" or (args.graph == "auto" and enqueue > 0.9 * per):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(args.steps):
                step()
        graph.replay()
        torch.cuda.synchronize()
        if args.graph == "auto":
            # the runtime can replay a graph of kernels of a few microseconds
            # slower than it runs eager launches (256^3: 8.4 against 4.6-6.2
            # us per launch): keep the graph only where it is faster
            tg = time.perf_counter()
            graph.replay()
            torch.cuda.synchronize()
            if (time.perf_counter() - tg) / args.steps >= per:
                graph = None

    # Timed region: the K steps back to back between one pair of HIP events
    # on the stream the kernels are launched on, plus the host wall clock.
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for _ in range(args.steps):
            step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean_launch_s = e0.elapsed_time(e1) / args.steps / 1e3
    # after the timed region: spread of single launches (each reading holds
    # the ~2.5 us event overhead), and optionally with cold caches
    med_ms, min_ms = launch_spread(step, min(args.steps, 30))
    cold = None
    if args.cold:
        flush_buf = torch.empty(512 * 1024 * 1024, dtype=torch.uint8, device=dev)
        cmed, cmin = launch_spread(step, min(args.steps, 30), flush=lambda: flush_buf.fill_(1))
        cold = {"flush": "512 MiB fill before each launch", "kernel_ms_median": round(cmed, 4),
                "kernel_ms_min": round(cmin, 4)}
        del flush_buf

    flops = 2.0 * M * N * K
    value = flops * args.steps / wall / 1e12
    achieved = flops / mean_launch_s / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4),
                "traffic": load_traffic(args.workload, vname), "traffic_kind": "l2_egress_bytes"}
    algo_bytes = 2.0 * (M * K + N * K + M * N)
    ridge = PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)          # ~315 flop/B
    if flops / algo_bytes < ridge:
        # below the ridge (attention scores, tall-skinny): bound by HBM traffic
        gbs = algo_bytes / mean_launch_s / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                    "traffic": load_traffic(args.workload, vname), "traffic_kind": "l2_egress_bytes"}

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": args.workload, "M": M, "N": N, "K": K, "dist": dist,
                   "alpha": alpha if alpha is not None else 1.0,
                   "variant": vname,
                   "pct_of_fp16_peak": round(100.0 * value / PEAK_TFLOPS, 2),
                   "launch": "one HIP graph of the timed steps" if graph is not None else "eager",
                   "kernel_ms_mean": round(mean_launch_s * 1e3, 4),
                   "kernel_ms_median_single": round(med_ms, 4),
                   "kernel_ms_min_single": round(min_ms, 4),
                   # dispatches of the step's kernel in this process before the
                   # timed ones (calibration, warm-up, graph check): a kernel
                   # trace of this run averages dispatches [first, first + steps)
                   "trace_window": {"first": 60 + args.warmup + (args.steps if graph is not None else 0),
                                    "count": args.steps}},
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if cold is not None:
        out["config"]["cold_cache"] = cold
    if roofline["bound"] == "mfma":
        # measured after the timed region so it does not heat the GPU first
        ceil = mfma_ceiling(a, b)
        out["config"]["mfma_ceiling_tflops"] = round(ceil, 1)
        out["config"]["frac_of_mfma_ceiling"] = round(achieved / ceil, 4)
        # the same loop on 16x16x32 MFMAs, which draw less power per flop
        # (the shape the large-shape kernel uses)
        ceil16 = mfma_ceiling(a, b, shape16=True)
        out["config"]["mfma_ceiling_16x16x32_tflops"] = round(ceil16, 1)
        out["config"]["frac_of_mfma_ceiling_16x16x32"] = round(achieved / ceil16, 4)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(A, B, args.cpu_seconds)
    if not args.no_per_config:
        del a, b, d, step
        out["per_config"] = per_config(args)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

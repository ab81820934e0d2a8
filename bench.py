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
               graph that the timed region replays); traffic = HBM
               bytes per launch from the committed rocprofv3 counter summary,
               or null if the kernel source changed since it was taken
  cpu_baseline the CPU oracle timed on a bounded row sample of the same
               workload, on this host's cores
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


# the sources that decide which GEMM kernel runs and what it does (the
# attention forward and the measurement probe are separate sources)
GEMM_SOURCES = ("gemm_kernel.hpp", "persistent_kernel.hpp", "shortk_kernel.hpp", "stagegemm.hip")


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "stage_pipelined_mainloop_amd", "csrc")
    for name in GEMM_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per launch from profiles/traffic_<workload>.json when it was
    measured on the current kernel source; otherwise None."""
    p = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_source_sha():
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
                          "info": variant_info(c)}), flush=True)
    return 0


def mode_ksweep(args) -> int:
    """M = N = 2048, K in the sweep list, every compiled stage count of the
    128x128x32 and 256x256x32 (8-wave) tiles; LDS bytes and occupancy from
    the library's query."""
    import torch

    import stage_pipelined_mainloop_amd as sg
    from stage_pipelined_mainloop_amd import inputs
    for K in inputs.KSWEEP_K:
        A, B = inputs.ksweep(K)
        a = torch.from_numpy(A).cuda()
        b = torch.from_numpy(B).cuda()
        M = N = inputs.KSWEEP_MN
        d = torch.empty((M, N), dtype=torch.float16, device="cuda")
        for c in sg.configs():
            if (c.tile_m, c.tile_n, c.waves) not in ((128, 128, 4), (256, 256, 8)) or not takes(c, K):
                continue
            mean = time_launches(lambda: sg.gemm(a, b, out=d, config=c), args.steps, args.warmup)
            t = 2.0 * M * N * K / (mean / 1e3) / 1e12
            gbs = 2.0 * (M * K + N * K + M * N) / (mean / 1e3) / 1e9
            print(json.dumps({"mode": "ksweep", "M": M, "N": N, "K": K,
                              "variant": c.as_tuple(), "ms_mean": round(mean, 4),
                              "tflops": round(t, 1), "pct_peak": round(100 * t / PEAK_TFLOPS, 2),
                              "hbm_gbs_compulsory": round(gbs, 1),
                              "info": variant_info(c)}), flush=True)
    return 0


def mode_attention(args) -> int:
    """The fused attention forward O = softmax(alpha Q K^T) V on H heads of
    the attention-score shape (M = N = 4096, d = 128, N(0,1) inputs), next to
    the unfused route on the same GPU: this library's GEMM for the scores,
    then torch's softmax and batched product (one JSON line per head count)."""
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
        flops = 4.0 * H * M * N * d
        tf = flops / (fused / 1e3) / 1e12
        print(json.dumps({"mode": "attention", "metric": "fused attention forward TFLOP/s (4 H M N d)",
                          "heads": H, "M": M, "N": N, "d": d, "splits": splits, "ms": round(fused, 4),
                          "ms_one_split": round(unsplit, 4),
                          "tflops": round(tf, 1),
                          "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_TFLOPS,
                                       "unit": "TFLOP/s", "frac": round(tf / PEAK_TFLOPS, 4)},
                          "unfused_ms": round(ref_ms, 4),
                          "unfused": "library GEMM for S, torch softmax (fp32) and bmm"}), flush=True)
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


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--mode", default="bench",
                    choices=["bench", "variants", "ksweep", "calibrate_copy", "attention"])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed launches first (default: about 100 ms of them, at least 30)")
    ap.add_argument("--workload", default="square8192")
    ap.add_argument("--config", default=None,
                    help="explicit variant tile_m,tile_n,tile_k,stages,waves,schedule")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
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
    if args.mode == "variants":
        return mode_variants(args)
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
    chosen = sg.SgConfig(*cfg) if cfg else sg.sg_select_config(M, N, K)

    def step():
        sg.gemm(a, b, out=d, alpha=alpha, config=cfg)

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
                "traffic": load_traffic(args.workload)}
    algo_bytes = 2.0 * (M * K + N * K + M * N)
    ridge = PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)          # ~315 flop/B
    if flops / algo_bytes < ridge:
        # below the ridge (attention scores, tall-skinny): bound by HBM traffic
        gbs = algo_bytes / mean_launch_s / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                    "traffic": load_traffic(args.workload)}

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
                   "variant": "x".join(str(v) for v in chosen.as_tuple()[:3])
                              + f" S{chosen.stages} w{chosen.waves} sched{chosen.schedule}",
                   "pct_of_fp16_peak": round(100.0 * value / PEAK_TFLOPS, 2),
                   "launch": "one HIP graph of the timed steps" if graph is not None else "eager",
                   "kernel_ms_mean": round(mean_launch_s * 1e3, 4),
                   "kernel_ms_median_single": round(med_ms, 4),
                   "kernel_ms_min_single": round(min_ms, 4)},
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
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

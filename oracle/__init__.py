"""Plain CPU oracle for the stage-pipelined half-precision TN GEMM.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__ and
the cpu_baseline leg of bench.py may import this package.  The product path
(stage_pipelined_mainloop_amd) never imports it, and this package never
imports the product path; the two share no code.  The only module both sides
use is the seeded input generator, which holds none of the method's
arithmetic.

Contents:
  _native   fp16 codec, fp64 and exact (128-bit integer) GEMM evaluations,
            and the fp64 attention forward, written in plain C (oracle.c)
            and loaded with ctypes;
  models    stage-count / LDS-footprint / occupancy model and the ring-buffer
            schedule simulator;
  check     the element-wise tolerance check.

Every function names the passage of the pages it follows in its own
docstring or source comment.  Parity is pinned by tests that check these
functions against values the pages print, closed forms, brute force and an
independent library routine, not against themselves.
"""
from ._native import (attention_f64, build, f16_to_f64, f64_to_f16, gemm_tn_exact, gemm_tn_exact_beta,
                      gemm_tn_f64, gemm_tn_f64_at, gemm_tn_f64_beta, gemm_tn_f64_rows,
                      num_threads)
from .check import CheckReport, check, ulp16
from .models import (blocks_per_unit, lds_bytes, loosest_persistent_wait_counts,
                     loosest_wait_counts, minimum_stages, schedule_cute_loads,
                     schedule_cute_multistage, schedule_persistent_loads, schedule_three_phase,
                     simulate, simulate_loads)

__all__ = [
    "attention_f64", "build", "f16_to_f64", "f64_to_f16", "gemm_tn_exact", "gemm_tn_exact_beta",
    "gemm_tn_f64", "gemm_tn_f64_beta",
    "gemm_tn_f64_at", "gemm_tn_f64_rows", "num_threads", "CheckReport", "check",
    "ulp16", "blocks_per_unit", "lds_bytes", "loosest_wait_counts", "minimum_stages",
    "schedule_cute_loads", "schedule_cute_multistage", "schedule_three_phase", "simulate",
    "simulate_loads", "loosest_persistent_wait_counts", "schedule_persistent_loads",
]

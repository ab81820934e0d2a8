"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module only draws random numbers and holds none of the GEMM's
arithmetic.  Every matrix is row-major, C-contiguous float16.

Recipe (fixed so that any run can be reproduced):
  * generator: numpy.random.Generator(PCG64(seed));
  * "uniform": i.i.d. uniform on [-1, 1) drawn in float64, then rounded to
    float16 by numpy's round-to-nearest-even cast;
  * "normal":  i.i.d. standard normal drawn in float64, then cast the same way.
"""
from __future__ import annotations

import numpy as np

# Workloads: name -> (M, N, K, distribution, seed of A; B uses seed + 1)
WORKLOADS = {
    "square256": (256, 256, 256, "uniform", 1),
    "square4096": (4096, 4096, 4096, "uniform", 3),
    "attn_scores": (4096, 4096, 128, "normal", 7),
    "square8192": (8192, 8192, 8192, "uniform", 9),
    "ragged8000": (8000, 7936, 8200, "uniform", 11),
    # the tall-skinny shape of the multistage page's own test run
    "tall81920": (81920, 256, 256, "uniform", 13),
}
KSWEEP_K = (128, 512, 2048, 8192, 16384)
KSWEEP_MN = 2048
KSWEEP_SEED = 5


def matrix(rows: int, cols: int, seed: int, dist: str = "uniform") -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed))
    if dist == "uniform":
        x = g.uniform(-1.0, 1.0, size=(rows, cols))
    elif dist == "normal":
        x = g.standard_normal(size=(rows, cols))
    else:
        raise ValueError(dist)
    return np.ascontiguousarray(x.astype(np.float16))


def operands(M: int, N: int, K: int, seed: int, dist: str = "uniform"):
    """A (M x K) from `seed`, B (N x K) from `seed + 1`."""
    return matrix(M, K, seed, dist), matrix(N, K, seed + 1, dist)


def workload(name: str):
    M, N, K, dist, seed = WORKLOADS[name]
    A, B = operands(M, N, K, seed, dist)
    return A, B


def ksweep(K: int):
    return operands(KSWEEP_MN, KSWEEP_MN, K, KSWEEP_SEED, "uniform")

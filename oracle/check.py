"""Element-wise tolerance check of a half-precision result against the oracle.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Bound (per element, D_ref from the oracle):
    |D - D_ref| <= 2 * ulp16(|D_ref|) + 1e-4 * sqrt(K)
with ulp16(x) = 2^(max(floor(log2 x), -14) - 10) for x > 0 and ulp16(0) = 2^-24,
the spacing of binary16 numbers at x (the subnormal spacing below 2^-14).
Every element of D must also be finite wherever D_ref is.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def ulp16(x: np.ndarray) -> np.ndarray:
    """Spacing of binary16 values at |x| (2^-24 at and below the subnormal range)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    out = np.full(a.shape, 2.0 ** -24)
    pos = a > 0
    e = np.floor(np.log2(a[pos]))
    # guard the floor(log2) against rounding just below a power of two
    e = np.where(np.exp2(e) > a[pos], e - 1, e)
    e = np.where(np.exp2(e + 1) <= a[pos], e + 1, e)
    out[pos] = np.exp2(np.maximum(e, -14.0) - 10.0)
    return out


@dataclass
class CheckReport:
    ok: bool
    count: int
    max_abs_err: float
    max_excess: float          # max of (|err| - bound); <= 0 when ok
    argmax: int                # flat index of the worst element (by excess)
    over_1ulp: int             # elements whose error exceeds 1 ulp16(|ref|)
    nonfinite: int             # non-finite results where the reference is finite
    bound_const: float

    def __str__(self) -> str:
        return (f"ok={self.ok} n={self.count} max|err|={self.max_abs_err:.3g} "
                f"max_excess={self.max_excess:.3g} at {self.argmax} "
                f">1ulp={self.over_1ulp} nonfinite={self.nonfinite}")


def check(d: np.ndarray, d_ref: np.ndarray, K: int) -> CheckReport:
    d64 = np.asarray(d, dtype=np.float16).astype(np.float64).ravel()
    r64 = np.asarray(d_ref, dtype=np.float16).astype(np.float64).ravel()
    assert d64.shape == r64.shape
    if d64.size == 0:
        return CheckReport(True, 0, 0.0, 0.0, -1, 0, 0, 1e-4 * np.sqrt(max(K, 0)))
    ref_finite = np.isfinite(r64)
    nonfinite = int(np.count_nonzero(ref_finite & ~np.isfinite(d64)))
    err = np.abs(d64 - r64)
    err = np.where(ref_finite, err, np.where(d64 == r64, 0.0, np.inf))
    u = ulp16(np.where(ref_finite, r64, 0.0))
    const = 1e-4 * np.sqrt(max(K, 0))
    bound = 2.0 * u + const
    excess = err - bound
    k = int(np.nanargmax(np.where(np.isnan(excess), np.inf, excess)))
    over1 = int(np.count_nonzero(err > u))
    ok = bool(np.all(excess <= 0)) and nonfinite == 0 and not np.any(np.isnan(d64) & ~np.isnan(r64))
    return CheckReport(ok, int(d64.size), float(np.max(err)), float(excess[k]), k,
                       over1, nonfinite, const)

"""ctypes wrapper around the plain C oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the product path.

The shared object is built with the system C compiler (no HIP, no GPU code).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# IEEE semantics are required: no -ffast-math; contraction off so every
# product and sum is the separately rounded fp64 operation the source shows.
CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
          "-Wall", "-Wextra"]


# Address and undefined-behaviour sanitizers for a checking build of the same
# source (run by the test suite with the sanitizer runtimes preloaded).
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                  "-fno-omit-frame-pointer", "-g"]

# A test run may point the loader at another build of oracle.c (the
# sanitized one) through this variable.
LIBRARY_ENV = "SGO_LIBRARY"


def build(force: bool = True, out: str | None = None, sanitize: bool = False) -> str:
    """Compile oracle.c into liboracle.so next to it (or into `out`) and
    return the path.  sanitize=True adds SANITIZE_FLAGS."""
    target = out or _LIB
    if force or not os.path.exists(target):
        tmp = target + ".tmp"
        cmd = ["gcc", *CFLAGS, *(SANITIZE_FLAGS if sanitize else []), _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, target)
    return target


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        path = os.environ.get(LIBRARY_ENV) or _LIB
        if path == _LIB and not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(path)
        u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
        f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
        i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
        L.sgo_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.sgo_f16_to_f64.restype = ctypes.c_double
        L.sgo_f64_to_f16.argtypes = [ctypes.c_double]
        L.sgo_f64_to_f16.restype = ctypes.c_uint16
        L.sgo_f16_to_f64_array.argtypes = [u16p, f64p, ctypes.c_long]
        L.sgo_f16_to_f64_array.restype = None
        L.sgo_f64_to_f16_array.argtypes = [f64p, u16p, ctypes.c_long]
        L.sgo_f64_to_f16_array.restype = None
        L.sgo_gemm_tn_f64.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_float, u16p, u16p, u16p]
        L.sgo_gemm_tn_f64.restype = None
        L.sgo_gemm_tn_f64_at.argtypes = [ctypes.c_int, ctypes.c_float, u16p, u16p,
                                         ctypes.c_long, i32p, i32p, u16p]
        L.sgo_gemm_tn_f64_at.restype = None
        L.sgo_gemm_tn_f64_rows.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                           u16p, u16p, ctypes.c_int, ctypes.c_int, u16p]
        L.sgo_gemm_tn_f64_rows.restype = None
        L.sgo_gemm_tn_exact.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_float, u16p, u16p, u16p]
        L.sgo_gemm_tn_exact.restype = ctypes.c_int
        L.sgo_gemm_tn_f64_beta.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_float, ctypes.c_float, u16p, u16p,
                                           ctypes.c_void_p, u16p]
        L.sgo_gemm_tn_f64_beta.restype = None
        L.sgo_gemm_tn_exact_beta.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_float, ctypes.c_float, u16p, u16p,
                                             ctypes.c_void_p, u16p]
        L.sgo_gemm_tn_exact_beta.restype = ctypes.c_int
        L.sgo_attention_f64.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_float, u16p, u16p, u16p, u16p, ctypes.c_void_p]
        L.sgo_attention_f64.restype = None
        L.sgo_num_threads.argtypes = []
        L.sgo_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _bits(x: np.ndarray) -> np.ndarray:
    """fp16 array (or its uint16 bit view) as C-contiguous uint16 bits."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float16:
        return x.view(np.uint16)
    if x.dtype == np.uint16:
        return x
    raise TypeError(f"expected float16 or uint16 bits, got {x.dtype}")


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = _bits(np.asarray(bits)).ravel()
    out = np.empty(b.size, np.float64)
    lib().sgo_f16_to_f64_array(b, out, b.size)
    return out.reshape(np.shape(bits))


def f64_to_f16(x: np.ndarray) -> np.ndarray:
    """Round to binary16 (RNE); returns uint16 bit patterns."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(a.size, np.uint16)
    lib().sgo_f64_to_f16_array(a.ravel(), out, a.size)
    return out.reshape(a.shape)


def gemm_tn_f64(A, B, alpha: float = 1.0) -> np.ndarray:
    """D = RNE16(alpha * A @ B.T), fp64 accumulation in index order.

    A: (M, K) fp16, B: (N, K) fp16.  Returns D as (M, N) float16."""
    a, b = _bits(A), _bits(B)
    M, K = a.shape
    N, K2 = b.shape
    assert K == K2
    d = np.empty((M, N), np.uint16)
    if M and N:
        lib().sgo_gemm_tn_f64(M, N, K, float(alpha), a, b, d)
    return d.view(np.float16)


def gemm_tn_f64_at(A, B, rows, cols, alpha: float = 1.0) -> np.ndarray:
    """The same definition evaluated at the (rows[t], cols[t]) pairs only."""
    a, b = _bits(A), _bits(B)
    M, K = a.shape
    N, K2 = b.shape
    assert K == K2
    r = np.ascontiguousarray(rows, dtype=np.int32).ravel()
    c = np.ascontiguousarray(cols, dtype=np.int32).ravel()
    assert r.size == c.size
    if r.size:
        assert r.min() >= 0 and r.max() < M and c.min() >= 0 and c.max() < N
    out = np.empty(r.size, np.uint16)
    if r.size:
        lib().sgo_gemm_tn_f64_at(K, float(alpha), a, b, r.size, r, c, out)
    return out.view(np.float16)


def gemm_tn_f64_rows(A, B, r0: int, r1: int, alpha: float = 1.0) -> np.ndarray:
    """Rows [r0, r1) of D (used to time the oracle on a bounded sample)."""
    a, b = _bits(A), _bits(B)
    M, K = a.shape
    N, _ = b.shape
    assert 0 <= r0 <= r1 <= M
    out = np.empty((r1 - r0, N), np.uint16)
    if r1 > r0 and N:
        lib().sgo_gemm_tn_f64_rows(N, K, float(alpha), a, b, r0, r1, out)
    return out.view(np.float16)


def gemm_tn_exact(A, B, alpha: float = 1.0) -> np.ndarray:
    """Exact (128-bit integer) evaluation of RNE16(alpha * A @ B.T)."""
    a, b = _bits(A), _bits(B)
    M, K = a.shape
    N, K2 = b.shape
    assert K == K2
    d = np.empty((M, N), np.uint16)
    if M and N:
        rc = lib().sgo_gemm_tn_exact(M, N, K, float(alpha), a, b, d)
        if rc != 0:
            raise ValueError(f"exact oracle refused the input (code {rc})")
    return d.view(np.float16)


def _c_arg(C, M, N, beta):
    if beta == 0.0:
        return None, None
    c = _bits(C)
    assert c.shape == (M, N)
    return c, c.ctypes.data


def gemm_tn_f64_beta(A, B, C, alpha: float = 1.0, beta: float = 0.0) -> np.ndarray:
    """D = RNE16(alpha * A @ B.T + beta * C); C is not read when beta == 0."""
    a, b = _bits(A), _bits(B)
    M, K = a.shape
    N, K2 = b.shape
    assert K == K2
    keep, cptr = _c_arg(C, M, N, float(np.float32(beta)))
    d = np.empty((M, N), np.uint16)
    if M and N:
        lib().sgo_gemm_tn_f64_beta(M, N, K, float(alpha), float(beta), a, b, cptr, d)
    del keep
    return d.view(np.float16)


def gemm_tn_exact_beta(A, B, C, alpha: float = 1.0, beta: float = 0.0) -> np.ndarray:
    """Exact (128-bit integer) RNE16(alpha * A @ B.T + beta * C)."""
    a, b = _bits(A), _bits(B)
    M, K = a.shape
    N, K2 = b.shape
    assert K == K2
    keep, cptr = _c_arg(C, M, N, float(np.float32(beta)))
    d = np.empty((M, N), np.uint16)
    if M and N:
        rc = lib().sgo_gemm_tn_exact_beta(M, N, K, float(alpha), float(beta), a, b, cptr, d)
        if rc != 0:
            raise ValueError(f"exact oracle refused the input (code {rc})")
    del keep
    return d.view(np.float16)


def attention_f64(Q, K, V, alpha: float, with_bound: bool = False):
    """O = RNE16(softmax(alpha * Q K^T) V), row-wise softmax, fp64 inside.

    Q: (H, M, d) or (M, d); K, V: (H, N, d) or (N, d), fp16.  Returns O with
    Q's shape (float16), and with `with_bound` also the per-element weight
    sum_j p_j |v_jc| (float64)."""
    q, k, v = _bits(Q), _bits(K), _bits(V)
    squeeze = q.ndim == 2
    if squeeze:
        q, k, v = q[None], k[None], v[None]
    H, M, d = q.shape
    Hk, N, dk = k.shape
    assert (Hk, dk) == (H, d) and v.shape == k.shape and N >= 1
    q, k, v = (np.ascontiguousarray(x) for x in (q, k, v))
    o = np.empty((H, M, d), np.uint16)
    wb = np.empty((H, M, d), np.float64) if with_bound else None
    if H and M and d:
        lib().sgo_attention_f64(H, M, N, d, float(alpha), q, k, v, o,
                                wb.ctypes.data if wb is not None else None)
    o = o.view(np.float16)
    if squeeze:
        o = o[0]
        wb = wb[0] if wb is not None else None
    return (o, wb) if with_bound else o


def num_threads() -> int:
    return int(lib().sgo_num_threads())

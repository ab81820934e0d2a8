"""Pins of the oracle's beta variant, D = RNE16(alpha * A @ B^T + beta * C)
("CUDA operator notes 2", section "GEMM": C = alpha A B + beta C), against
closed forms, the exact evaluation and the plain variant."""
import numpy as np
import pytest

import oracle
from stage_pipelined_mainloop_amd import inputs


def test_beta_zero_ignores_c_even_nan():
    A, B = inputs.operands(40, 48, 72, 401)
    C = np.full((40, 48), np.nan, np.float16)
    d = oracle.gemm_tn_f64_beta(A, B, C, 0.75, 0.0)
    assert np.array_equal(d.view(np.uint16), oracle.gemm_tn_f64(A, B, 0.75).view(np.uint16))


@pytest.mark.parametrize("beta", [1.0, -0.5, 0.3, 1e-3])
def test_alpha_zero_is_rounded_beta_c(beta):
    # beta (fp32) times c (fp16) is exact in fp64, so numpy's single RNE cast
    # of that product is the closed form
    A, B = inputs.operands(33, 24, 40, 403)
    C = inputs.matrix(33, 24, 405)
    b32 = float(np.float32(beta))
    d = oracle.gemm_tn_f64_beta(A, B, C, 0.0, b32)
    ref = (b32 * C.astype(np.float64)).astype(np.float16)
    assert np.array_equal(d.astype(np.float64), ref.astype(np.float64))


@pytest.mark.parametrize("alpha,beta", [(1.0, 1.0), (0.5, -2.0), (-1.25, 0.375), (1.0 / 3.0, 0.1)])
def test_f64_equals_exact_small_shapes(alpha, beta):
    g = np.random.Generator(np.random.PCG64(407))
    a32, b32 = float(np.float32(alpha)), float(np.float32(beta))
    for _ in range(30):
        M, N, K = (int(v) for v in g.integers(1, 24, size=3))
        A = g.uniform(-1, 1, (M, K)).astype(np.float16)
        B = g.uniform(-1, 1, (N, K)).astype(np.float16)
        C = g.uniform(-4, 4, (M, N)).astype(np.float16)
        d1 = oracle.gemm_tn_f64_beta(A, B, C, a32, b32)
        d2 = oracle.gemm_tn_exact_beta(A, B, C, a32, b32)
        assert np.array_equal(d1.astype(np.float64), d2.astype(np.float64)), (M, N, K)


def test_in_place_cancellation_is_exact_zero():
    # B = I, C = A: alpha * A + beta * A with beta = -alpha cancels exactly
    K = 64
    A, _ = inputs.operands(50, K, K, 409)
    eye = np.eye(K, dtype=np.float16)
    d = oracle.gemm_tn_f64_beta(A, eye, A, 1.0, -1.0)
    assert np.all(d.astype(np.float64) == 0.0)
    d = oracle.gemm_tn_exact_beta(A, eye, A, 0.5, -0.5)
    assert np.all(d.astype(np.float64) == 0.0)


def test_beta_one_adds_a_second_product():
    # D = A1 B1^T + C with C = A2 B2^T evaluated exactly in fp16 only when the
    # sum is exact: use small integers so every value is representable
    g = np.random.Generator(np.random.PCG64(411))
    A1 = g.integers(-3, 4, (20, 16)).astype(np.float16)
    B1 = g.integers(-3, 4, (12, 16)).astype(np.float16)
    C = g.integers(-50, 51, (20, 12)).astype(np.float16)
    d = oracle.gemm_tn_f64_beta(A1, B1, C, 1.0, 1.0)
    ref = A1.astype(np.int64) @ B1.astype(np.int64).T + C.astype(np.int64)
    assert np.array_equal(d.astype(np.float64), ref.astype(np.float64))

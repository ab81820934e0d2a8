"""Pins of the oracle's GEMM (D = RNE16(alpha * A @ B^T)) against things other
than itself: exact rational brute force, closed forms (identity, permutation,
rank one), an independent library routine (numpy's fp64 matmul), the
attention worked example of "CUDA operator notes 2", and moments of the
output distribution."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from stage_pipelined_mainloop_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_f16(g, shape, kind="uniform"):
    if kind == "uniform":
        return g.uniform(-1, 1, size=shape).astype(np.float16)
    if kind == "wide":
        # signs, zeros, subnormals and large magnitudes (products stay finite)
        mant = g.uniform(-1, 1, size=shape)
        expo = g.integers(-26, 8, size=shape)
        x = (mant * np.exp2(expo)).astype(np.float16)
        x[g.random(shape) < 0.05] = 0.0
        x[g.random(shape) < 0.03] = -0.0
        return x
    raise ValueError(kind)


def _nearest_f16_check(value: Fraction, got: np.float16) -> bool:
    """True if `got` is a binary16 nearest to the exact `value`, with ties
    resolved to the even fraction field.  Uses only exact rational
    arithmetic and numpy's nextafter to enumerate neighbours."""
    g = np.float16(got)
    if not np.isfinite(g):
        return abs(value) >= 65520
    cands = {float(g), float(np.nextafter(g, np.float16(np.inf))),
             float(np.nextafter(g, np.float16(-np.inf)))}
    cands = [c for c in cands if math.isfinite(c)]
    dist = {c: abs(Fraction(c) - value) for c in cands}
    best = min(dist.values())
    if dist[float(g)] != best:
        return False
    ties = [c for c in cands if dist[c] == best]
    if len(ties) > 1:
        even = [c for c in ties if int(np.float16(c).view(np.uint16)) & 1 == 0]
        return float(g) in even
    return True


@pytest.mark.parametrize("seed", range(6))
def test_exact_matches_rational_brute_force(seed):
    g = np.random.Generator(np.random.PCG64(100 + seed))
    for _ in range(20):
        M, N, K = (int(v) for v in g.integers(1, 6, size=3))
        A = _rand_f16(g, (M, K), "wide")
        B = _rand_f16(g, (N, K), "wide")
        alpha = float(np.float32(g.choice([1.0, 0.5, -0.375, 1 / 3, 3.0])))
        D = oracle.gemm_tn_exact(A, B, alpha)
        for i in range(M):
            for j in range(N):
                s = sum(Fraction(float(A[i, k])) * Fraction(float(B[j, k])) for k in range(K))
                v = Fraction(alpha) * s
                assert _nearest_f16_check(v, D[i, j]), (M, N, K, i, j, v, D[i, j])


@pytest.mark.parametrize("kind", ["uniform", "wide"])
@pytest.mark.parametrize("alpha", [1.0, -1.0, -0.375])
def test_f64_equals_exact_on_all_tiny_shapes(kind, alpha):
    # bit patterns, so the sign of every zero is compared too (K = 0 included)
    g = np.random.Generator(np.random.PCG64(7))
    for M in range(1, 9):
        for N in range(1, 9):
            for K in range(0, 9):
                A = _rand_f16(g, (M, K), kind)
                B = _rand_f16(g, (N, K), kind)
                d1 = oracle.gemm_tn_f64(A, B, alpha)
                d2 = oracle.gemm_tn_exact(A, B, alpha)
                assert np.array_equal(d1.view(np.uint16), d2.view(np.uint16)), (M, N, K, alpha)


def test_f64_equals_exact_random_shapes_to_64():
    g = np.random.Generator(np.random.PCG64(8))
    for _ in range(40):
        M, N, K = (int(v) for v in g.integers(1, 65, size=3))
        A = _rand_f16(g, (M, K))
        B = _rand_f16(g, (N, K))
        alpha = float(np.float32(g.choice([1.0, 0.125, 1 / math.sqrt(128), -0.5, -3.0])))
        d1 = oracle.gemm_tn_f64(A, B, alpha)
        d2 = oracle.gemm_tn_exact(A, B, alpha)
        assert np.array_equal(d1.view(np.uint16), d2.view(np.uint16)), (M, N, K, alpha)


@pytest.mark.parametrize("alpha", [1.0, -1.0, -0.125, 0.0, -0.0])
def test_exactly_zero_sums_are_plus_zero(alpha):
    # The real sum 0 has no sign and round-to-nearest gives +0 for it, for any
    # alpha: the empty sum (K = 0), an all-zero row, signed zeros in the
    # operands and a row whose products cancel exactly.  A nonzero negative
    # value too small for binary16 still rounds to -0.
    A = np.zeros((4, 8), np.float16)
    A[1] = -0.0
    A[2] = [0, 1, -1, 2, -2, 0.5, -0.5, 0]        # products with B row 0 cancel
    A[3, 0] = np.float16(2.0 ** -14)
    B = np.zeros((2, 8), np.float16)
    B[0] = 1.0
    B[1, 0] = np.float16(-2.0 ** -14)             # A[3] . B[1] = -2^-28
    want = np.zeros((4, 2), np.uint16)
    if alpha != 0:
        want[3, 0] = np.float16(alpha * 2.0 ** -14).view(np.uint16)   # exact in binary16
        if alpha > 0:
            want[3, 1] = 0x8000                   # -2^-28 * alpha rounds to -0
    for f in (oracle.gemm_tn_f64, oracle.gemm_tn_exact):
        d = f(A, B, alpha).view(np.uint16)
        assert np.array_equal(d, want), (alpha, d, want)
        d0 = f(np.zeros((3, 0), np.float16), np.zeros((5, 0), np.float16), alpha)
        assert np.array_equal(d0.view(np.uint16), np.zeros((3, 5), np.uint16)), alpha
    # beta: alpha * 0 = -0 and beta * c = -0 still give +0
    C = np.full((2, 2), -0.0, np.float16)
    for f in (oracle.gemm_tn_f64_beta, oracle.gemm_tn_exact_beta):
        d = f(A[:2], B, C, alpha, 1.0).view(np.uint16)
        assert np.array_equal(d, np.zeros((2, 2), np.uint16)), (alpha, d)


def test_f64_against_numpy_matmul():
    # numpy's fp64 matmul sums in a different order; after rounding to fp16
    # the two may differ only where the exact sum sits at a rounding tie.
    A, B = inputs.operands(96, 80, 200, 21)
    d = oracle.gemm_tn_f64(A, B).astype(np.float64)
    ref = (A.astype(np.float64) @ B.astype(np.float64).T).astype(np.float16).astype(np.float64)
    diff = d != ref
    assert diff.sum() <= 2
    if diff.any():
        assert np.all(np.abs(d - ref)[diff] <= oracle.ulp16(ref[diff]))


def test_identity_and_transposed_identity():
    A, B = inputs.operands(37, 24, 24, 31)
    eye = np.eye(24, dtype=np.float16)
    # B = I_K  ->  D = A exactly
    assert np.array_equal(oracle.gemm_tn_f64(A, eye).view(np.uint16), A.view(np.uint16))
    # A = I_K  ->  D = B^T exactly
    assert np.array_equal(oracle.gemm_tn_f64(eye, B).view(np.uint16),
                          np.ascontiguousarray(B.T).view(np.uint16))


def test_permutation_gives_permuted_columns_of_A():
    g = np.random.Generator(np.random.PCG64(5))
    K = 40
    A, _ = inputs.operands(29, K, K, 41)
    perm = g.permutation(K)
    P = np.zeros((K, K), np.float16)
    P[np.arange(K), perm] = 1.0            # B[j][perm[j]] = 1
    D = oracle.gemm_tn_f64(A, P)
    assert np.array_equal(D.view(np.uint16), A[:, perm].view(np.uint16))
    assert np.array_equal(oracle.gemm_tn_exact(A, P).view(np.uint16), A[:, perm].view(np.uint16))


@pytest.mark.parametrize("K", [1, 7, 2048, 2049, 8200])
def test_all_ones_gives_K(K):
    A = np.ones((3, K), np.float16)
    B = np.ones((5, K), np.float16)
    D = oracle.gemm_tn_f64(A, B)
    expect = np.float16(K)          # 2049 is a tie -> 2048; 8200 is representable
    assert np.all(D == expect)
    assert np.all(oracle.gemm_tn_exact(A, B) == expect)


def test_rank_one_powers_of_two_closed_form():
    g = np.random.Generator(np.random.PCG64(77))
    M, N, K = 9, 11, 300
    u = g.choice([-1, 1], M) * np.exp2(g.integers(-3, 3, M))
    v = g.choice([-1, 1], N) * np.exp2(g.integers(-3, 3, N))
    x = g.choice([-1, 1], K) * np.exp2(g.integers(-6, 1, K))
    y = g.choice([-1, 1], K) * np.exp2(g.integers(-6, 1, K))
    A = np.outer(u, x).astype(np.float16)
    B = np.outer(v, y).astype(np.float16)
    assert np.array_equal(A.astype(np.float64), np.outer(u, x))   # all exact
    # x.y as an exact rational, then D_ij = u_i v_j (x.y) rounded once
    xy = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x, y))
    D = oracle.gemm_tn_f64(A, B)
    for i in range(M):
        for j in range(N):
            assert _nearest_f16_check(Fraction(float(u[i])) * Fraction(float(v[j])) * xy, D[i, j])


def test_alpha_one_and_powers_of_two():
    A, B = inputs.operands(48, 40, 96, 51)
    d = oracle.gemm_tn_f64(A, B)
    assert np.array_equal(oracle.gemm_tn_f64(A, B, 1.0).view(np.uint16), d.view(np.uint16))
    for j in (1, 2, 5):
        dj = oracle.gemm_tn_f64(A, B, 2.0 ** -j).astype(np.float64)
        # exact scaling while the result stays in the normal range
        big = np.abs(d.astype(np.float64)) * 2.0 ** -j >= 2.0 ** -14
        assert np.array_equal(dj[big], d.astype(np.float64)[big] * 2.0 ** -j)


def test_attention_worked_example():
    with open(os.path.join(GOLDEN, "attention_example.json")) as f:
        ex = json.load(f)
    Q = np.array(ex["Q"], np.float16)
    Kt = np.array(ex["K"], np.float16)
    V = np.array(ex["V"], np.float64)
    d = Q.shape[1]
    alpha = float(np.float32(1.0 / math.sqrt(d)))
    S = oracle.gemm_tn_f64(Q, Kt, alpha).astype(np.float64)
    assert np.array_equal(S, np.array([[0.5, 0, 0], [0, 0.5, 0]]))
    # row-wise softmax and P V, computed here in fp64 only to reach the
    # printed output of the page
    P = np.exp(S - S.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    O = P @ V
    assert np.array_equal(np.round(O, ex["printed_decimals"]), np.array(ex["O_printed"]))


def test_moments_of_uniform_products():
    # entries uniform on [-1, 1]: E[a b] = 0, Var[sum of K products] = K / 9
    M = N = 192
    K = 1024
    A, B = inputs.operands(M, N, K, 61)
    D = oracle.gemm_tn_f64(A, B).astype(np.float64)
    assert abs(D.mean()) < 0.05 * math.sqrt(K / 9)
    assert abs(D.var() / (K / 9) - 1.0) < 0.05


def test_sampled_and_row_evaluations_agree_with_full():
    A, B = inputs.operands(70, 50, 64, 71)
    full = oracle.gemm_tn_f64(A, B, 0.75)
    g = np.random.Generator(np.random.PCG64(9))
    r = g.integers(0, 70, 300)
    c = g.integers(0, 50, 300)
    assert np.array_equal(oracle.gemm_tn_f64_at(A, B, r, c, 0.75).view(np.uint16),
                          full[r, c].view(np.uint16))
    assert np.array_equal(oracle.gemm_tn_f64_rows(A, B, 13, 29, 0.75).view(np.uint16),
                          full[13:29].view(np.uint16))


def test_empty_sum_is_positive_zero():
    A = np.zeros((4, 0), np.float16)
    B = np.zeros((3, 0), np.float16)
    for f in (oracle.gemm_tn_f64, oracle.gemm_tn_exact):
        D = f(A, B)
        assert D.shape == (4, 3)
        assert np.all(D.view(np.uint16) == 0)


def test_tolerance_check_detects_planted_errors():
    A, B = inputs.operands(64, 64, 512, 81)
    ref = oracle.gemm_tn_f64(A, B)
    assert oracle.check(ref, ref, 512).ok
    bad = ref.copy()
    bad[3, 7] = np.float16(float(bad[3, 7]) + 0.1)
    rep = oracle.check(bad, ref, 512)
    assert not rep.ok and rep.argmax == 3 * 64 + 7
    bad = ref.copy()
    bad[5, 5] = np.float16(np.nan)
    assert not oracle.check(bad, ref, 512).ok


def test_ulp16_values():
    x = np.array([0.0, 2.0 ** -24, 2.0 ** -15, 2.0 ** -14, 1.0, 1.5, 1024.0, 65504.0])
    assert list(oracle.ulp16(x)) == [2.0 ** -24, 2.0 ** -24, 2.0 ** -24, 2.0 ** -24,
                                     2.0 ** -10, 2.0 ** -10, 1.0, 32.0]

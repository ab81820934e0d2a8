"""Pins of the oracle's attention forward, O = softmax(alpha Q K^T) V with a
row-wise softmax ("CUDA operator notes 2", section "Softmax Attention"),
against the page's printed example, closed forms, invariances and an
independent library softmax."""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
from stage_pipelined_mainloop_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def ulp16(x):
    return oracle.ulp16(np.abs(np.asarray(x, np.float64)))


def test_printed_example():
    # the page's Q (2x4), K and V (3x4), scale 1/sqrt(d); its printed O to
    # two decimals (tests/golden/attention_example.json)
    with open(os.path.join(GOLDEN, "attention_example.json")) as f:
        ex = json.load(f)
    Q = np.array(ex["Q"], np.float16)
    K = np.array(ex["K"], np.float16)
    V = np.array(ex["V"], np.float16)
    alpha = float(np.float32(1.0 / math.sqrt(Q.shape[1])))
    O = oracle.attention_f64(Q, K, V, alpha).astype(np.float64)
    assert np.array_equal(np.round(O, ex["printed_decimals"]), np.array(ex["O_printed"]))


def test_one_key_returns_its_value_row():
    # softmax over a single key is 1: O = v exactly
    g = np.random.Generator(np.random.PCG64(3001))
    Q = g.standard_normal((3, 17, 32)).astype(np.float16)
    K = g.standard_normal((3, 1, 32)).astype(np.float16)
    V = g.standard_normal((3, 1, 32)).astype(np.float16)
    O = oracle.attention_f64(Q, K, V, 0.25)
    assert np.array_equal(O.view(np.uint16), np.broadcast_to(V, O.shape).view(np.uint16))


def test_equal_scores_average_the_values():
    # alpha = 0 (or identical keys): uniform weights, O = mean of the V rows
    A, V = inputs.operands(40, 24, 16, 3003)
    Kk = inputs.matrix(24, 16, 3005)
    mean = V.astype(np.float64).mean(axis=0)
    O = oracle.attention_f64(A, Kk, V, 0.0).astype(np.float64)
    assert np.all(np.abs(O - mean) <= 0.5 * ulp16(mean) + 1e-15)
    Ksame = np.repeat(Kk[:1], 24, axis=0)
    O2 = oracle.attention_f64(A, Ksame, V, 0.7).astype(np.float64)
    assert np.all(np.abs(O2 - mean) <= 0.5 * ulp16(mean) + 1e-15)


def test_dominant_key_selects_its_value():
    # q aligned with key j* and a large scale: every other weight is below
    # e^-60, so O rounds to v_{j*}
    g = np.random.Generator(np.random.PCG64(3007))
    N, d = 50, 16
    K = g.choice([-1.0, 1.0], (N, d)).astype(np.float16)
    V = g.standard_normal((N, d)).astype(np.float16)
    js = [3, 17, 49]
    Q = K[js]
    O = oracle.attention_f64(Q, K, V, 30.0)
    # scores: d * 30 for j*, at most (d - 2) * 30 for any other key
    assert np.array_equal(O.view(np.uint16), V[js].view(np.uint16))


def test_key_value_permutation_invariance():
    Q, K = inputs.operands(30, 64, 32, 3009, "normal")
    V = inputs.matrix(64, 32, 3011, "normal")
    perm = np.random.Generator(np.random.PCG64(3013)).permutation(64)
    O1 = oracle.attention_f64(Q, K, V, 0.2).astype(np.float64)
    O2 = oracle.attention_f64(Q, K[perm], V[perm], 0.2).astype(np.float64)
    # same value up to fp64 summation order; after the fp16 rounding at most
    # one ulp apart (at a rounding tie)
    assert np.all(np.abs(O1 - O2) <= ulp16(O1))


def test_matches_library_softmax():
    # an independent evaluation: scipy's softmax and numpy's matmul in fp64
    g = np.random.Generator(np.random.PCG64(3015))
    for (H, M, N, d) in [(2, 9, 33, 16), (1, 40, 100, 64), (3, 5, 7, 8)]:
        Q = g.standard_normal((H, M, d)).astype(np.float16)
        K = g.standard_normal((H, N, d)).astype(np.float16)
        V = g.standard_normal((H, N, d)).astype(np.float16)
        alpha = float(np.float32(1.0 / math.sqrt(d)))
        O, wb = oracle.attention_f64(Q, K, V, alpha, with_bound=True)
        S = alpha * np.einsum("hmd,hnd->hmn", Q.astype(np.float64), K.astype(np.float64))
        P = scipy.special.softmax(S, axis=-1)
        ref = np.einsum("hmn,hnd->hmd", P, V.astype(np.float64))
        O = O.astype(np.float64)
        assert np.all(np.abs(O - ref) <= 0.5 * ulp16(ref) * (1 + 1e-9) + 1e-12), (H, M, N, d)
        wref = np.einsum("hmn,hnd->hmd", P, np.abs(V.astype(np.float64)))
        assert np.allclose(wb, wref, rtol=1e-12, atol=0)
        assert np.all(wb + 1e-12 >= np.abs(ref))


def test_heads_are_independent():
    g = np.random.Generator(np.random.PCG64(3017))
    Q = g.standard_normal((4, 12, 16)).astype(np.float16)
    K = g.standard_normal((4, 20, 16)).astype(np.float16)
    V = g.standard_normal((4, 20, 16)).astype(np.float16)
    O = oracle.attention_f64(Q, K, V, 0.3)
    for h in range(4):
        assert np.array_equal(O[h].view(np.uint16),
                              oracle.attention_f64(Q[h], K[h], V[h], 0.3).view(np.uint16))


def _exact_rounded(Q, K, V, alpha):
    """O rounded once to fp16 from a 60-digit evaluation of the definition
    (decimal module: exact products and sums of the fp16 inputs, exp to 60
    digits); None where the value lies within 1e-12 (relative) of an fp16
    rounding midpoint, where the oracle's fp64 evaluation (error far below
    that) may legitimately round either way."""
    import decimal
    from decimal import Decimal
    ctx = decimal.Context(prec=60)
    M, d = Q.shape
    N = K.shape[0]
    a = Decimal(float(alpha))
    out = np.empty((M, d), dtype=object)
    for i in range(M):
        s = [ctx.multiply(a, sum((Decimal(float(Q[i, c])) * Decimal(float(K[j, c])) for c in range(d)),
                                 Decimal(0))) for j in range(N)]
        m = max(s)
        w = [ctx.exp(ctx.subtract(sj, m)) for sj in s]
        tot = sum(w, Decimal(0))
        for c in range(d):
            v = ctx.divide(sum((ctx.multiply(w[j], Decimal(float(V[j, c]))) for j in range(N)), Decimal(0)), tot)
            h = np.float16(float(v))                  # RNE of the nearest double
            # the two fp16 neighbours of v and their midpoint, exactly
            up = np.nextafter(h, np.float16(np.inf))
            dn = np.nextafter(h, np.float16(-np.inf))
            for other in (up, dn):
                mid = (Decimal(float(h)) + Decimal(float(other))) / 2
                if abs(v - mid) <= abs(v) * Decimal("1e-12"):
                    h = None
                    break
            out[i, c] = h
    return out


@pytest.mark.parametrize("seed,alpha", [(3019, 1 / math.sqrt(8)), (3021, 0.9), (3023, -0.6), (3025, 4.0),
                                        (3027, 0.0)])
def test_equals_correctly_rounded_exact_value(seed, alpha):
    # the oracle's fp64 evaluation rounds to the same fp16 as a 60-digit
    # evaluation of the definition, element by element (flat, sharp and
    # negative-alpha softmaxes; any dropped term, wrong sign or index breaks it)
    g = np.random.Generator(np.random.PCG64(seed))
    M, N, d = 4, 6, 8
    Q = g.standard_normal((M, d)).astype(np.float16)
    K = g.standard_normal((N, d)).astype(np.float16)
    V = g.standard_normal((N, d)).astype(np.float16)
    a32 = float(np.float32(alpha))
    O = oracle.attention_f64(Q, K, V, a32)
    ex = _exact_rounded(Q, K, V, a32)
    decided = 0
    for i in range(M):
        for c in range(d):
            if ex[i, c] is None:
                continue
            decided += 1
            assert O[i, c].view(np.uint16) == ex[i, c].view(np.uint16), (i, c, O[i, c], ex[i, c])
    assert decided >= M * d - 2

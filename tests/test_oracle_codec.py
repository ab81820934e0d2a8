"""Pins of the oracle's binary16 codec against numpy's float16 conversions (an
independent library routine) over every bit pattern and every rounding tie."""
import numpy as np

import oracle


def test_decode_every_pattern_matches_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signs of zeros and infinities are kept
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_encode_roundtrips_every_finite_value():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    fin = np.isfinite(vals)
    back = oracle.f64_to_f16(vals[fin])
    assert np.array_equal(back, bits[fin])


def test_encode_ties_round_to_even():
    # every midpoint between consecutive positive finite halves, both signs
    pos = np.arange(0, 0x7c00, dtype=np.uint16)
    lo = pos[:-1].view(np.float16).astype(np.float64)
    hi = pos[1:].view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2.0  # exact in fp64
    for sgn in (1.0, -1.0):
        got = oracle.f64_to_f16(sgn * mid)
        ref = (sgn * mid).astype(np.float16).view(np.uint16)
        assert np.array_equal(got, ref)
        # and the chosen neighbour has an even fraction field
        assert np.all((got & 1) == 0)


def test_encode_random_doubles_matches_numpy():
    g = np.random.Generator(np.random.PCG64(1234))
    for scale in (1e-9, 1e-6, 1e-3, 1.0, 1e3, 6e4):
        x = g.standard_normal(200_000) * scale
        assert np.array_equal(oracle.f64_to_f16(x), x.astype(np.float16).view(np.uint16))


def test_encode_overflow_boundary():
    got = oracle.f64_to_f16(np.array([65504.0, 65519.999, 65520.0, 1e6, -65520.0]))
    assert list(got.view(np.float16).astype(np.float64)) == [65504.0, 65504.0, np.inf, np.inf, -np.inf]


def test_encode_subnormals():
    tiny = 2.0 ** -24
    got = oracle.f64_to_f16(np.array([tiny, tiny / 2, tiny * 0.5000001, 3 * tiny / 2, -tiny / 4]))
    # 2^-25 is a tie between 0 and 2^-24 -> 0 (even); just above -> 2^-24;
    # 1.5 * 2^-24 is a tie between 1 and 2 units -> 2 units (even)
    assert list(got) == [0x0001, 0x0000, 0x0001, 0x0002, 0x8000]

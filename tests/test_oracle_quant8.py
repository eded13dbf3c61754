"""Pins of the 8-bit storage lanes of the oracle (oracle/quant8.py).

The 0.4.0 README's support matrix names the lanes (``int8``: a blockwise
dynamic map; ``fp8``: an e4m3 codebook) and pins their fidelity ordering
(tests/test_oracle_moe.py); the tables themselves are readings (see the
module). What is pinned here: the fp8 table against an independent E4M3
decode (oracle.mx, from the bit definition) and hand-worked values; the int8
table against its decade construction; the quantization against brute-force
nearest search in exact rational arithmetic, on random blocks and on exact
midpoints; the round trip; the dequantization rule.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import quant8
from oracle.mx import e4m3_value


def test_f32_rne_rounds_to_nearest_even():
    one = Fraction(1)
    ulp = Fraction(1, 2**23)
    assert quant8.f32_rne(one) == np.float32(1.0)
    assert quant8.f32_rne(one + ulp / 2) == np.float32(1.0)  # tie -> even (1.0)
    assert quant8.f32_rne(one + ulp * 3 / 2) == np.float32(1.0 + 2 * 2**-23)  # tie -> even
    assert quant8.f32_rne(one + ulp / 2 + Fraction(1, 2**60)) == np.float32(1.0 + 2**-23)
    assert quant8.f32_rne(Fraction(1, 10)) == np.float32(0.1)
    assert quant8.f32_rne(Fraction(1, 3)) == np.float32(1.0 / 3.0)


def test_fp8_table_is_e4m3_over_480():
    m = quant8.magnitudes("fp8")
    assert m.shape == (128,) and m.dtype == np.float32
    # independent decode of the finite E4M3 patterns (bias 7, subnormals at e = 0)
    for i in range(127):
        assert m[i] == np.float32(np.float64(e4m3_value(i)) / 480.0), i
    # the top pattern is the codebook's 480 (a codebook has no NaN), i.e. 1
    assert m[127] == np.float32(1.0)
    assert m[126] == np.float32(448.0 / 480.0)
    assert m[8] == np.float32(2.0**-6 / 480.0)  # the smallest normal
    assert m[1] == np.float32(2.0**-9 / 480.0)  # the smallest subnormal
    assert m[0] == 0.0
    assert np.all(np.diff(m.astype(np.float64)) > 0)


def test_int8_table_is_the_decade_construction():
    m = quant8.magnitudes("int8").astype(np.float64)
    assert m.shape == (128,) and m[0] == 0.0 and m[-1] == 1.0
    assert np.all(np.diff(m) > 0)
    lo = 1
    for z in range(6, -1, -1):  # decade (10^-(z+1), 10^-z] holds 2^(6-z) magnitudes
        n = 6 - z
        dec = m[lo : lo + 2**n]
        assert np.all(dec > 10.0 ** -(z + 1)) and np.all(dec <= 10.0**-z * (1 + 1e-7)), z
        assert dec[-1] == np.float32(10.0**-z)  # the decade's top is 10^-z
        # linear steps of 0.9 * 10^-z / 2^n (each value rounded once to fp32)
        if n > 0:
            step = 0.9 * 10.0**-z / 2**n
            assert np.allclose(np.diff(dec), step, rtol=1e-5), z
        assert abs(dec[0] - 10.0**-z * (0.1 + 0.9 / 2**n)) <= 1e-7 * 10.0**-z
        lo += 2**n
    assert lo == 128
    assert m[1] == np.float32(1e-6)


@pytest.mark.parametrize("kind", quant8.KINDS8)
def test_midpoints_are_exact_in_fp64(kind):
    m = quant8.magnitudes(kind)
    for a, b in zip(m[:-1], m[1:]):
        mid = (np.float64(a) + np.float64(b)) / 2.0
        assert Fraction(mid) == (Fraction(float(a)) + Fraction(float(b))) / 2
        # at most 28 significant bits: times a 24-bit absmax stays exact in fp64
        num = Fraction(mid).numerator
        while num % 2 == 0 and num:
            num //= 2
        assert num.bit_length() <= 28


def _brute_force_codes(w, absmax, kind):
    """Nearest magnitude of |w|/absmax by exact rational distance, ties to the
    smaller magnitude; sign bit from w."""
    mags = [Fraction(float(v)) for v in quant8.magnitudes(kind)]
    out = []
    for x, am in zip(w, absmax):
        a = Fraction(float(abs(x)))
        t = a / Fraction(float(am)) if am != 0 else Fraction(0)
        best = min(range(128), key=lambda i: (abs(t - mags[i]), i))
        out.append(best + (128 if np.signbit(x) else 0))
    return np.array(out)


@pytest.mark.parametrize("kind", quant8.KINDS8)
def test_quantize_matches_brute_force(kind):
    rng = np.random.default_rng(3)
    scales = [1.0, 1e-3, 37.5, 2.0**-60]
    w = np.concatenate(
        [(rng.standard_normal((1, 2, 64)) * s).astype(np.float32) for s in scales]
        + [(rng.standard_normal((1, 2, 64)) ** 5).astype(np.float32)],  # heavy tails: tiny ratios
        axis=1,
    )
    codes, absmax = quant8.quantize_blockwise8(w, kind)
    blocks = w.reshape(-1, 64)
    am = np.repeat(absmax.reshape(-1), 64)
    ref = _brute_force_codes(blocks.reshape(-1), am, kind)
    assert np.array_equal(codes.reshape(-1), ref)
    assert np.array_equal(absmax.reshape(-1), np.abs(blocks).max(axis=1))


@pytest.mark.parametrize("kind", quant8.KINDS8)
def test_exact_midpoints_go_to_the_smaller_magnitude(kind):
    m = quant8.magnitudes(kind).astype(np.float64)
    mids = (m[:-1] + m[1:]) / 2
    # midpoints that are fp32 values: a block with absmax 1 holding them ties exactly
    ties = [(i, mid) for i, mid in enumerate(mids) if np.float64(np.float32(mid)) == mid]
    assert len(ties) >= 4
    vals = np.array([t[1] for t in ties][:63], dtype=np.float32)
    row = np.concatenate([[1.0], vals, np.zeros(64 - 1 - len(vals))]).astype(np.float32)
    w = np.stack([row, -row])[None]  # [1, 2, 64]
    codes, absmax = quant8.quantize_blockwise8(w, kind)
    assert absmax[0, 0] == 1.0 and absmax[0, 1] == 1.0
    want = np.array([t[0] for t in ties][:63])
    assert np.array_equal(codes[0, 1 : 1 + len(want)], want)
    assert np.array_equal(codes[0, 65 : 65 + len(want)], want + 128)


@pytest.mark.parametrize("kind", quant8.KINDS8)
def test_round_trip_zero_block_and_max_element(kind):
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((2, 4, 128)) * 0.02).astype(np.float32)
    w[0, 0, :64] = 0.0
    w[0, 1, :64] = -0.0
    codes, absmax = quant8.quantize_blockwise8(w, kind)
    deq = quant8.dequantize8(codes, absmax, 4, 128, kind)
    # re-quantizing the dequantized stack gives the same codes and absmax
    c2, a2 = quant8.quantize_blockwise8(deq, kind)
    assert np.array_equal(c2, codes) and np.array_equal(a2, absmax)
    # zero blocks: absmax 0, +0 -> code 0, -0 -> code 128
    assert absmax[0, 0] == 0 and np.all(codes[0, :64] == 0)
    assert absmax[0, 2] == 0
    assert np.all(codes[0, 128:192] == 128)
    # the block maximum reconstructs exactly
    blocks = w.reshape(2, -1, 64)
    for e in range(2):
        for b in range(blocks.shape[1]):
            j = np.argmax(np.abs(blocks[e, b]))
            assert deq.reshape(2, -1, 64)[e, b, j] == blocks[e, b, j]


@pytest.mark.parametrize("kind", quant8.KINDS8)
def test_dequantize_is_one_rounding_of_the_exact_product(kind):
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((1, 2, 64)) * 3.3).astype(np.float32)
    codes, absmax = quant8.quantize_blockwise8(w, kind)
    deq = quant8.dequantize8(codes, absmax, 2, 64, kind).reshape(-1)
    vals = quant8.code_values(kind)
    for i in range(0, 128, 7):
        exact = Fraction(float(vals[codes[0, i]])) * Fraction(float(absmax[0, i // 64]))
        want = quant8.f32_rne(abs(exact)) * (1 if exact >= 0 else -1)
        assert deq[i] == np.float32(want)

"""Pins for the oracle's two codebooks (no GPU)."""

import numpy as np
import pytest
from scipy.stats import norm

from oracle import codebook, NF4_CODE, FP4_CODE
from conftest import read_golden


def test_nf4_matches_published_table_bitwise():
    golden = np.array([float(r[0]) for r in read_golden("nf4_codebook.txt")], dtype=np.float32)
    assert golden.shape == (16,)
    assert np.array_equal(golden.view(np.uint32), NF4_CODE.view(np.uint32))


def test_nf4_structure():
    c = codebook("nf4").astype(np.float64)
    assert c.shape == (16,)
    assert np.all(np.diff(c) > 0)
    assert c[0] == -1.0 and c[7] == 0.0 and c[15] == 1.0
    assert np.sum(c < 0) == 7 and np.sum(c > 0) == 8


def test_nf4_normal_quantile_construction():
    # Asymmetric normal-quantile construction: 8 positive quantiles and 7
    # negative ones on evenly spaced probabilities from 1 - delta down to 1/2
    # (1/2 itself dropped), plus an exact zero, scaled so the maximum is 1.
    delta = 0.5 * (1.0 / 30.0 + 1.0 / 32.0)
    pos = norm.ppf(np.linspace(1.0 - delta, 0.5, 9)[:-1])
    neg = -norm.ppf(np.linspace(1.0 - delta, 0.5, 8)[:-1])
    v = np.sort(np.concatenate([pos, [0.0], neg]))
    v = v / v.max()
    assert np.max(np.abs(v - NF4_CODE.astype(np.float64))) <= 1e-6


def _e2m1_decode(bits):
    e, m = (bits >> 1) & 3, bits & 1
    return m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)


def test_fp4_matches_e2m1_definition():
    golden = {int(r[0], 2): float(r[1]) for r in read_golden("fp4_e2m1.txt")}
    c = codebook("fp4")
    for code in range(16):
        sign = -1.0 if code & 8 else 1.0
        mag = _e2m1_decode(code & 7)
        assert mag == golden[code & 7]
        want = np.float32(sign * mag / 6.0)
        assert np.array_equal(np.float32(c[code]).view(np.uint32), want.view(np.uint32)), code
    assert c[8].view(np.uint32) == np.float32(-0.0).view(np.uint32)
    assert np.max(np.abs(c)) == 1.0


def test_fp4_coarser_than_nf4_near_zero_and_monotone_magnitudes():
    mags = FP4_CODE[:8].astype(np.float64)
    assert np.all(np.diff(mags) > 0)
    # NF4 spends more codes inside [-0.5, 0.5] than FP4 does (its design goal)
    assert np.sum(np.abs(NF4_CODE) <= 0.5) > np.sum(np.abs(FP4_CODE[:8]) <= 0.5)


def test_unknown_codebook_rejected():
    with pytest.raises(ValueError):
        codebook("int8")

"""Pins for the oracle's blockwise quantizer, dequantizer and bf16 rounding (no GPU)."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import (
    codebook,
    quantize_blockwise,
    dequantize,
    unpack_codes,
    bf16_rne_bits,
    bf16_bits_to_f32,
)

KINDS = ("nf4", "fp4")


def _brute_force_code(w, absmax, kind):
    """Nearest entry by exhaustive exact search with the stated tie rules."""
    c = [Fraction(float(v)) for v in codebook(kind)]
    W, A = Fraction(float(w)), Fraction(float(absmax))
    if A == 0:
        if kind == "nf4":
            return 7
        return 8 if np.signbit(w) else 0
    d = [abs(W - A * ci) for ci in c]
    best = min(d)
    cands = [i for i in range(16) if d[i] == best]
    if kind == "nf4":
        return min(cands)  # ties -> lower code
    # fp4: smaller magnitude first, then the sign bit of w decides +0 / -0
    mag = min(abs(c[i]) for i in cands)
    cands = [i for i in cands if abs(c[i]) == mag]
    want_neg = bool(np.signbit(w))
    for i in cands:
        if bool(i & 8) == want_neg:
            return i
    return cands[0]


def _adversarial_block(kind, rng):
    """A 64-block around every decision boundary, with absmax 1.0 pinned by an element."""
    c = codebook(kind).astype(np.float64)
    if kind == "nf4":
        mids = (c[:-1] + c[1:]) / 2
    else:
        m = c[:8]
        mids = np.concatenate([(m[:-1] + m[1:]) / 2, -(m[:-1] + m[1:]) / 2])
    vals = [1.0, -0.0, 0.0]
    for mi in mids:
        f = np.float32(mi)
        vals += [f, np.nextafter(f, np.float32(2)), np.nextafter(f, np.float32(-2))]
    vals = np.array(vals, dtype=np.float32)
    vals = vals[np.abs(vals) <= 1.0]
    out = np.concatenate([vals, rng.uniform(-1, 1, 64).astype(np.float32)])[:64]
    out[0] = 1.0
    return out


def test_brute_force_agrees_random_and_adversarial():
    rng = np.random.default_rng(1234)
    for kind in KINDS:
        blocks = [rng.standard_normal(64).astype(np.float32) * 0.02 for _ in range(6)]
        blocks += [_adversarial_block(kind, rng) for _ in range(3)]
        blocks += [(rng.standard_normal(64) * 1e-30).astype(np.float32)]  # tiny / subnormal-ish products
        w = np.stack(blocks)[None]  # [1, nblocks, 64]
        packed, absmax = quantize_blockwise(w, kind)
        q = unpack_codes(packed).reshape(-1, 64)
        for b in range(w.shape[1]):
            for i in range(64):
                assert q[b, i] == _brute_force_code(w[0, b, i], absmax[0, b], kind), (kind, b, i)


def test_exact_midpoint_ties():
    # NF4: ties to the lower code. FP4: ties to the smaller magnitude.
    for kind in KINDS:
        c = codebook(kind).astype(np.float64)
        if kind == "nf4":
            mids = (c[:-1] + c[1:]) / 2
            lower = np.arange(15)
        else:
            mids = (c[:7] + c[1:8]) / 2
            lower = np.arange(7)
        hit = 0
        for mi, lo in zip(mids, lower):
            f = np.float32(mi)
            if float(f) != mi:
                continue  # midpoint not representable in fp32: no exact tie possible at absmax 1
            w = np.zeros((1, 1, 64), dtype=np.float32)
            w[0, 0, 0] = 1.0
            w[0, 0, 1] = f
            if kind == "fp4":
                w[0, 0, 2] = -f
            p, a = quantize_blockwise(w, kind)
            q = unpack_codes(p)[0]
            assert q[1] == lo
            if kind == "fp4":
                assert q[2] == 8 + lo
            hit += 1
        # NF4 has several fp32-representable midpoints at absmax 1; FP4 only a/2
        assert hit >= (3 if kind == "nf4" else 1), kind


def test_error_bound_half_gap():
    rng = np.random.default_rng(7)
    for kind in KINDS:
        w = (rng.standard_normal((2, 8, 128)) * 0.02).astype(np.float32)
        p, a = quantize_blockwise(w, kind)
        wh = dequantize(p, a, 8, 128, kind)
        c = np.sort(codebook(kind).astype(np.float64))
        amax = np.repeat(a.astype(np.float64), 64, axis=1).reshape(w.shape)
        # gap of the codebook interval holding w/absmax (decided with exact products)
        x = w.astype(np.float64)
        i = np.clip(np.sum(x[..., None] >= amax[..., None] * c, axis=-1) - 1, 0, 14)
        gap = c[i + 1] - c[i]
        ulp = np.spacing(np.abs(wh).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(x - wh.astype(np.float64)) <= amax * gap / 2 + ulp / 2)


def test_max_element_exact_and_zero_block():
    rng = np.random.default_rng(3)
    for kind in KINDS:
        w = (rng.standard_normal((3, 4, 64)) * 0.02).astype(np.float32)
        w[1, 2, :] = 0.0
        p, a = quantize_blockwise(w, kind)
        wh = dequantize(p, a, 4, 64, kind)
        q = unpack_codes(p).reshape(3, 4, 64)
        for e in range(3):
            for r in range(4):
                blk = w[e, r]
                if np.all(blk == 0):
                    assert a[e, r] == 0.0
                    assert np.all(q[e, r] == (7 if kind == "nf4" else 0))
                    assert np.all(wh[e, r] == 0.0)
                    continue
                j = int(np.argmax(np.abs(blk)))
                assert a[e, r] == abs(blk[j])
                assert wh[e, r, j] == blk[j]  # +-1 entry times absmax is exact


def test_round_trip_is_exact():
    rng = np.random.default_rng(11)
    for kind in KINDS:
        w = (rng.standard_normal((2, 16, 192)) * 0.02).astype(np.float32)
        w[0, 3, 64:128] = 0.0
        w[1, 0, :64] = -0.0
        p, a = quantize_blockwise(w, kind)
        wh = dequantize(p, a, 16, 192, kind)
        p2, a2 = quantize_blockwise(wh, kind)
        assert np.array_equal(p, p2) and np.array_equal(a.view(np.uint32), a2.view(np.uint32))


def test_pack_order_even_element_high_nibble():
    # codebook entries placed exactly: element 2j -> high nibble of byte j
    c = codebook("nf4")
    codes = np.array([15, 0, 3, 12] + [7] * 60)
    w = (c[codes].astype(np.float64) * 0.5).astype(np.float32)[None, None, :]
    p, a = quantize_blockwise(w, "nf4")
    assert a[0, 0] == 0.5
    assert p[0, 0] == 0xF0 and p[0, 1] == 0x3C and p[0, 2] == 0x77


def test_dequant_definition_bit_patterns():
    rng = np.random.default_rng(5)
    for kind in KINDS:
        p = rng.integers(0, 256, size=(2, 64), dtype=np.uint8)
        a = (np.abs(rng.standard_normal((2, 2))) * 0.05).astype(np.float32)
        a[1, 1] = 0.25  # power of two: every product representable
        wh = dequantize(p, a, 2, 64, kind)
        q = unpack_codes(p).reshape(2, 2, 64)
        c = codebook(kind)
        for e in range(2):
            for b in range(2):
                for i in range(0, 64, 7):
                    cv = c[q[e, b, i]]
                    exact = Fraction(float(cv)) * Fraction(float(a[e, b]))
                    # single rounding of the exact product; the sign of a zero is the code's
                    want = np.float32(np.copysign(float(exact), cv))
                    got = np.float32(wh[e].reshape(2, 64)[b, i])
                    assert got.view(np.uint32) == want.view(np.uint32)
        blk = wh[1].reshape(2, 64)[1]
        qq = q[1, 1]
        assert np.array_equal(blk.astype(np.float64), c[qq].astype(np.float64) * 0.25)
    # -0.0 survives dequantization (FP4 code 8)
    p = np.full((1, 32), 0x88, dtype=np.uint8)
    wh = dequantize(p, np.array([[0.5]], np.float32), 1, 64, "fp4")
    assert np.all(np.signbit(wh)) and np.all(wh == 0)


def test_bf16_rne_matches_torch_including_ties():
    rng = np.random.default_rng(9)
    x = rng.standard_normal(100000).astype(np.float32) * np.float32(3.0)
    u = x.view(np.uint32)
    ties = ((u[:2000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, np.array([0.0, -0.0, 1e-40, -3e-39], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_rne_bits(x), ref)
    assert np.array_equal(bf16_bits_to_f32(ref), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_rejects_bad_stacks():
    with pytest.raises(ValueError):
        quantize_blockwise(np.zeros((1, 2, 96), np.float32))  # in % 64 != 0
    with pytest.raises(ValueError):
        quantize_blockwise(np.zeros((2, 64), np.float32))
    w = np.zeros((1, 1, 64), np.float32)
    w[0, 0, 3] = np.inf
    with pytest.raises(ValueError):
        quantize_blockwise(w)
    with pytest.raises(ValueError):
        quantize_blockwise(np.zeros((1, 1, 64), np.float32), kind="int4")

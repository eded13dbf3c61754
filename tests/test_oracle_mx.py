"""Pins of the MXFP4 oracle (oracle/mx.py) against the format definitions of
the OCP Microscaling Formats (MX) v1.0 specification that the pages' "MXFP4"
refers to: the E2M1 bit-level decode, the E8M0 scale, the shared-exponent
rule, round-to-nearest-even with saturation, brute force and round trips."""

import math

import numpy as np
import pytest

import oracle
from oracle import mx


def _e2m1_from_bits(code):
    # sign | 2 exponent bits (bias 1) | 1 mantissa bit; exponent 0: subnormal
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    v = m * 0.5 if e == 0 else math.ldexp(1.0 + m / 2.0, e - 1)
    return -v if s else v


def test_e2m1_values_from_the_bit_definition():
    got = mx.e2m1_value(np.arange(16))
    want = np.array([_e2m1_from_bits(c) for c in range(16)])
    assert np.array_equal(got, want)
    assert list(np.abs(want[:8])) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert np.signbit(got[8]) and got[8] == 0.0  # code 8 is -0


def test_e8m0_scale():
    assert mx.e8m0_value(127) == 1.0
    assert mx.e8m0_value(0) == 2.0 ** -127
    assert mx.e8m0_value(254) == 2.0 ** 127
    with pytest.raises(ValueError):
        mx.e8m0_value(255)  # NaN code


def _one_block(vals):
    w = np.zeros((1, 1, 32), dtype=np.float32)
    w[0, 0, : len(vals)] = vals
    p, s = oracle.quantize_mx(w)
    q = np.empty(32, dtype=np.int64)
    q[0::2] = p[0] >> 4
    q[1::2] = p[0] & 15
    return q, int(s[0, 0])


@pytest.mark.parametrize(
    "amax,shared",
    [(6.0, 0), (4.0, 0), (7.99, 0), (1.0, -2), (0.75, -3), (2.0 ** -100, -102), (3.0e38, 125)],
)
def test_shared_exponent_rule(amax, shared):
    # floor(log2(amax)) - 2, by hand
    q, s = _one_block([amax])
    assert s - 127 == shared
    assert shared == math.floor(math.log2(amax)) - 2


def test_zero_block_and_negative_zero():
    q, s = _one_block([0.0])
    assert s == 0 and np.all(q == 0)
    q, s = _one_block([4.0, -0.01, -0.0])
    # scale 2^0: -0.01 rounds to magnitude 0 and keeps its sign (code 8), as does -0.0
    assert s == 127 and q[0] == 6 and q[1] == 8 and q[2] == 8


def test_round_to_nearest_even_and_saturation():
    # scale 2^0 fixed by the 6.0 in the block; values on every midpoint
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    q, s = _one_block([6.0] + mids + [5.0000005, 4.9999995])
    assert s == 127
    # ties go to the even mantissa: 0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0
    assert list(q[1:8]) == [0, 2, 2, 4, 4, 6, 6]
    assert q[8] == 7 and q[9] == 6  # just above / below 5
    q, s = _one_block([7.99, 6.5, -7.0])
    assert s == 127 and list(q[:3]) == [7, 7, 15]  # saturated to +-6


def test_brute_force_nearest_value():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((3, 8, 96)) * np.exp(rng.uniform(-6, 6, (3, 8, 1)))).astype(np.float32)
    p, s = oracle.quantize_mx(w)
    vals = oracle.dequantize_mx(p, s, 8, 96).reshape(-1, 32).astype(np.float64)
    blocks = w.reshape(-1, 32).astype(np.float64)
    scale = mx.e8m0_value(s.reshape(-1))
    cand = np.array([_e2m1_from_bits(c) for c in range(8)])
    for b in range(blocks.shape[0]):
        amax = np.abs(blocks[b]).max()
        assert scale[b] == 2.0 ** (math.floor(math.log2(amax)) - 2)
        for i in range(32):
            a = abs(blocks[b, i]) / scale[b]
            d = np.abs(cand - a)
            best = np.flatnonzero(d == d.min())
            idx = best[0] if len(best) == 1 else [k for k in best if k % 2 == 0][0]
            assert abs(vals[b, i]) == cand[idx] * scale[b]
            if vals[b, i] != 0.0:
                assert np.sign(vals[b, i]) == np.sign(blocks[b, i])


def test_round_trip_and_exact_dequantization():
    rng = np.random.default_rng(4)
    E, out, inn = 2, 6, 64
    nb = out * inn // 32
    q = rng.integers(0, 16, size=(E, nb, 32))
    # a magnitude index of 6 or 7 in every block keeps its shared exponent
    q[:, :, 5] = rng.choice([6, 7, 14, 15], size=(E, nb))
    s = rng.integers(1, 253, size=(E, nb)).astype(np.uint8)
    flat = q.reshape(E, -1)
    packed = ((flat[:, 0::2] << 4) | flat[:, 1::2]).astype(np.uint8)
    w = oracle.dequantize_mx(packed, s, out, inn)
    for e, b, i in [(0, 0, 0), (1, nb - 1, 31), (1, 3, 5)]:
        assert float(w[e].reshape(-1, 32)[b, i]) == mx.mx_value_exact(int(q[e, b, i]), int(s[e, b]))
    p2, s2 = oracle.quantize_mx(w)
    # codes and scales come back bit for bit (-0 keeps its sign through fp32)
    assert np.array_equal(s2, s)
    assert np.array_equal(p2, packed)


def test_stored_weights_mxfp4_dispatch():
    rng = np.random.default_rng(5)
    w = rng.normal(0, 0.02, (2, 4, 64)).astype(np.float32)
    got = oracle.stored_weights(w, "mxfp4")
    assert np.array_equal(got, oracle.dequantize_mx(*oracle.quantize_mx(w), 4, 64))
    # the MX reconstruction is coarser than nf4's on Gaussian weights
    e_mx = np.linalg.norm(got - w) / np.linalg.norm(w)
    e_nf4 = np.linalg.norm(oracle.stored_weights(w, "nf4") - w) / np.linalg.norm(w)
    assert e_mx > e_nf4


def test_shape_errors():
    with pytest.raises(ValueError):
        oracle.quantize_mx(np.zeros((1, 2, 48), dtype=np.float32))  # in % 32
    with pytest.raises(ValueError):
        oracle.quantize_mx(np.zeros((2, 64), dtype=np.float32))


# ---- MXFP8 (E4M3) activation rows ----

def _e4m3_from_bits(c):
    s, e, m = (c >> 7) & 1, (c >> 3) & 15, c & 7
    v = math.ldexp(m / 8.0, -6) if e == 0 else math.ldexp(1.0 + m / 8.0, e - 7)
    return -v if s else v


def test_e4m3_values_by_hand_and_from_bits():
    got = oracle.e4m3_value(np.arange(0x7F))
    assert np.array_equal(got, [_e4m3_from_bits(c) for c in range(0x7F)])
    for code, val in [(0x38, 1.0), (0x7E, 448.0), (0x01, 2.0 ** -9), (0x08, 2.0 ** -6),
                      (0x77, 240.0), (0x78, 256.0), (0x07, 7 * 2.0 ** -9)]:
        assert _e4m3_from_bits(code) == val
        assert oracle.e4m3_value(code) == val
    assert np.signbit(oracle.e4m3_value(0x80))
    assert np.all(np.diff(got) > 0)  # codes 0..0x7E are ascending magnitudes
    with pytest.raises(ValueError):
        oracle.e4m3_value(0x7F)


def _row(vals):
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, : len(vals)] = vals
    return oracle.quantize_mx8_rows(x)


def test_mx8_scale_rule_ties_and_saturation():
    # 448 pins the shared exponent at 0 (floor(log2 448) - 8)
    c, s = _row([448.0, 432.0, 440.0, 1.0625, 1.1875, 2.0 ** -10, 3.0 * 2.0 ** -10, 464.0])
    assert s[0, 0] == 127
    v = oracle.e4m3_value(c[0])
    # 432 is the midpoint of 416 (odd mantissa) and 448 (even): 448; 1.0625 between
    # 1.0 (even) and 1.125: 1.0; 1.1875 between 1.125 and 1.25 (even): 1.25;
    # 2^-10 between 0 and 2^-9: 0 (even); 3 * 2^-10 between 2^-9 and 2^-8 (even): 2^-8
    assert list(v[:7]) == [448.0, 448.0, 448.0, 1.0, 1.25, 0.0, 2.0 ** -8]
    assert v[7] == 448.0  # above the largest finite value: saturated
    c, s = _row([1.0, -0.5])
    assert s[0, 0] == 127 - 8 and c[0, 0] == 0x78 and c[0, 1] == 0xF0  # 1.0 / 2^-8 = 256
    c, s = _row([0.0])
    assert s[0, 0] == 0 and np.all(c == 0)


def test_mx8_brute_force():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((6, 128)) * np.exp(rng.uniform(-10, 10, (6, 1)))).astype(np.float32)
    c, s = oracle.quantize_mx8_rows(x)
    vals = oracle.dequantize_mx8_rows(c, s)
    mags = np.array([_e4m3_from_bits(k) for k in range(0x7F)])
    for r in range(6):
        for b in range(4):
            blk = x[r, 32 * b : 32 * b + 32].astype(np.float64)
            sc = 2.0 ** (math.floor(math.log2(np.abs(blk).max())) - 8)
            assert int(s[r, b]) - 127 == math.floor(math.log2(np.abs(blk).max())) - 8
            for i in range(32):
                a = abs(blk[i]) / sc
                d = np.abs(mags - a)
                best = np.flatnonzero(d == d.min())
                k = best[0] if len(best) == 1 else [q for q in best if q % 2 == 0][0]
                assert abs(vals[r, 32 * b + i]) == mags[k] * sc


def test_mx8_forward_close_to_unquantized_activations():
    # the activation conversion is a rounding of relative size <= 2^-4 per
    # element: the MX forward stays within a few percent of the same weights
    # applied to unrounded activations
    from workloads import get_config, gen_x, gen_logits, gen_weights

    cfg = get_config("tiny")
    x, lg = gen_x(cfg, 1), gen_logits(cfg, 1)
    idx, w = oracle.route(lg, cfg.k)
    wgu = oracle.stored_weights(gen_weights(cfg, 1, "gate_up"), "mxfp4")
    wdn = oracle.stored_weights(gen_weights(cfg, 1, "down"), "mxfp4")
    y_mx = oracle.mx8_forward(x, idx, w, wgu, wdn)
    y = oracle.moe_forward(x, idx, w, wgu, wdn)
    err = np.abs(y_mx - y).max() / np.abs(y).max()
    assert 1e-4 < err < 0.1


# ---- exact pin of the MX forward's composition ----------------------------
# An independent recomputation in rational arithmetic (fractions.Fraction,
# with silu from decimal at 60 digits): every conversion is a brute-force
# nearest search over the E4M3 values built from the bit definition, the bf16
# rounding of a goes through its fp32 value (the gate_up epilogue computes a
# in fp32 and stores it as bf16, nearest even), and the contractions are exact.

from decimal import Decimal, getcontext
from fractions import Fraction


def _e4m3_mags_exact():
    out = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        out.append(Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))
    return out


_MAGS = _e4m3_mags_exact()


def _floor_log2(q):
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    return e


def _mx8_round_row(vals):
    """MXFP8 values of one row of Fractions (blocks of 32), by brute force."""
    out = []
    for b in range(0, len(vals), 32):
        blk = vals[b:b + 32]
        amax = max(abs(v) for v in blk)
        sh = -127 if amax == 0 else max(-127, min(127, _floor_log2(amax) - 8))
        sc = Fraction(2) ** sh
        for v in blk:
            a = abs(v) / sc
            d = [abs(m - a) for m in _MAGS]
            best = [k for k in range(len(_MAGS)) if d[k] == min(d)]
            k = best[0] if len(best) == 1 else [q for q in best if q % 2 == 0][0]
            out.append((-1 if v < 0 else 1) * _MAGS[k] * sc)
    return out


def _round_bits(q, bits, emin):
    """Nearest binary value of q with `bits` significant bits (ties to even), exponent >= emin."""
    if q == 0:
        return Fraction(0)
    s = -1 if q < 0 else 1
    q = abs(q)
    e = max(_floor_log2(q), emin)
    ulp = Fraction(2) ** (e - bits + 1)
    n, r = divmod(q, ulp)
    if r > ulp / 2 or (r == ulp / 2 and n % 2 == 1):
        n += 1
    return s * n * ulp


def _silu_exact(g):
    getcontext().prec = 60
    gd = Decimal(g.numerator) / Decimal(g.denominator)
    return Fraction(gd / (1 + (-gd).exp()))


def test_mx8_forward_equals_exact_rational_recomputation():
    rng = np.random.default_rng(20)
    E, H, I, T, k = 2, 64, 64, 3, 2
    # MXFP4-stored weights: E2M1 values times a power of two per 32-block
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])

    def mx_weights(out, inn):
        v = mags[rng.integers(0, 8, (E, out, inn))] * np.where(rng.random((E, out, inn)) < 0.5, -1, 1)
        s = rng.integers(-9, -5, (E, out, inn // 32))
        return (v * np.ldexp(1.0, np.repeat(s, 32, axis=2))).astype(np.float32)

    wgu, wdn = mx_weights(2 * I, H), mx_weights(H, I)
    x = oracle.bf16_bits_to_f32(oracle.bf16_rne_bits(
        (rng.standard_normal((T, H)) * np.exp(rng.uniform(-3, 3, (T, 1)))).astype(np.float32)))
    idx = np.array([[0, 1], [1, 0], [1, 0]], np.int32)
    w = rng.random((T, k))
    w /= w.sum(1, keepdims=True)

    def reference(round_a_to_bf16):
        y = [[Fraction(0)] * H for _ in range(T)]
        for t in range(T):
            xq = _mx8_round_row([Fraction(float(v)) for v in x[t]])
            for j in range(k):
                e = int(idx[t, j])
                h = [sum(Fraction(float(wgu[e, n, c])) * xq[c] for c in range(H)) for n in range(2 * I)]
                a = [_silu_exact(h[n]) * h[I + n] for n in range(I)]
                if round_a_to_bf16:
                    a = [_round_bits(_round_bits(v, 24, -126), 8, -126) for v in a]
                aq = _mx8_round_row(a)
                for n in range(H):
                    o = sum(Fraction(float(wdn[e, n, c])) * aq[c] for c in range(I))
                    y[t][n] += Fraction(float(w[t, j])) * o
        return np.array([[float(v) for v in row] for row in y])

    ref = reference(True)
    got = oracle.mx8_forward(x, idx, w, wgu, wdn)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))
    # the case tells the bf16 rounding of a apart: without it the E4M3
    # decisions of some elements of a change
    assert np.max(np.abs(reference(False) - ref)) > 1e-6 * np.max(np.abs(ref))

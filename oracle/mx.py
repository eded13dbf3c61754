"""MXFP4 expert storage (oracle): FP4 E2M1 elements, one E8M0 power-of-two
scale per 32 consecutive elements of a row.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources. The pages name the format without defining it: the experts4bit-qlora
0.31.1 project page lists gpt-oss among the supported families with MXFP4
experts that are dequantized bit-identically, and its "which door" table has a
native-MXFP4 row; the author's project page plans an MXFP4 lane for the
kernel. The name refers to the Open Compute Project "Microscaling Formats
(MX) v1.0" specification, which this module follows:

* element FP4 E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit, no
  infinities or NaN; exponent field 0 is subnormal (value m / 2), otherwise
  2^(e - 1) * (1 + m / 2). Magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* scale E8M0: an 8-bit biased exponent, value 2^(s - 127); s = 255 is NaN and
  is never written here.
* block: 32 consecutive elements.
* conversion (the specification's conversion of a vector of scalars to an MX
  block): shared exponent = floor(log2(max |v|)) - emax, with emax = 2 the
  exponent of E2M1's largest normal (6 = 1.5 * 2^2), clamped to [-127, 127];
  each element is v / 2^shared rounded to the nearest E2M1 value, ties to the
  even mantissa, magnitudes beyond 6 saturated to 6.

Readings for what neither fixes:

* a block of zeros takes scale code 0 (2^-127) and element code 0;
* a negative value that rounds to magnitude 0 stores -0 (code 8), as the FP4
  lane does; the element code is the sign bit (bit 3) over the E2M1
  magnitude index (bits 2..0), the same code layout as the library's FP4 lane;
* rows hold in % 32 == 0 elements, so a block never straddles a row;
* storage: two codes per byte with the even element in the high nibble (the
  library's 4-bit convention) ``[E, out*in/2]``, scales uint8 ``[E, out*in/32]``;
* the dequantized weight is the element value times 2^(s - 127). It is exact
  in fp32 and in bf16 for every scale the conversion writes (s <= 252 for
  finite fp32 input), which is what makes the bit-identical dequantization
  the pages ask for possible.

Exactness of the oracle: max |v| is an fp32 value, its floor(log2) comes from
frexp exactly, v / 2^shared is exact in fp64, and the rounding compares the
scaled magnitude with exact midpoints.
"""

import math

import numpy as np

MX_BLOCK = 32
E2M1_EMAX = 2
# E2M1 magnitudes by index (code bits 2..0), from the bit-level definition
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
_MIDS = (E2M1_MAG[:-1] + E2M1_MAG[1:]) / 2.0  # 0.25 0.75 1.25 1.75 2.5 3.5 5.0


def e2m1_value(code):
    """Value of 4-bit E2M1 codes (array of ints 0..15)."""
    c = np.asarray(code, dtype=np.int64)
    mag = E2M1_MAG[c & 7]
    return np.where(c & 8, -mag, mag)


def e8m0_value(s):
    """2^(s - 127) for scale codes s in 0..254 (fp64, exact)."""
    s = np.asarray(s, dtype=np.int64)
    if np.any((s < 0) | (s > 254)):
        raise ValueError("E8M0 codes are 0..254 (255 is NaN)")
    return np.ldexp(1.0, s - 127)


def _check_stack(w):
    w = np.asarray(w)
    if w.ndim != 3:
        raise ValueError("weights must be a 3-D [E, out, in] stack")
    if w.dtype != np.float32:
        raise ValueError("weights must be float32")
    E, out, inn = w.shape
    if E <= 0 or out <= 0 or inn <= 0:
        raise ValueError("empty stack")
    if inn % MX_BLOCK != 0:
        raise ValueError("in_features must be divisible by 32")
    if not np.all(np.isfinite(w)):
        raise ValueError("weights must be finite")
    return w


def shared_exponent(amax):
    """floor(log2(amax)) - 2 clamped to [-127, 127]; -127 for amax == 0."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)  # amax = m * 2^ex, 0.5 <= m < 1, so floor(log2) = ex - 1
    sh = ex.astype(np.int64) - 1 - E2M1_EMAX
    sh = np.where(amax == 0.0, -127, sh)
    return np.clip(sh, -127, 127)


def round_e2m1_magnitude(a):
    """Index of the E2M1 magnitude nearest to ``a >= 0`` (ties to the even
    mantissa, i.e. the even index; beyond 6 saturates to index 7)."""
    a = np.asarray(a, dtype=np.float64)
    q = np.zeros(a.shape, dtype=np.int64)
    for m in _MIDS:
        q += a > m
    # a exactly on the midpoint between q and q + 1: take the even index
    tie = np.zeros(a.shape, dtype=bool)
    for i, m in enumerate(_MIDS):
        tie |= (a == m) & (q == i) & (i % 2 == 1)
    return q + tie


def quantize_mx(w, chunk_blocks=1 << 16):
    """MXFP4 conversion of a float32 ``[E, out, in]`` stack.

    Returns ``(packed uint8 [E, out*in/2], scales uint8 [E, out*in/32])``.
    """
    w = _check_stack(w)
    E, out, inn = w.shape
    nb = out * inn // MX_BLOCK
    packed = np.empty((E, out * inn // 2), dtype=np.uint8)
    scales = np.empty((E, nb), dtype=np.uint8)
    for e in range(E):
        blocks_all = w[e].reshape(nb, MX_BLOCK)
        for b0 in range(0, nb, chunk_blocks):
            b1 = min(nb, b0 + chunk_blocks)
            blocks = blocks_all[b0:b1].astype(np.float64)
            sh = shared_exponent(np.abs(blocks).max(axis=1))
            scaled = blocks / np.ldexp(1.0, sh)[:, None]  # exact: power of two
            q = round_e2m1_magnitude(np.abs(scaled)) + 8 * np.signbit(blocks)
            q = q.reshape(-1)
            scales[e, b0:b1] = (sh + 127).astype(np.uint8)
            packed[e, b0 * MX_BLOCK // 2 : b1 * MX_BLOCK // 2] = ((q[0::2] << 4) | q[1::2]).astype(np.uint8)
    return packed, scales


def dequantize_mx(packed, scales, out, inn):
    """fp32 ``[E, out, in]``: element value times 2^(s - 127) (exact)."""
    packed = np.asarray(packed, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    E = packed.shape[0]
    if packed.shape != (E, out * inn // 2) or scales.shape != (E, out * inn // MX_BLOCK):
        raise ValueError("packed/scales shapes do not match [E, out, in]")
    q = np.empty((E, out * inn), dtype=np.int64)
    q[:, 0::2] = packed >> 4
    q[:, 1::2] = packed & 0xF
    vals = e2m1_value(q).reshape(E, -1, MX_BLOCK) * e8m0_value(scales)[:, :, None]
    f32 = vals.astype(np.float32)
    if not np.array_equal(f32.astype(np.float64), vals):
        raise ValueError("an MXFP4 value is not representable in fp32 (scale code > 252)")
    return f32.reshape(E, out, inn)


def mx_value_exact(code, s):
    """Reference value of one element by Python float arithmetic (exact)."""
    mag = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0][code & 7]
    v = math.ldexp(mag, int(s) - 127)
    return -v if code & 8 else v


# ---------------------------------------------------------------------------
# MXFP8 activations for the scaled-MFMA forward (the MX forward path)
#
# The MX forward feeds the MFMA 8-bit activations: every activation row is
# converted to MXFP8 (OCP MX v1.0: element FP8 E4M3, scale E8M0 per 32
# elements) with the same rule as the weights, emax = 8 for E4M3 (448 =
# 1.75 * 2^8). E4M3 (the OCP 8-bit format): sign, 4 exponent bits (bias 7),
# 3 mantissa bits; exponent 0 is subnormal (value m / 8 * 2^-6); the only NaN
# is S.1111.111, there are no infinities, so the largest finite magnitude is
# 448; conversion rounds to nearest even and saturates at 448.
# Reading (the pages do not describe the activations of an MXFP4 lane): the
# gate_up input x and the down input a = bf16(silu(g) * u) are each converted
# per row; products and sums are exact up to fp32 accumulation.

E4M3_EMAX = 8
E4M3_MAX = 448.0


def e4m3_value(code):
    """Value of 8-bit E4M3 codes (0x7F / 0xFF are NaN)."""
    c = np.asarray(code, dtype=np.int64)
    if np.any((c & 0x7F) == 0x7F):
        raise ValueError("E4M3 NaN code")
    e, m = (c >> 3) & 15, c & 7
    v = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    return np.where(c & 0x80, -v, v)


# every finite non-negative E4M3 magnitude, ascending (codes 0x00..0x7E)
E4M3_MAGS = e4m3_value(np.arange(0x7F))


def round_e4m3_magnitude(a):
    """Code (0..0x7E) of the E4M3 magnitude nearest to ``a >= 0``; ties to
    the even code (the even mantissa), beyond 448 saturated."""
    a = np.asarray(a, dtype=np.float64)
    mids = (E4M3_MAGS[:-1] + E4M3_MAGS[1:]) / 2.0
    q = np.searchsorted(mids, a, side="left")  # number of midpoints strictly below a
    tie = (q < len(mids)) & (a == mids[np.minimum(q, len(mids) - 1)]) & (q % 2 == 1)
    return np.minimum(q + tie, 0x7E)


def quantize_mx8_rows(x):
    """MXFP8 conversion of fp32 rows ``[n, K]`` (K % 32 == 0).

    Returns ``(codes uint8 [n, K], scales uint8 [n, K/32])`` in element order.
    """
    x = np.asarray(x, dtype=np.float32)
    n, K = x.shape
    if K % MX_BLOCK:
        raise ValueError("row length must be divisible by 32")
    if not np.all(np.isfinite(x)):
        raise ValueError("activations must be finite")
    blocks = x.reshape(n, K // MX_BLOCK, MX_BLOCK).astype(np.float64)
    amax = np.abs(blocks).max(axis=2)
    _, ex = np.frexp(amax)
    sh = np.where(amax == 0.0, -127, ex.astype(np.int64) - 1 - E4M3_EMAX)
    sh = np.clip(sh, -127, 127)
    scaled = blocks / np.ldexp(1.0, sh)[:, :, None]
    q = round_e4m3_magnitude(np.abs(scaled)) | (np.signbit(blocks).astype(np.int64) << 7)
    return q.reshape(n, K).astype(np.uint8), (sh + 127).astype(np.uint8)


def dequantize_mx8_rows(codes, scales):
    """fp64 ``[n, K]`` values of MXFP8 rows (exact)."""
    codes = np.asarray(codes, dtype=np.uint8)
    n, K = codes.shape
    v = e4m3_value(codes).reshape(n, K // MX_BLOCK, MX_BLOCK)
    return (v * e8m0_value(scales)[:, :, None]).reshape(n, K)


def mx8_forward(x, idx, w, w_gu, w_dn):
    """The MX forward path: y [T, H] (fp64) of the routed SwiGLU MLP whose
    expert inputs are MXFP8-converted: x per token row, and a = silu(g) * u
    rounded to bf16 (as the gate_up epilogue stores it) per pair row. The
    weights are the stored (MXFP4-dequantized) stacks."""
    from .moe import _check_moe, _pairs_by_expert, silu
    from .quant import bf16_rne_bits, bf16_bits_to_f32

    x, idx, w, E, H, I = _check_moe(x, idx, w, w_gu, w_dn)
    xq = dequantize_mx8_rows(*quantize_mx8_rows(x.astype(np.float32)))
    T, k = idx.shape
    y = np.zeros((T, H), dtype=np.float64)
    for e, t, j in _pairs_by_expert(idx, E):
        h = xq[t] @ np.asarray(w_gu[e], dtype=np.float64).T
        a = silu(h[:, :I]) * h[:, I:]
        a16 = bf16_bits_to_f32(bf16_rne_bits(a.astype(np.float32)))
        aq = dequantize_mx8_rows(*quantize_mx8_rows(a16))
        o = aq @ np.asarray(w_dn[e], dtype=np.float64).T
        np.add.at(y, t, w[t, j][:, None] * o)
    return y

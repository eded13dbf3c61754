"""Blockwise absmax 8-bit storage lanes, int8 and fp8 (oracle).

Test infrastructure: only tests/, the smoke check and the benchmark's CPU
baseline use this module.

The 0.4.0 README's storage-modes support matrix lists two 8-bit blockwise
modes next to nf4 and fp4: ``int8``, a "blockwise dynamic map" (explicitly not
LLM.int8()), and ``fp8``, an "e4m3 codebook" (not torch's float8 type); the
same matrix and the experts-4bit project page state the test-pinned fidelity
ordering fp16 < bf16 < int8 < fp8 < nf4 < fp4 (reconstruction error). The
pages print neither 256-entry table. Readings:

* Layout as the 4-bit stacks, one code byte per element: codes uint8
  ``[E, out*in]``, absmax fp32 ``[E, out*in/64]`` = max |w| of each block of 64
  consecutive row-major elements.
* A code is sign bit 7 | magnitude index bits 6..0 into 128 ascending
  magnitudes m[0] = 0 < ... < m[127] = 1 (absmax scaling maps a block onto
  [-1, 1]); the sign bit is the sign bit of w (so -0.0 stores 0x80).
* fp8: the magnitudes of the E4M3 bit patterns 0x00..0x7F read with exponent
  bias 7, subnormals at exponent 0 and no reserved NaN pattern (a codebook,
  not a float format: the top pattern is 1.875 * 2^8 = 480), divided by 480;
  each rounded once to fp32, nearest even.
* int8: the dynamic tree map of block-wise 8-bit quantization (Dettmers et
  al., "8-bit Optimizers via Block-wise Quantization", arXiv:2110.02861,
  section "Dynamic Tree Quantization"): after the sign, z leading zero bits
  set the decimal exponent 10^-z, the first one bit is the indicator and the
  remaining n = 6 - z bits f choose a linear fraction of [0.1, 1]:
  magnitude = 10^-z * (0.1 + 0.9 * (f + 1) / 2^n), z = 0..6. With the all-zero
  pattern as 0 these are 128 magnitudes, 10^-6 .. 1, stored by ascending
  rank; each rounded once to fp32, nearest even. How the fraction bits map
  onto [0.1, 1] is not fixed by the paper: this is the reading.
* The code of w is the magnitude nearest |w| / absmax, ties to the smaller
  magnitude, decided exactly (see below).
* The dequantized weight is fl32(value(code) * absmax) (one rounding of the
  exact product); its bf16 view is that value rounded to nearest even.

Exactness of the decision: two adjacent magnitudes are fp32 numbers whose
exponents differ by at most 3 (or one of them is 0), so their midpoint needs
at most 28 significant bits and absmax * midpoint (24 more) is exact in fp64.
"""

from fractions import Fraction

import numpy as np

KINDS8 = ("int8", "fp8")


def f32_rne(x):
    """The fp32 value nearest the non-negative rational ``x`` (ties to even)."""
    x = Fraction(x)
    if x < 0:
        raise ValueError("non-negative values only")
    if x == 0:
        return np.float32(0.0)
    c = np.float32(float(x))  # within one fp32 ulp of x
    lo = c if Fraction(float(c)) <= x else np.nextafter(c, np.float32(0.0))
    hi = np.nextafter(lo, np.float32(np.inf))
    dl, dh = x - Fraction(float(lo)), Fraction(float(hi)) - x
    if dl < dh:
        return np.float32(lo)
    if dh < dl:
        return np.float32(hi)
    return np.float32(lo) if (int(lo.view(np.uint32)) & 1) == 0 else np.float32(hi)


def fp8_magnitude_exact(idx):
    """E4M3 pattern ``idx`` (0..127) read with bias 7, no specials, over 480."""
    e, m = idx >> 3, idx & 7
    v = Fraction(m, 8) * Fraction(1, 2**6) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return v / 480


def int8_magnitudes_exact():
    """The 128 dynamic-map magnitudes, ascending (exact rationals)."""
    mags = [Fraction(0)]
    for z in range(6, -1, -1):  # smallest decade first
        n = 6 - z
        for f in range(2**n):
            mags.append(Fraction(1, 10**z) * (Fraction(1, 10) + Fraction(9, 10) * Fraction(f + 1, 2**n)))
    return mags


def magnitudes(kind):
    """fp32 ``[128]`` ascending magnitudes of an 8-bit lane."""
    if kind == "fp8":
        exact = [fp8_magnitude_exact(i) for i in range(128)]
    elif kind == "int8":
        exact = int8_magnitudes_exact()
    else:
        raise ValueError(f"8-bit lane must be 'int8' or 'fp8', got {kind!r}")
    return np.array([f32_rne(v) for v in exact], dtype=np.float32)


def code_values(kind):
    """fp32 ``[256]`` value of every code (bit 7 = sign)."""
    m = magnitudes(kind)
    return np.concatenate([m, -m]).astype(np.float32)


def _check_stack(w, blocksize):
    w = np.asarray(w)
    if w.ndim != 3 or w.dtype != np.float32:
        raise ValueError("weights must be a float32 [E, out, in] stack")
    if blocksize != 64:
        raise ValueError("blocksize must be 64")
    E, out, inn = w.shape
    if E <= 0 or out <= 0 or inn <= 0 or inn % blocksize != 0:
        raise ValueError("bad stack shape")
    if not np.all(np.isfinite(w)):
        raise ValueError("weights must be finite")
    return w


def quantize_blockwise8(w, kind, blocksize=64, chunk_blocks=1 << 15):
    """Quantize a float32 ``[E, out, in]`` stack into an 8-bit lane.

    Returns ``(codes uint8 [E, out*in], absmax float32 [E, out*in/64])``.
    """
    w = _check_stack(w, blocksize)
    mags = magnitudes(kind).astype(np.float64)
    mids = (mags[:-1] + mags[1:]) / 2.0  # exact in fp64
    E, out, inn = w.shape
    nb = out * inn // blocksize
    codes = np.empty((E, out * inn), dtype=np.uint8)
    absmax = np.empty((E, nb), dtype=np.float32)
    for e in range(E):
        blocks_all = w[e].reshape(nb, blocksize)
        for b0 in range(0, nb, chunk_blocks):
            b1 = min(nb, b0 + chunk_blocks)
            blocks = blocks_all[b0:b1].astype(np.float64)
            a = np.abs(blocks)
            am = a.max(axis=1)
            # index = number of midpoints strictly below |w| / absmax (ties stay low)
            idx = np.zeros(blocks.shape, dtype=np.int64)
            for m in mids:
                idx += a > am[:, None] * m
            q = idx + 128 * np.signbit(blocks)
            absmax[e, b0:b1] = am.astype(np.float32)
            codes[e, b0 * blocksize : b1 * blocksize] = q.reshape(-1).astype(np.uint8)
    return codes, absmax


def dequantize8(codes, absmax, out, inn, kind, blocksize=64):
    """fp32 ``[E, out, in]``, every element fl32(value(code) * absmax)."""
    codes = np.asarray(codes, dtype=np.uint8)
    absmax = np.asarray(absmax, dtype=np.float32)
    E = codes.shape[0]
    if codes.shape != (E, out * inn) or absmax.shape != (E, out * inn // blocksize):
        raise ValueError("codes/absmax shapes do not match [E, out, in]")
    v = code_values(kind).astype(np.float64)
    prod = v[codes.reshape(E, -1, blocksize)] * absmax.astype(np.float64)[:, :, None]  # exact
    return prod.astype(np.float32).reshape(E, out, inn)

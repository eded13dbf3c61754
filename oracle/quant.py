"""Blockwise absmax 4-bit quantization of a fused expert stack (oracle).

Follows the experts4bit-qlora 0.1.0 sdist, ``_vendor/experts.py``:
``Experts4bit._quantize_stack`` quantizes each expert of an
``[E, out, in]`` stack on its own with blocksize 64 and no double
quantization (``compress_statistics=False``); ``__init__`` requires
``in % blocksize == 0`` so that a block never straddles a row or an expert,
and stores the packed stack as uint8 ``[E, out*in/2]`` and the scales as
fp32 ``[E, out*in/blocksize]``; ``_dequantize_expert`` recovers one expert as
code value times block absmax.

Readings for what the pages leave open:

* absmax of a block is max |w| over its 64 consecutive row-major elements,
  stored exactly as fp32;
* the code of w is the nearest codebook entry to w/absmax; ties go to the
  lower code for NF4 and to the smaller magnitude for FP4; the decision is
  made exactly (fp64 products absmax * midpoint are exact, see below);
* an NF4 block whose absmax is 0 stores the zero code 7;
* the FP4 sign bit (code bit 3) is the sign bit of w, so a negative value that
  rounds to magnitude 0 stores -0 (code 8), and so does -0.0 itself;
* two codes per byte, the even element in the high nibble;
* the dequantized weight is fl32(code * absmax): one fp64 product (exact for
  fp32 operands) rounded once to fp32; its bf16 view is that fp32 value
  rounded to nearest-even bf16.

Exactness of the decision: every midpoint (c_i + c_{i+1})/2 of two fp32 codes
needs at most 26 significant bits and absmax at most 24, so absmax * midpoint
is exact in fp64 and the comparison w > absmax * midpoint equals the real
comparison w/absmax > midpoint.
"""

import numpy as np

from .codebooks import codebook, ZERO_CODE


def _check_stack(w, blocksize):
    w = np.asarray(w)
    if w.ndim != 3:
        raise ValueError("weights must be a 3-D [E, out, in] stack")
    if w.dtype != np.float32:
        raise ValueError("weights must be float32")
    if blocksize != 64:
        raise ValueError("blocksize must be 64")
    E, out, inn = w.shape
    if E <= 0 or out <= 0 or inn <= 0:
        raise ValueError("empty stack")
    if inn % blocksize != 0:
        raise ValueError("in_features must be divisible by blocksize")
    if not np.all(np.isfinite(w)):
        raise ValueError("weights must be finite")
    return w


def _codes_for_blocks(blocks, absmax, kind):
    """Codes (int) for fp64 ``blocks [n, bs]`` with fp64 ``absmax [n]``."""
    c = codebook(kind).astype(np.float64)
    amax = absmax[:, None]
    if kind == "nf4":
        # thresholds between consecutive entries, ascending
        mids = (c[:-1] + c[1:]) / 2.0
        q = np.zeros(blocks.shape, dtype=np.int64)
        for m in mids:
            q += blocks > amax * m
    else:
        mags = c[:8]
        mids = (mags[:-1] + mags[1:]) / 2.0
        a = np.abs(blocks)
        q = np.zeros(blocks.shape, dtype=np.int64)
        for m in mids:
            q += a > amax * m
        q += 8 * np.signbit(blocks)
    if kind == "nf4":
        q[absmax == 0.0, :] = ZERO_CODE[kind]
    return q


def quantize_blockwise(w, kind="nf4", blocksize=64, chunk_blocks=1 << 16):
    """Quantize a float32 ``[E, out, in]`` stack.

    Returns ``(packed uint8 [E, out*in/2], absmax float32 [E, out*in/64])``.
    """
    if kind not in ("nf4", "fp4"):
        raise ValueError(f"codebook must be 'nf4' or 'fp4', got {kind!r}")
    w = _check_stack(w, blocksize)
    E, out, inn = w.shape
    nb = out * inn // blocksize
    packed = np.empty((E, out * inn // 2), dtype=np.uint8)
    absmax = np.empty((E, nb), dtype=np.float32)
    for e in range(E):
        blocks_all = w[e].reshape(nb, blocksize)
        for b0 in range(0, nb, chunk_blocks):
            b1 = min(nb, b0 + chunk_blocks)
            blocks = blocks_all[b0:b1].astype(np.float64)
            am = np.abs(blocks).max(axis=1)
            q = _codes_for_blocks(blocks, am, kind).reshape(-1)
            absmax[e, b0:b1] = am.astype(np.float32)  # exact: am is an fp32 value
            packed[e, b0 * blocksize // 2 : b1 * blocksize // 2] = (
                (q[0::2] << 4) | q[1::2]
            ).astype(np.uint8)
    return packed, absmax


def unpack_codes(packed):
    """Codes ``[E, 2*n]`` from packed bytes ``[E, n]`` (even element = high nibble)."""
    p = np.asarray(packed, dtype=np.uint8)
    q = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    q[..., 0::2] = p >> 4
    q[..., 1::2] = p & 0xF
    return q


def dequantize(packed, absmax, out, inn, kind="nf4", blocksize=64):
    """fp32 ``[E, out, in]`` with every element fl32(code * absmax)."""
    packed = np.asarray(packed, dtype=np.uint8)
    absmax = np.asarray(absmax, dtype=np.float32)
    E = packed.shape[0]
    if packed.shape != (E, out * inn // 2) or absmax.shape != (E, out * inn // blocksize):
        raise ValueError("packed/absmax shapes do not match [E, out, in]")
    c = codebook(kind).astype(np.float64)
    q = unpack_codes(packed).reshape(E, -1, blocksize)
    prod = c[q] * absmax.astype(np.float64)[:, :, None]  # exact product
    return prod.astype(np.float32).reshape(E, out, inn)  # one rounding


def bf16_rne_bits(x):
    """bf16 bit patterns (uint16) of float32 ``x``, rounding to nearest even."""
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16 rounding is defined here for finite values only")
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """float32 values of bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def stored_weights(w, kind):
    """fp32 values that a stack stored in mode ``kind`` represents.

    ``nf4`` / ``fp4``: blockwise quantize then dequantize (above). ``mxfp4``:
    the MX conversion and its exact dequantization (``oracle.mx``). ``bf16``:
    the 16-bit passthrough lane of the 0.4.0 README's support matrix (the
    reference baseline, no absmax): each weight rounded to bf16, nearest
    even.
    """
    w = np.asarray(w, dtype=np.float32)
    if kind == "bf16":
        return bf16_bits_to_f32(bf16_rne_bits(w))
    E, out, inn = w.shape
    if kind in ("int8", "fp8"):
        from .quant8 import quantize_blockwise8, dequantize8

        return dequantize8(*quantize_blockwise8(w, kind), out, inn, kind)
    if kind == "mxfp4":
        from .mx import quantize_mx, dequantize_mx

        return dequantize_mx(*quantize_mx(w), out, inn)
    packed, absmax = quantize_blockwise(w, kind)
    return dequantize(packed, absmax, out, inn, kind)

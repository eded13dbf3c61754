"""The two 16-entry 4-bit codebooks (oracle copy).

The pages name both storage types without printing their values: the
experts4bit-qlora 0.1.0 sdist's ``Experts4bit.__init__`` rebuilds a 16-entry
fp32 code buffer from ``quant_type`` ("nf4" or "fp4"), and the 0.4.0 README's
support matrix describes fp4 as the alternative codebook that is coarser than
nf4 on roughly Gaussian weights.

* NF4: the NormalFloat-4 table published in the QLoRA paper (Dettmers et al.
  2023, arXiv:2305.14314, appendix "NormalFloat 4-bit data type"), code
  order 0..15, every value an exact fp32 number. Pinned in the tests against
  the published table (tests/golden/nf4_codebook.txt) and against its
  normal-quantile construction.
* FP4: reading of "FP4 (e2m1)": code = sign bit 3 | e2m1 magnitude bits 2..0,
  magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6} divided by 6 so that the largest
  magnitude is 1 (absmax scaling maps a block onto [-1, 1]). Code 8 is -0.0.
  Compatibility with bitsandbytes' own fp4 table is not claimed (that table is
  not on the pages). Pinned in the tests against an independent e2m1 decode.
"""

import numpy as np

# NormalFloat-4, QLoRA appendix table, code order 0..15.
NF4_CODE = np.array(
    [
        -1.0,
        -0.6961928009986877,
        -0.5250730514526367,
        -0.39491748809814453,
        -0.28444138169288635,
        -0.18477343022823334,
        -0.09105003625154495,
        0.0,
        0.07958029955625534,
        0.16093020141124725,
        0.24611230194568634,
        0.33791524171829224,
        0.44070982933044434,
        0.5626170039176941,
        0.7229568362236023,
        1.0,
    ],
    dtype=np.float32,
)

# FP4 e2m1 magnitudes over 6, fp32; codes 8..15 are the negated codes 0..7.
_FP4_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64) / 6.0
FP4_CODE = np.concatenate([_FP4_MAG, -_FP4_MAG]).astype(np.float32)

# The code of +0.0 (an NF4 block whose absmax is 0 stores it everywhere; FP4
# stores +0 as 0 and -0 as 8).
ZERO_CODE = {"nf4": 7, "fp4": 0}


def codebook(kind):
    """Return the 16-entry fp32 codebook for ``kind`` in {"nf4", "fp4"}."""
    if kind == "nf4":
        return NF4_CODE.copy()
    if kind == "fp4":
        return FP4_CODE.copy()
    raise ValueError(f"codebook must be 'nf4' or 'fp4', got {kind!r}")

"""Storage fidelity measures (oracle).

The 0.4.0 README (storage-modes support matrix) and the experts-4bit project
page state a fidelity ordering of the storage modes by reconstruction error,
fp16 < bf16 < int8 < fp8 < nf4 < fp4 (fp16 is not a lane here). The pages' absolute numbers use a metric they do not
define and bitsandbytes' own tables, so only the ordering is reproduced here
(absolute values: parity unpinned).

Reading of the metric: relative Frobenius error ||A - B||_F / ||A||_F, applied
to the weights themselves and to the forward output computed from them.
"""

import numpy as np

from .quant import quantize_blockwise, dequantize, bf16_rne_bits, bf16_bits_to_f32


def rel_fro(ref, approx):
    ref = np.asarray(ref, dtype=np.float64)
    approx = np.asarray(approx, dtype=np.float64)
    return float(np.linalg.norm(ref - approx) / np.linalg.norm(ref))


def reconstruction_errors(w):
    """rel_fro of a float32 ``[E, out, in]`` stack under bf16, int8, fp8, nf4 and fp4 storage."""
    from .quant8 import quantize_blockwise8, dequantize8

    w = np.asarray(w, dtype=np.float32)
    E, out, inn = w.shape
    res = {"bf16": rel_fro(w, bf16_bits_to_f32(bf16_rne_bits(w)))}
    for kind in ("int8", "fp8"):
        c, a = quantize_blockwise8(w, kind)
        res[kind] = rel_fro(w, dequantize8(c, a, out, inn, kind))
    for kind in ("nf4", "fp4"):
        p, a = quantize_blockwise(w, kind)
        res[kind] = rel_fro(w, dequantize(p, a, out, inn, kind))
    return res

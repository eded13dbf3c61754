"""CPU oracle for the fused blockwise-4-bit Mixture-of-Experts expert MLP.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code, table or
helper with the HIP library; each side holds its own copy of every constant.

What it computes (float64 unless a step fixes another precision):

* ``codebooks``  -- the two 16-entry 4-bit codebooks (NF4, FP4 e2m1).
* ``quant``      -- blockwise absmax quantization of a fused ``[E, out, in]``
  expert stack, nibble packing, dequantization, and the bf16 rounding used to
  define the bf16 view of a dequantized weight.
* ``moe``        -- top-k routing, the token-by-expert permutation, the
  SwiGLU expert forward, and the frozen-base input gradient (dgrad).
* ``fidelity``   -- relative reconstruction / forward error used for the
  storage-fidelity ordering.
* ``lora``       -- per-expert LoRA adapters over the frozen base: forward,
  dgrad and the adapter weight gradients.
* ``mx``         -- MXFP4 storage: E2M1 elements with an E8M0 scale per 32
  elements (the conversion rule of the OCP MX v1.0 specification), and its
  exact dequantization; MXFP8 (E4M3) activation rows and the MX forward that
  feeds them to the MXFP4 weights.

Sources: the experts4bit-qlora / bitsandbytes pages on fused 4-bit expert
storage (the 0.1.0 sdist's ``_vendor/experts.py`` module ``Experts4bit``; the
bitsandbytes pull request #1965 "Add Experts4bit for 4-bit quantization of
fused MoE experts"; the 0.4.0 README's support matrix). Each function cites
the passage it follows.

Pin status (see tests/test_oracle_*.py):

* codebooks, quantize, dequantize, bf16 rounding, route, permute, forward,
  dgrad, fidelity ordering, LoRA forward / backward, MXFP4 conversion and
  dequantization: pinned by published
  tables, closed forms (merged weights W + s B A), brute force, finite
  differences and library cross-checks.
* absolute fidelity magnitudes quoted on the pages (forward relative error
  about 0.17 nf4 / 0.22 fp4 / 0.003 bf16) use an undefined metric and
  bitsandbytes' own tables: parity unpinned. Only the ordering is checked.
"""

from .codebooks import codebook, NF4_CODE, FP4_CODE, ZERO_CODE  # noqa: F401
from .quant import (  # noqa: F401
    quantize_blockwise,
    dequantize,
    bf16_rne_bits,
    bf16_bits_to_f32,
    unpack_codes,
    stored_weights,
)
from .moe import route, permute, moe_forward, moe_dgrad, silu  # noqa: F401
from .fidelity import rel_fro, reconstruction_errors  # noqa: F401
from .lora import lora_forward, lora_backward  # noqa: F401
from .mx import (  # noqa: F401
    quantize_mx,
    dequantize_mx,
    e2m1_value,
    e8m0_value,
    e4m3_value,
    quantize_mx8_rows,
    dequantize_mx8_rows,
    mx8_forward,
)

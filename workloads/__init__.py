"""Seeded synthetic inputs for the routed 4-bit expert MLP workloads.

This module holds no arithmetic of the method itself: it only draws random
inputs (activations, fp32 expert weights, router logits, output gradients)
with the shapes and distributions of the pages' workloads. Both the HIP
path's tests/bench and the CPU oracle read the same arrays from here.

Every tensor is drawn from its own PCG64 stream keyed by
``(seed, tensor id[, expert])`` so that a tensor (or one expert of a weight
stack) can be regenerated alone, in any order, bit-identically.

Distributions (the workloads' recipe):

* activations x and output gradients grad_y: N(0, 1) drawn in fp32, rounded
  to bf16 (nearest even, via torch's conversion);
* expert weights: fp32 N(0, 0.02^2);
* per-expert LoRA adapters (fp32): N(0, 0.02^2), A [E, r, in], B [E, out, r];
* router logits (fp32): ``normal`` N(0, 1); ``uniform`` i.i.d. U[0, 1);
  ``zipf`` ``-s*ln(e+1) + Gumbel(0, 1)`` so that Gumbel top-k draws k
  distinct experts with P(e) proportional to (e+1)^-s (expert 0 hottest).
"""

from .configs import CONFIGS, MoEConfig, get_config  # noqa: F401
from .gen import (  # noqa: F401
    gen_x,
    gen_grad_y,
    gen_logits,
    gen_weights,
    gen_expert_weight,
    gen_lora,
    to_bf16_tensor,
)

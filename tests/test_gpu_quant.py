"""GPU parity: e4b_quantize_nf4 / e4b_dequantize_nf4 against the oracle, bit-exact."""

import numpy as np
import pytest
import torch

import oracle
import bit_quantized_mixture_nf4_amd as e4b
from workloads import get_config, gen_weights
from gpu_util import DEV, announce

pytestmark = pytest.mark.gpu

KINDS = ("nf4", "fp4")


def _adversarial(kind, rows=32, inn=128, seed=0):
    """Blocks holding exact codebook points, midpoints and their fp32 neighbours, zeros, -0.0."""
    rng = np.random.default_rng(seed)
    c = oracle.codebook(kind).astype(np.float64)
    pts = np.concatenate([c, (c[:-1] + c[1:]) / 2]).astype(np.float32)
    pts = np.concatenate([pts, np.nextafter(pts, np.float32(2)), np.nextafter(pts, np.float32(-2))])
    pts = pts[np.abs(pts) <= 1]
    w = (rng.standard_normal((rows, inn)) * 0.02).astype(np.float32)
    for r in range(0, rows, 2):
        blk = rng.choice(pts, size=64).astype(np.float32) * np.float32(2.0 ** rng.integers(-8, 2))
        blk[0] = np.float32(2.0 ** rng.integers(-8, 2))  # pins absmax
        w[r, :64] = blk
    w[1, 64:] = 0.0
    w[3, 64:] = -0.0
    w[5, 70] = -1e-30
    return w[None]


def _check_stack(w, kind):
    announce(f"quantize {kind} shape={w.shape}")
    st = e4b.quantize(torch.from_numpy(w).to(DEV), kind)
    p_ref, a_ref = oracle.quantize_blockwise(w, kind)
    assert np.array_equal(st.packed.cpu().numpy(), p_ref)
    assert np.array_equal(st.absmax.cpu().numpy().view(np.uint32), a_ref.view(np.uint32))
    E, out, inn = w.shape
    ref32 = oracle.dequantize(p_ref, a_ref, out, inn, kind)
    got32 = e4b.dequantize(st, torch.float32).cpu().numpy()
    assert np.array_equal(got32.view(np.uint32), ref32.view(np.uint32))
    got16 = e4b.dequantize(st, torch.bfloat16).cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got16, oracle.bf16_rne_bits(ref32))


@pytest.mark.parametrize("kind", KINDS)
def test_quant_dequant_tiny_layer_bit_exact(kind):
    cfg = get_config("tiny")
    _check_stack(gen_weights(cfg, 0, "gate_up"), kind)
    _check_stack(gen_weights(cfg, 0, "down"), kind)


@pytest.mark.parametrize("kind", KINDS)
def test_quant_adversarial_blocks_bit_exact(kind):
    _check_stack(_adversarial(kind), kind)

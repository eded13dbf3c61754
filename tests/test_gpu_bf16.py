"""GPU parity of the bf16 passthrough lane (storage mode BF16: the weight is
kept as bf16, no absmax; the same grouped GEMMs stage it without a codebook).

Bar: stored bits equal the oracle's round-to-nearest-even bit for bit and
dequantize returns them exactly; forward, dgrad and LoRA outputs within
1e-2 * max|oracle| per tensor; the decode path is refused for a bf16 layer.
"""

import numpy as np
import pytest
import torch

import oracle
import bit_quantized_mixture_nf4_amd as e4b
from workloads import MoEConfig, get_config, gen_lora
from gpu_util import DEV, Problem, announce, tol_check, to_np

pytestmark = pytest.mark.gpu


def test_bf16_store_and_dequantize_exact():
    announce("bf16 lane store E3 out96 in192")
    w = (np.random.default_rng(0).standard_normal((3, 96, 192)) * 0.05).astype(np.float32)
    w[0, 0, :8] = [0.0, -0.0, 1e-30, -1e-30, 3.0e38, -3.0e38, 1.00390625, 1.01171875]  # ties, tiny, huge
    st = e4b.quantize(torch.from_numpy(w).to(DEV), "bf16")
    assert st.absmax is None
    bits = st.packed.view(torch.int16).cpu().numpy().view(np.uint16).reshape(3, 96 * 192)
    assert np.array_equal(bits, oracle.bf16_rne_bits(w).reshape(3, -1))
    f32 = e4b.dequantize(st).cpu().numpy()
    assert np.array_equal(f32.view(np.uint32), oracle.stored_weights(w, "bf16").view(np.uint32))
    b16 = e4b.dequantize(st, torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(b16.reshape(3, -1), bits)


@pytest.mark.parametrize("shape", ["tiny", "ragged"])
def test_bf16_forward_dgrad(shape):
    cfg = get_config("tiny") if shape == "tiny" else MoEConfig(
        "bf16_ragged", E=6, H=192, I=320, k=2, T=300, routing="normal")
    announce(f"bf16 lane forward/dgrad {cfg.name}")
    pb = Problem(cfg, seed=4, codebook="bf16")
    y, idx, w, saved = e4b.moe_forward(pb.layer, pb.x_d, cfg.k, logits=pb.logits_d, save=True)
    idx_ref, w_ref = oracle.route(pb.logits, cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    wgu, wdn = pb.oracle_weights()
    tol_check(to_np(y), oracle.moe_forward(pb.x, idx_ref, w_ref, wgu, wdn), f"y bf16 {cfg.name}")
    gx, gw = e4b.moe_dgrad(pb.layer, idx, w, pb.grad_y_d, saved=saved)
    gx_ref, gw_ref = oracle.moe_dgrad(pb.x, idx_ref, w_ref, wgu, wdn, pb.grad_y)
    tol_check(to_np(gx), gx_ref, f"grad_x bf16 {cfg.name}")
    tol_check(to_np(gw), gw_ref, f"grad_w bf16 {cfg.name}")
    gx2, gw2 = e4b.moe_dgrad(pb.layer, idx, w, pb.grad_y_d, x=pb.x_d)
    assert torch.equal(gx.view(torch.int16), gx2.view(torch.int16)) and torch.equal(gw, gw2)


def test_bf16_small_batch_takes_the_grouped_path():
    cfg = get_config("tiny", 6)
    announce("bf16 lane T=6 auto path")
    pb = Problem(cfg, seed=5, codebook="bf16", with_grad=False)
    with pytest.raises(ValueError):
        e4b.moe_forward(pb.layer, pb.x_d, cfg.k, logits=pb.logits_d, path="decode")
    y, idx, w, _ = e4b.moe_forward(pb.layer, pb.x_d, cfg.k, logits=pb.logits_d)
    wgu, wdn = pb.oracle_weights()
    idx_ref, w_ref = oracle.route(pb.logits, cfg.k)
    tol_check(to_np(y), oracle.moe_forward(pb.x, idx_ref, w_ref, wgu, wdn), "y bf16 T=6")


def test_bf16_base_with_lora():
    cfg = get_config("tiny")
    announce("bf16 lane + lora r8")
    pb = Problem(cfg, seed=6, codebook="bf16")
    host = gen_lora(cfg, 3, 8)
    lo = e4b.Lora(*(torch.from_numpy(m).to(DEV) for m in host), alpha=16.0)
    y, idx, w, saved = e4b.moe_lora_forward(pb.layer, lo, pb.x_d, cfg.k, logits=pb.logits_d, save=True)
    idx_ref, w_ref = oracle.route(pb.logits, cfg.k)
    wgu, wdn = pb.oracle_weights()
    tol_check(to_np(y), oracle.lora_forward(pb.x, idx_ref, w_ref, wgu, wdn, *host, 16.0), "y bf16 lora")
    gx, gw, grads = e4b.moe_lora_backward(pb.layer, lo, idx, w, pb.x_d, pb.grad_y_d, saved=saved)
    ref = oracle.lora_backward(pb.x, idx_ref, w_ref, wgu, wdn, *host, 16.0, pb.grad_y)
    for name, got, want in zip(("grad_x", "grad_w", "dA_gu", "dB_gu", "dA_dn", "dB_dn"),
                               (gx, gw) + grads, ref):
        tol_check(to_np(got), want, f"{name} bf16 lora")

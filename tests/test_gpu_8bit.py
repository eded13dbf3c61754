"""GPU parity of the 8-bit storage lanes INT8 (dynamic tree map) and FP8
(E4M3 codebook), against oracle/quant8.py.

Bar: stored codes and absmax bit-exact, dequantize (fp32, bf16) bit-exact;
forward, dgrad and LoRA outputs within 1e-2 * max|oracle| per tensor; the
decode path is refused (the support matrix gives these lanes no GEMV) and
`auto` takes the grouped path for T <= 8; on the GPU's own outputs the
fidelity ordering bf16 < int8 < fp8 < nf4 < fp4 of the support matrix holds.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import quant8
import bit_quantized_mixture_nf4_amd as e4b
from workloads import MoEConfig, get_config, gen_lora
from gpu_util import DEV, Problem, announce, bf16_tensor, tol_check, to_np

pytestmark = pytest.mark.gpu
KINDS = ("int8", "fp8")


def _adversarial(kind):
    """Blocks with exact midpoint ties (absmax 1), zeros, -0, heavy tails and
    extreme scales, [1, 8, 64] fp32."""
    rng = np.random.default_rng(11)
    m = quant8.magnitudes(kind).astype(np.float64)
    mids = (m[:-1] + m[1:]) / 2
    ties = np.array([v for v in mids if np.float64(np.float32(v)) == v][:63], np.float32)
    rows = [np.concatenate([[1.0], ties, np.zeros(63 - len(ties))])]
    rows.append(-rows[0])
    rows.append(np.zeros(64))
    rows.append(-np.zeros(64))
    rows.append(rng.standard_normal(64) ** 7)
    rows.append(rng.standard_normal(64) * 3.0e38 / 8)
    rows.append(rng.standard_normal(64) * 1e-30)
    # values next to every magnitude boundary, scaled by a non-power-of-two absmax
    rows.append(np.concatenate([[0.7], 0.7 * rng.choice(mids, 63)]) * (1 + 2e-7 * rng.standard_normal(64)))
    return np.stack(rows).astype(np.float32)[None]


@pytest.mark.parametrize("kind", KINDS)
def test_quantize_and_dequantize_bit_exact(kind):
    announce(f"{kind} store: tiny stack + adversarial blocks")
    cfg = get_config("tiny")
    pb = Problem(cfg, seed=2, codebook=kind, with_grad=False)
    for host, st in ((pb.w_gu, pb.layer.gate_up), (pb.w_dn, pb.layer.down)):
        codes, absmax = quant8.quantize_blockwise8(host, kind)
        assert np.array_equal(st.packed.cpu().numpy(), codes)
        assert np.array_equal(st.absmax.cpu().numpy().view(np.uint32), absmax.view(np.uint32))
    w = _adversarial(kind)
    st = e4b.quantize(torch.from_numpy(w).to(DEV), kind)
    codes, absmax = quant8.quantize_blockwise8(w, kind)
    assert np.array_equal(st.packed.cpu().numpy(), codes)
    assert np.array_equal(st.absmax.cpu().numpy().view(np.uint32), absmax.view(np.uint32))
    ref = quant8.dequantize8(codes, absmax, 8, 64, kind)
    f32 = e4b.dequantize(st).cpu().numpy()
    assert np.array_equal(f32.view(np.uint32), ref.view(np.uint32))
    b16 = e4b.dequantize(st, torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(b16, oracle.bf16_rne_bits(ref))


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("shape", ["tiny", "ragged"])
def test_forward_dgrad(kind, shape):
    cfg = get_config("tiny") if shape == "tiny" else MoEConfig(
        "w8_ragged", E=6, H=192, I=320, k=2, T=700, routing="normal")
    announce(f"{kind} lane forward/dgrad {cfg.name}")
    pb = Problem(cfg, seed=4, codebook=kind)
    y, idx, w, saved = e4b.moe_forward(pb.layer, pb.x_d, cfg.k, logits=pb.logits_d, save=True)
    idx_ref, w_ref = oracle.route(pb.logits, cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    wgu, wdn = pb.oracle_weights()
    tol_check(to_np(y), oracle.moe_forward(pb.x, idx_ref, w_ref, wgu, wdn), f"y {kind} {cfg.name}")
    gx, gw = e4b.moe_dgrad(pb.layer, idx, w, pb.grad_y_d, saved=saved)
    gx_ref, gw_ref = oracle.moe_dgrad(pb.x, idx_ref, w_ref, wgu, wdn, pb.grad_y)
    tol_check(to_np(gx), gx_ref, f"grad_x {kind} {cfg.name}")
    tol_check(to_np(gw), gw_ref, f"grad_w {kind} {cfg.name}")
    gx2, gw2 = e4b.moe_dgrad(pb.layer, idx, w, pb.grad_y_d, x=pb.x_d)
    assert torch.equal(gx.view(torch.int16), gx2.view(torch.int16)) and torch.equal(gw, gw2)


@pytest.mark.parametrize("kind", KINDS)
def test_small_batch_takes_the_grouped_path(kind):
    cfg = get_config("tiny", 5)
    announce(f"{kind} lane T=5: decode refused, auto is grouped")
    pb = Problem(cfg, seed=5, codebook=kind, with_grad=False)
    with pytest.raises(ValueError):
        e4b.moe_forward(pb.layer, pb.x_d, cfg.k, logits=pb.logits_d, path="decode")
    y, idx, w, _ = e4b.moe_forward(pb.layer, pb.x_d, cfg.k, logits=pb.logits_d)
    wgu, wdn = pb.oracle_weights()
    idx_ref, w_ref = oracle.route(pb.logits, cfg.k)
    tol_check(to_np(y), oracle.moe_forward(pb.x, idx_ref, w_ref, wgu, wdn), f"y {kind} T=5")


def test_int8_base_with_lora():
    cfg = get_config("tiny")
    announce("int8 lane + lora r8")
    pb = Problem(cfg, seed=6, codebook="int8")
    host = gen_lora(cfg, 3, 8)
    lo = e4b.Lora(*(torch.from_numpy(m).to(DEV) for m in host), alpha=16.0)
    y, idx, w, saved = e4b.moe_lora_forward(pb.layer, lo, pb.x_d, cfg.k, logits=pb.logits_d, save=True)
    idx_ref, w_ref = oracle.route(pb.logits, cfg.k)
    wgu, wdn = pb.oracle_weights()
    tol_check(to_np(y), oracle.lora_forward(pb.x, idx_ref, w_ref, wgu, wdn, *host, 16.0), "y int8 lora")
    gx, gw, grads = e4b.moe_lora_backward(pb.layer, lo, idx, w, pb.x_d, pb.grad_y_d, saved=saved)
    ref = oracle.lora_backward(pb.x, idx_ref, w_ref, wgu, wdn, *host, 16.0, pb.grad_y)
    for name, got, want in zip(("grad_x", "grad_w", "dA_gu", "dB_gu", "dA_dn", "dB_dn"),
                               (gx, gw) + grads, ref):
        tol_check(to_np(got), want, f"{name} int8 lora")


def test_fidelity_ordering_from_gpu_outputs():
    """The support matrix's ordering bf16 < int8 < fp8 < nf4 < fp4, measured on
    the GPU forward of each storage mode against the oracle's forward on the
    unquantized weights (same routing)."""
    cfg = MoEConfig("w8_fid", E=8, H=1024, I=512, k=2, T=512, routing="uniform")
    announce("fidelity ordering of the storage modes on GPU outputs E8 H1024 I512 T512")
    rel = {}
    y_exact = None
    for kind in ("bf16", "int8", "fp8", "nf4", "fp4"):
        pb = Problem(cfg, seed=0, codebook=kind, with_grad=False)
        idx_ref, w_ref = oracle.route(pb.logits, cfg.k)
        if y_exact is None:
            y_exact = oracle.moe_forward(pb.x, idx_ref, w_ref, pb.w_gu, pb.w_dn)
        y, _, _, _ = e4b.moe_forward(pb.layer, pb.x_d, cfg.k, logits=pb.logits_d, path="grouped")
        rel[kind] = oracle.rel_fro(y_exact, to_np(y).astype(np.float64))
        del pb
    announce(f"rel(y): {rel}")
    assert rel["bf16"] < rel["int8"] < rel["fp8"] < rel["nf4"] < rel["fp4"], rel

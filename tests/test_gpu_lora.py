"""GPU parity of the per-expert LoRA forward / backward against the oracle.

Bar: y, grad_x, grad_topk_w and every adapter gradient within
1e-2 * max|oracle| per tensor; with B = 0 the outputs equal the base path's
bit for bit; backward with the saved state equals the recomputing backward
bit for bit; two runs are bitwise identical.
"""

import numpy as np
import pytest
import torch

import oracle
import bit_quantized_mixture_nf4_amd as e4b
from workloads import MoEConfig, get_config, gen_lora
from gpu_util import DEV, Problem, announce, tol_check, to_np

pytestmark = pytest.mark.gpu


def _adapters(cfg, seed, r, alpha, zero_b=False):
    host = list(gen_lora(cfg, seed, r))
    if zero_b:
        host[1] = np.zeros_like(host[1])
        host[3] = np.zeros_like(host[3])
    dev = [torch.from_numpy(m).to(DEV) for m in host]
    return host, e4b.Lora(*dev, alpha=alpha)


def _routing(pb, cfg):
    idx, w = oracle.route(pb.logits, cfg.k)
    return idx, w


def _check_all(pb, cfg, r, alpha, seed=0, save=True):
    host, lo = _adapters(cfg, seed, r, alpha)
    y, idx, w, saved = e4b.moe_lora_forward(pb.layer, lo, pb.x_d, cfg.k, logits=pb.logits_d,
                                            save=save)
    idx_ref, w_ref = _routing(pb, cfg)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    wgu, wdn = pb.oracle_weights()
    y_ref = oracle.lora_forward(pb.x, idx_ref, w_ref, wgu, wdn, *host, alpha)
    tol_check(to_np(y), y_ref, f"y lora {cfg.name}")
    gx, gw, grads = e4b.moe_lora_backward(pb.layer, lo, idx, w, pb.x_d, pb.grad_y_d, saved=saved)
    ref = oracle.lora_backward(pb.x, idx_ref, w_ref, wgu, wdn, *host, alpha, pb.grad_y)
    names = ("grad_x", "grad_w", "dA_gu", "dB_gu", "dA_dn", "dB_dn")
    for name, got, want in zip(names, (gx, gw) + grads, ref):
        tol_check(to_np(got), want, f"{name} lora {cfg.name}")
    return lo, idx, w, saved, (y, gx, gw) + grads


@pytest.fixture(scope="module")
def tiny():
    announce("lora tiny E8 H256 I128 k2 T64")
    return Problem(get_config("tiny"), seed=0)


def test_lora_tiny_forward_backward(tiny):
    _check_all(tiny, tiny.cfg, r=8, alpha=16.0)


def test_lora_recompute_equals_saved_and_runs_are_deterministic(tiny):
    cfg = tiny.cfg
    lo, idx, w, saved, outs = _check_all(tiny, cfg, r=8, alpha=16.0)
    gx2, gw2, grads2 = e4b.moe_lora_backward(tiny.layer, lo, idx, w, tiny.x_d, tiny.grad_y_d)
    for a, b in zip(outs[1:], (gx2, gw2) + grads2):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    y3, _, _, saved3 = e4b.moe_lora_forward(tiny.layer, lo, tiny.x_d, cfg.k, logits=tiny.logits_d,
                                            save=True)
    gx3, gw3, grads3 = e4b.moe_lora_backward(tiny.layer, lo, idx, w, tiny.x_d, tiny.grad_y_d,
                                             saved=saved3)
    for a, b in zip(outs, (y3, gx3, gw3) + grads3):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_lora_zero_b_is_the_base_path(tiny):
    cfg = tiny.cfg
    _, lo = _adapters(cfg, 1, 8, 16.0, zero_b=True)
    y, idx, w, saved = e4b.moe_lora_forward(tiny.layer, lo, tiny.x_d, cfg.k, logits=tiny.logits_d,
                                            save=True)
    yb, _, _, savedb = e4b.moe_forward(tiny.layer, tiny.x_d, cfg.k, logits=tiny.logits_d,
                                       save=True, path="grouped")
    assert torch.equal(y.view(torch.uint8), yb.view(torch.uint8))
    gx, gw, (dA_gu, dB_gu, dA_dn, dB_dn) = e4b.moe_lora_backward(tiny.layer, lo, idx, w, tiny.x_d,
                                                                 tiny.grad_y_d, saved=saved)
    gxb, gwb = e4b.moe_dgrad(tiny.layer, idx, w, tiny.grad_y_d, saved=savedb)
    assert torch.equal(gx.view(torch.uint8), gxb.view(torch.uint8))
    assert torch.equal(gw, gwb)
    assert not dA_gu.any() and not dA_dn.any()


@pytest.mark.parametrize("r", [5, 16])
def test_lora_ragged_shapes(r):
    """I not a multiple of 128, an expert with several m-tiles, ranks 5 and 16."""
    cfg = MoEConfig("lora_ragged", E=6, H=192, I=320, k=2, T=300, routing="normal")
    announce(f"lora ragged E6 H192 I320 k2 T300 r{r}")
    pb = Problem(cfg, seed=3)
    _check_all(pb, cfg, r=r, alpha=2.0 * r, seed=2, save=(r == 16))

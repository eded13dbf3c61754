"""GPU parity of the ungated expert MLP (has_gate=False: the first stack is a
plain up projection [E, I, H] and a = silu(h)) against the oracle.

Bar: y, grad_x, grad_topk_w within 1e-2 * max|oracle| per tensor; the
recomputing dgrad equals the saved-state dgrad bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
import bit_quantized_mixture_nf4_amd as e4b
from workloads import MoEConfig
from gpu_util import Problem, announce, tol_check, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("E,H,I,k,T,kind", [(8, 256, 128, 2, 64, "nf4"), (6, 192, 320, 2, 300, "nf4"),
                                            (6, 192, 320, 2, 300, "bf16"), (4, 128, 64, 2, 5, "fp4"),
                                            (6, 192, 320, 2, 300, "int8"), (6, 192, 320, 2, 300, "fp8")])
def test_ungated_forward_dgrad(E, H, I, k, T, kind):
    cfg = MoEConfig("ungated", E=E, H=H, I=I, k=k, T=T, routing="normal", gated=False)
    announce(f"ungated {kind} E{E} H{H} I{I} k{k} T{T}")
    pb = Problem(cfg, seed=7, codebook=kind)
    assert pb.layer.gate_up.out == I
    y, idx, w, saved = e4b.moe_forward(pb.layer, pb.x_d, k, logits=pb.logits_d, save=True)
    idx_ref, w_ref = oracle.route(pb.logits, k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    wup, wdn = pb.oracle_weights()
    tol_check(to_np(y), oracle.moe_forward(pb.x, idx_ref, w_ref, wup, wdn), f"y ungated {kind}")
    gx, gw = e4b.moe_dgrad(pb.layer, idx, w, pb.grad_y_d, saved=saved)
    gx_ref, gw_ref = oracle.moe_dgrad(pb.x, idx_ref, w_ref, wup, wdn, pb.grad_y)
    tol_check(to_np(gx), gx_ref, f"grad_x ungated {kind}")
    tol_check(to_np(gw), gw_ref, f"grad_w ungated {kind}")
    gx2, gw2 = e4b.moe_dgrad(pb.layer, idx, w, pb.grad_y_d, x=pb.x_d)
    assert torch.equal(gx.view(torch.int16), gx2.view(torch.int16)) and torch.equal(gw, gw2)

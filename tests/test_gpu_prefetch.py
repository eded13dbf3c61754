"""Layer-granular prefetch for decode: layers kept in pinned host memory are
copied into two device slots on a side stream while the previous layer
computes. Every streamed output must match the oracle's forward on that
layer's weights (1e-2 * max|oracle|) and equal, bit for bit, the output of
the same layer kept resident on the device."""

import numpy as np
import pytest
import torch

import oracle
import bit_quantized_mixture_nf4_amd as e4b
from workloads import get_config
from gpu_util import DEV, Problem, announce, tol_check, to_np

pytestmark = pytest.mark.gpu


def _pinned(layer):
    stacks = []
    for st in (layer.gate_up, layer.down):
        stacks.append(e4b.QuantStack(st.packed.cpu().pin_memory(),
                                     None if st.absmax is None else st.absmax.cpu().pin_memory(),
                                     st.E, st.out, st.inn, st.codebook))
    return e4b.MoELayer(*stacks)


@pytest.mark.parametrize("kind,path", [("nf4", "decode"), ("bf16", "grouped")])
def test_streamed_layers_equal_resident_layers(kind, path):
    cfg = get_config("tiny", 4)
    announce(f"prefetch {kind} {path} 3 layers x 2 passes")
    probs = [Problem(cfg, seed=s, codebook=kind, with_grad=False) for s in (11, 12, 13)]
    x = probs[0].x_d
    idx = torch.tensor([[0, 1], [2, 3], [1, 5], [7, 0]], dtype=torch.int32, device=DEV)
    w = torch.full((4, 2), 0.5, dtype=torch.float32, device=DEV)
    resident = [e4b.moe_forward(p.layer, x, 2, topk_idx=idx, topk_w=w, path=path)[0] for p in probs]
    pf = e4b.LayerPrefetcher([_pinned(p.layer) for p in probs])
    order = [0, 1, 2, 0, 1, 2]
    outs = []
    pf.prefetch(order[0])
    for i, l in enumerate(order):
        if i + 1 < len(order):
            pf.prefetch(order[i + 1])  # copies while layer l computes
        layer = pf.acquire(l)
        outs.append(e4b.moe_forward(layer, x, 2, topk_idx=idx, topk_w=w, path=path)[0])
        pf.release(l)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    w_np = w.cpu().numpy().astype(np.float64)
    refs = []
    for p in probs:
        wgu, wdn = p.oracle_weights()
        refs.append(oracle.moe_forward(probs[0].x, idx_np, w_np, wgu, wdn))
    for i, (l, y) in enumerate(zip(order, outs)):
        tol_check(to_np(y), refs[l], f"streamed layer {l} (step {i})")
        assert torch.equal(y.view(torch.int16), resident[l].view(torch.int16)), l

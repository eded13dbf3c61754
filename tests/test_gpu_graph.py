"""The decode forward captured in a HIP graph (torch.cuda.CUDAGraph around the
library call): every replay must equal the eager call bit for bit, with eager
work and host synchronizations between the replays. The library enqueues only
kernels (no allocation, no memset, no host sync), so the call is capturable."""

import pytest
import torch

import bit_quantized_mixture_nf4_amd as e4b
from workloads import get_config
from gpu_util import DEV, Problem, announce

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T", [1, 8])
def test_decode_forward_graph_replays_equal_eager(T):
    cfg = get_config("tiny", T)
    announce(f"graph replay decode T={T}")
    pb = Problem(cfg, seed=21, with_grad=False)
    ws = torch.empty(e4b.workspace_bytes(pb.layer, T, cfg.k), dtype=torch.uint8, device=DEV)
    idx = torch.empty(T, cfg.k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, cfg.k, dtype=torch.float32, device=DEV)
    y = torch.empty(T, cfg.H, dtype=torch.bfloat16, device=DEV)
    x = pb.x_d.clone()
    lg = pb.logits_d.clone()

    def call():
        e4b.moe_forward(pb.layer, x, cfg.k, logits=lg, topk_idx=idx, topk_w=w, path="decode",
                        workspace=ws, out=y)

    call()
    torch.cuda.synchronize()
    y_eager, idx_eager = y.clone(), idx.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm the per-device occupancy cache outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        y.zero_()
        idx.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, idx_eager), rep
        assert torch.equal(y.view(torch.int16), y_eager.view(torch.int16)), rep
        call()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_eager.view(torch.int16)), rep

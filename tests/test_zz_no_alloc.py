"""The allocation-free forward (e4b_moe_forward_noalloc): its workspace is the
library's fixed per-GPU scratch array. Its outputs must equal, bit for bit,
those of e4b_moe_forward with a caller workspace, on two calls in a row (the
second with a smaller input), on the grouped and the decode paths; a size
beyond the array is refused."""

import ctypes

import pytest
import torch

import bit_quantized_mixture_nf4_amd as e4b
from bit_quantized_mixture_nf4_amd import _lib
from workloads import MoEConfig, get_config
from gpu_util import DEV, Problem, announce

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = _lib.NOALLOC_SCRATCH_BYTES


def _noalloc():
    return e4b.load().e4b_moe_forward_noalloc


def _vp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _run_noalloc(layer, x, k, logits, path):
    T = x.shape[0]
    idx = torch.full((T, k), -1, dtype=torch.int32, device=DEV)
    w = torch.zeros(T, k, dtype=torch.float32, device=DEV)
    y = torch.zeros(T, layer.H, dtype=torch.bfloat16, device=DEV)
    c = layer.as_c()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    code = _noalloc()(ctypes.byref(c), T, k, _vp(x), _vp(logits), _vp(idx), _vp(w), _vp(y), None,
                      e4b.PATHS[path], stream)
    assert code == 0, e4b._lib.status_string(code)
    return y, idx, w


@pytest.mark.parametrize("path,T1,T2", [("grouped", 300, 77), ("decode", 8, 3)])
def test_noalloc_forward_equals_forward(path, T1, T2):
    cfg = MoEConfig("na", E=16, H=512, I=256, k=4, T=T1, routing="normal")
    announce(f"noalloc forward {path} T={T1} then T={T2}")
    pb = Problem(cfg, seed=5, with_grad=False)
    for T in (T1, T2):
        x = pb.x_d[:T].contiguous()
        lg = pb.logits_d[:T].contiguous()
        assert e4b.workspace_bytes(pb.layer, T, cfg.k) <= SCRATCH_BYTES
        y, idx, w = _run_noalloc(pb.layer, x, cfg.k, lg, path)
        y_ref, idx_ref, w_ref, _ = e4b.moe_forward(pb.layer, x, cfg.k, logits=lg, path=path)
        torch.cuda.synchronize()
        assert torch.equal(idx, idx_ref), T
        assert torch.equal(w.view(torch.int32), w_ref.view(torch.int32)), T
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), T


def test_noalloc_refuses_a_workspace_beyond_the_scratch_array():
    cfg = get_config("olmoe")
    pb_layer = Problem(MoEConfig("na", E=cfg.E, H=cfg.H, I=64, k=cfg.k, T=8, routing="uniform"),
                       seed=0, with_grad=False).layer
    T = 4096
    assert e4b.workspace_bytes(pb_layer, T, cfg.k) > SCRATCH_BYTES
    x = torch.zeros(T, cfg.H, dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros(T, cfg.k, dtype=torch.int32, device=DEV)
    w = torch.zeros(T, cfg.k, dtype=torch.float32, device=DEV)
    y = torch.zeros(T, cfg.H, dtype=torch.bfloat16, device=DEV)
    c = pb_layer.as_c()
    code = _noalloc()(ctypes.byref(c), T, cfg.k, _vp(x), None, _vp(idx), _vp(w), _vp(y), None, 0,
                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert code == _lib.E4B_ERR_WORKSPACE

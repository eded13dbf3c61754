"""GPU parity at the workloads' full sizes, whole outputs, in the launch
configuration the benchmark times.

For each workload the oracle regenerates every expert's weights one expert
at a time, quantizes them (its own quantizer) and checks the stored bytes
(packed codes, absmax or E8M0 scales, bf16 bits) and the dequantized weight
(fp32 and bf16 views) against the GPU's bit for bit. It then runs its
forward and dgrad on that expert's routed pairs and accumulates them into the
whole y, grad_x and grad_topk_w, each compared with the GPU's whole tensor at
max|err| <= 1e-2 * max|oracle|. Properties that hold at any size (dgrad
with saved state == dgrad that recomputes it; the forward from given ids ==
the forward that routed them) are checked bitwise on the same outputs.
"""

import time

import numpy as np
import pytest
import torch

import oracle
import bit_quantized_mixture_nf4_amd as e4b
from workloads import get_config, gen_x, gen_grad_y, gen_logits, gen_expert_weight, gen_weights
from gpu_util import (DEV, announce, tol_check, to_np, bf16_tensor, oracle_store_expert, stack_bytes,
                      expert_view, routed_pairs)

pytestmark = pytest.mark.gpu


def _layer(cfg, seed, kind):
    stacks = []
    for which in ("gate_up", "down"):
        w = gen_weights(cfg, seed, which)
        wd = torch.from_numpy(w).to(DEV)
        del w
        stacks.append(e4b.quantize(wd, kind))
        del wd
    torch.cuda.empty_cache()
    return e4b.MoELayer(*stacks)


def _oracle_experts(cfg, seed, kind, layer, experts=None):
    """Yields (e, W_gu[e], W_dn[e]) as the oracle stores them (fp32 dequantized),
    after checking the GPU's stored bytes and dequantized weights of expert e
    against the oracle's bit for bit (every expert, or those in `experts`)."""
    host = {"gate_up": stack_bytes(layer.gate_up), "down": stack_bytes(layer.down)}
    t0 = time.time()
    for e in range(cfg.E):
        if experts is not None and e not in experts:
            continue
        if e % max(1, cfg.E // 8) == 0:
            announce(f"  oracle expert {e}/{cfg.E} ({time.time() - t0:.0f} s)")
        out = []
        for which, st in (("gate_up", layer.gate_up), ("down", layer.down)):
            w = gen_expert_weight(cfg, seed, which, e)
            codes, scales, deq = oracle_store_expert(w, kind)
            g_codes, g_scales = host[which]
            assert np.array_equal(g_codes[e], codes), f"{which}[{e}] stored bytes"
            if scales is not None:
                assert np.array_equal(g_scales[e], scales), f"{which}[{e}] scales"
            one = expert_view(st, e)
            d32 = e4b.dequantize(one, torch.float32)[0].cpu().numpy()
            assert np.array_equal(d32.view(np.uint32), deq.view(np.uint32)), f"{which}[{e}] dequant fp32"
            d16 = e4b.dequantize(one, torch.bfloat16)[0].view(torch.int16).cpu().numpy().view(np.uint16)
            assert np.array_equal(d16, oracle.bf16_rne_bits(deq)), f"{which}[{e}] dequant bf16"
            out.append(deq)
        yield e, out[0], out[1]


def _oracle_whole(cfg, seed, kind, layer, x, gy, idx, w, routed_only=False):
    """Whole y, grad_x [T, H] and grad_topk_w [T, k] from the oracle, run one expert at a time
    (with routed_only, the experts without tokens are skipped)."""
    T, H, k = cfg.T, cfg.H, cfg.k
    y = np.zeros((T, H))
    gx = np.zeros((T, H)) if gy is not None else None
    gw = np.zeros((T, k)) if gy is not None else None
    t0 = time.time()
    only = set(np.unique(idx).tolist()) if routed_only else None
    for e, wgu, wdn in _oracle_experts(cfg, seed, kind, layer, only):
        t, j = routed_pairs(idx, e)
        if t.size == 0:
            continue
        i1 = np.zeros((t.size, 1), np.int32)
        w1 = w[t, j][:, None]
        # one pair per row (k = 1): row i is w * o of pair i; summed per token in fp64
        np.add.at(y, t, oracle.moe_forward(x[t], i1, w1, wgu[None], wdn[None]))
        if gy is not None:
            gxe, gwe = oracle.moe_dgrad(x[t], i1, w1, wgu[None], wdn[None], gy[t])
            np.add.at(gx, t, gxe)
            gw[t, j] = gwe[:, 0]
    announce(f"oracle over {cfg.E} experts in {time.time() - t0:.1f} s")
    return y, gx, gw


@pytest.mark.parametrize("name,kind", [("olmoe", "nf4"), ("qwen3_prefill", "nf4"), ("mixtral", "nf4"),
                                       ("mixtral", "fp4"), ("olmoe", "bf16"), ("olmoe", "mxfp4"),
                                       ("olmoe", "int8"), ("olmoe", "fp8")])
def test_full_size_forward_dgrad_whole(name, kind):
    cfg = get_config(name)
    seed = 0
    announce(f"{name} {kind} full size E{cfg.E} H{cfg.H} I{cfg.I} k{cfg.k} T{cfg.T}: whole outputs")
    layer = _layer(cfg, seed, kind)
    x = gen_x(cfg, seed)
    gy = gen_grad_y(cfg, seed)
    lg = gen_logits(cfg, seed)
    x_d, gy_d = bf16_tensor(x), bf16_tensor(gy)
    ws = torch.empty(e4b.workspace_bytes(layer, cfg.T, cfg.k), dtype=torch.uint8, device=DEV)
    y, idx, w, saved = e4b.moe_forward(layer, x_d, cfg.k, logits=torch.from_numpy(lg).to(DEV),
                                       save=True, workspace=ws)
    y = y.clone()
    gx, gw = e4b.moe_dgrad(layer, idx, w, gy_d, saved=saved, workspace=ws)
    gx, gw = gx.clone(), gw.clone()
    gx2, gw2 = e4b.moe_dgrad(layer, idx, w, gy_d, x=x_d, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(gx.view(torch.int16), gx2.view(torch.int16))
    assert torch.equal(gw.view(torch.int32), gw2.view(torch.int32))
    y2, _, _, _ = e4b.moe_forward(layer, x_d, cfg.k, topk_idx=idx, topk_w=w, workspace=ws)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    del saved, ws, gx2, gw2, y2
    torch.cuda.empty_cache()

    idx_ref, w_ref = oracle.route(lg, cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    assert np.max(np.abs(w.cpu().numpy() - w_ref)) <= 1e-6
    y_ref, gx_ref, gw_ref = _oracle_whole(cfg, seed, kind, layer, x, gy, idx_ref, w_ref)
    tol_check(to_np(y), y_ref, f"{name} {kind} y")
    tol_check(to_np(gx), gx_ref, f"{name} {kind} grad_x")
    tol_check(to_np(gw), gw_ref, f"{name} {kind} grad_topk_w")
    del layer
    torch.cuda.empty_cache()


def test_mixtral_fidelity_ordering_from_gpu_outputs():
    """Storage fidelity on the Mixtral-shaped layer, measured on the GPU's own
    forward outputs: rel(y) = ||y_gpu - y|| / ||y|| against the oracle's fp64
    forward on the unquantized fp32 weights must order bf16 < nf4 < fp4 (the
    0.4.0 README support matrix ordering; its absolute values are not
    pinned). The same ordering holds for the weights themselves."""
    cfg = get_config("mixtral")
    seed = 0
    announce("mixtral fidelity: bf16 / nf4 / fp4 layers against the unquantized forward")
    x = gen_x(cfg, seed)
    lg = gen_logits(cfg, seed)
    idx, w = oracle.route(lg, cfg.k)
    t0 = time.time()
    y_exact = np.zeros((cfg.T, cfg.H))
    for e in range(cfg.E):
        t, j = routed_pairs(idx, e)
        wgu = gen_expert_weight(cfg, seed, "gate_up", e)[None]
        wdn = gen_expert_weight(cfg, seed, "down", e)[None]
        np.add.at(y_exact, t, oracle.moe_forward(x[t], np.zeros((t.size, 1), np.int32), w[t, j][:, None],
                                                 wgu, wdn))
    announce(f"unquantized oracle forward in {time.time() - t0:.1f} s")
    x_d, lg_d = bf16_tensor(x), torch.from_numpy(lg).to(DEV)
    rel = {}
    for kind in ("bf16", "nf4", "fp4"):
        layer = _layer(cfg, seed, kind)
        y, _, _, _ = e4b.moe_forward(layer, x_d, cfg.k, logits=lg_d, path="grouped")
        rel[kind] = oracle.rel_fro(y_exact, to_np(y).astype(np.float64))
        del layer, y
        torch.cuda.empty_cache()
    announce(f"rel(y): {rel}")
    assert rel["bf16"] < rel["nf4"] < rel["fp4"], rel
    # weights of one expert (the oracle's reconstruction errors, same ordering)
    rw = oracle.reconstruction_errors(gen_expert_weight(cfg, seed, "down", 0)[None])
    assert rw["bf16"] < rw["nf4"] < rw["fp4"], rw


@pytest.mark.parametrize("name,T", [("qwen3_decode", 1), ("qwen3_decode", 8), ("mixtral", 1), ("mixtral", 8)])
def test_decode_full_size(name, T):
    cfg = get_config(name, T)
    seed = 0
    announce(f"{name} decode full size E{cfg.E} H{cfg.H} I{cfg.I} k{cfg.k} T={T}")
    layer = _layer(cfg, seed, "nf4")
    x = gen_x(cfg, seed)
    lg = gen_logits(cfg, seed)
    y, idx, w, _ = e4b.moe_forward(layer, bf16_tensor(x), cfg.k, logits=torch.from_numpy(lg).to(DEV),
                                   path="decode")
    idx_ref, w_ref = oracle.route(lg, cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    assert np.max(np.abs(w.cpu().numpy() - w_ref)) <= 1e-6
    y_ref, _, _ = _oracle_whole(cfg, seed, "nf4", layer, x, None, idx_ref, w_ref, routed_only=True)
    tol_check(to_np(y), y_ref, f"decode T={T} y")
    yg, _, _, _ = e4b.moe_forward(layer, bf16_tensor(x), cfg.k, topk_idx=idx, topk_w=w, path="grouped")
    tol_check(to_np(yg), y_ref, f"grouped T={T} y")


def test_lora_full_size_olmoe_whole():
    """LoRA (r=8, alpha=16) on the OLMoE-shaped layer in the benchmark's
    launch configuration: whole y, grad_x, grad_topk_w and all four adapter
    gradients of every expert, the oracle run one expert at a time."""
    from workloads import gen_lora

    cfg = get_config("olmoe")
    seed, r, alpha = 0, 8, 16.0
    announce(f"olmoe lora full size E{cfg.E} H{cfg.H} I{cfg.I} k{cfg.k} T{cfg.T} r{r}: whole outputs")
    layer = _layer(cfg, seed, "nf4")
    host = gen_lora(cfg, seed, r)
    lo = e4b.Lora(*(torch.from_numpy(m).to(DEV) for m in host), alpha=alpha)
    x = gen_x(cfg, seed)
    gy = gen_grad_y(cfg, seed)
    lg = gen_logits(cfg, seed)
    x_d, gy_d = bf16_tensor(x), bf16_tensor(gy)
    ws = torch.empty(e4b.lora_workspace_bytes(layer, cfg.T, cfg.k), dtype=torch.uint8, device=DEV)
    y, idx, w, saved = e4b.moe_lora_forward(layer, lo, x_d, cfg.k, logits=torch.from_numpy(lg).to(DEV),
                                            save=True, workspace=ws)
    y = y.clone()
    gx, gw, grads = e4b.moe_lora_backward(layer, lo, idx, w, x_d, gy_d, saved=saved, workspace=ws)
    gx, gw, grads = gx.clone(), gw.clone(), tuple(g.clone() for g in grads)
    gx2, gw2, grads2 = e4b.moe_lora_backward(layer, lo, idx, w, x_d, gy_d, workspace=ws)
    torch.cuda.synchronize()
    for a, b in zip((gx, gw) + grads, (gx2, gw2) + grads2):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))

    idx_ref, w_ref = oracle.route(lg, cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    y_ref = np.zeros((cfg.T, cfg.H))
    gx_ref = np.zeros((cfg.T, cfg.H))
    gw_ref = np.zeros((cfg.T, cfg.k))
    dref = [np.zeros(m.shape) for m in host]
    for e, wgu, wdn in _oracle_experts(cfg, seed, "nf4", layer):
        t, j = routed_pairs(idx_ref, e)
        if t.size == 0:
            continue
        i1 = np.zeros((t.size, 1), np.int32)
        w1 = w_ref[t, j][:, None]
        ad = [m[e:e + 1] for m in host]
        np.add.at(y_ref, t, oracle.lora_forward(x[t], i1, w1, wgu[None], wdn[None], *ad, alpha))
        gxe, gwe, *de = oracle.lora_backward(x[t], i1, w1, wgu[None], wdn[None], *ad, alpha, gy[t])
        np.add.at(gx_ref, t, gxe)
        gw_ref[t, j] = gwe[:, 0]
        for acc, d in zip(dref, de):
            acc[e] = d[0]
    tol_check(to_np(y), y_ref, "olmoe lora y")
    tol_check(to_np(gx), gx_ref, "olmoe lora grad_x")
    tol_check(to_np(gw), gw_ref, "olmoe lora grad_topk_w")
    for name, got, want in zip(("dA_gu", "dB_gu", "dA_dn", "dB_dn"), grads, dref):
        tol_check(to_np(got), want, f"olmoe lora {name}")
    del layer, ws, saved
    torch.cuda.empty_cache()


def test_mx8_full_size_olmoe_whole():
    """The MX forward (MXFP8 activations on the block-scaled FP4 MFMA) on the
    OLMoE-shaped MXFP4 layer, in the benchmark's launch configuration: the
    whole output against the oracle's MX forward (run one expert at a time),
    against the exact-activation grouped forward (the activation rounding
    only), and bitwise run to run."""
    cfg = get_config("olmoe")
    seed = 0
    announce(f"olmoe mxfp4 full size, mx8 path E{cfg.E} H{cfg.H} I{cfg.I} k{cfg.k} T{cfg.T}: whole output")
    layer = _layer(cfg, seed, "mxfp4")
    x = gen_x(cfg, seed)
    lg = gen_logits(cfg, seed)
    x_d, lg_d = bf16_tensor(x), torch.from_numpy(lg).to(DEV)
    ws = torch.empty(e4b.workspace_bytes(layer, cfg.T, cfg.k), dtype=torch.uint8, device=DEV)
    y, idx, w, _ = e4b.moe_forward(layer, x_d, cfg.k, logits=lg_d, path="mx8", workspace=ws)
    y = y.clone()
    y2, _, _, _ = e4b.moe_forward(layer, x_d, cfg.k, logits=lg_d, path="mx8", workspace=ws)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    yg, _, _, _ = e4b.moe_forward(layer, x_d, cfg.k, logits=lg_d, path="grouped", workspace=ws)
    tol_check(to_np(y), to_np(yg).astype(np.float64), "olmoe mx8 vs grouped", rel=0.1)

    idx_ref, w_ref = oracle.route(lg, cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    y_ref = np.zeros((cfg.T, cfg.H))
    for e, wgu, wdn in _oracle_experts(cfg, seed, "mxfp4", layer):
        t, j = routed_pairs(idx_ref, e)
        if t.size:
            # x is bf16-valued as generated: the device converts the same values
            np.add.at(y_ref, t, oracle.mx8_forward(x[t], np.zeros((t.size, 1), np.int32),
                                                   w_ref[t, j][:, None], wgu[None], wdn[None]))
    tol_check(to_np(y), y_ref, "olmoe mx8 y")
    del layer, ws
    torch.cuda.empty_cache()

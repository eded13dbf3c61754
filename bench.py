#!/usr/bin/env python3
"""Benchmark of the fused 4-bit MoE expert MLP on one MI355X.

One step = the whole hot path on one batch: route + permute + grouped gate_up
GEMM (SiLU*up) + grouped down GEMM + gather-combine (forward, saving the
gate/up projections) followed by the frozen-base dgrad (down^T GEMM with the
SiLU-backward epilogue + gate_up^T GEMM + combines). Throughput = 12*P*H*I
algorithmic flops per step / wall time, inputs resident in HBM.

Headline (`value`): the Mixtral-8x7B-shaped layer (E=8, H=4096, I=14336,
top-2, T=8192, NF4, uniform router logits), the largest training
configuration. The same measurement runs on the Mixtral-shaped layer stored
in FP4, the Qwen3-30B-A3B-shaped prefill layer (E=128, H=2048, I=768, top-8,
T=16384, Zipf routing) and the OLMoE-1B-7B-shaped layer (E=64, H=2048,
I=1024, top-8, T=4096) under `workloads`. Each workload runs on seeds
{0, 1, 2}: per seed, W warmup steps and then exactly K timed steps bracketed
by device synchronizations; the reported step time is the median over the
seeds. Per-kernel durations come from HIP events that the library records at
the start and end of each kernel's dispatch on its launch stream
(`e4b_moe_forward_timed` / `e4b_moe_dgrad_timed`); the longest kernel gives
`roofline`.

Also measured: the decode dequant-GEMV path on the Qwen3-shaped layer at T=1
and T=8 (cold cache, 16 layer copies rotated; GB/s of the experts actually
touched over the GEMV kernels' dispatch durations), the same path with the
layers streamed from pinned host memory, the training step with per-expert
LoRA adapters and on the bf16 passthrough lane (OLMoE-shaped layer), the MX
forward of an MXFP4 copy of that layer, and the CPU oracle (numpy float64) on
a bounded sample of the headline workload.

Prints ONE JSON line. `--gpus N` with N > 1 exits: the library runs on one GPU.
"""

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
MFMA_FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 MFMA (the rate of an fp4 x fp8 product)
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E

# workload key -> (layer shape, storage codebook, what it is)
WORKLOADS = {
    "mixtral_nf4": ("mixtral", "nf4", "Mixtral-8x7B-shaped MoE layer, NF4, forward + frozen-base dgrad"),
    "mixtral_fp4": ("mixtral", "fp4", "Mixtral-8x7B-shaped MoE layer, FP4 (e2m1), forward + frozen-base dgrad"),
    "qwen3_prefill_nf4": ("qwen3_prefill", "nf4",
                          "Qwen3-30B-A3B-shaped prefill/training MoE layer (Zipf routing), NF4, "
                          "forward + frozen-base dgrad"),
    "olmoe_nf4": ("olmoe", "nf4", "OLMoE-1B-7B-shaped MoE layer, NF4, forward + frozen-base dgrad"),
}
HEADLINE = "mixtral_nf4"
GEMMS = ("gate_up_fwd", "down_fwd", "down_dgrad", "gate_up_dgrad")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class HipEvents:
    """HIP events through the runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(ev)) == 0
        return ev

    def elapsed_ms(self, start, stop):
        """Milliseconds between two recorded events; None if the pair was never recorded."""
        if self.hip.hipEventSynchronize(stop) != 0:
            return None
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), start, stop) != 0:
            return None
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(ev)


class KernelTimer:
    """One e4b_kernel_events set per step: every kernel of the call is
    bracketed by events taken at its dispatch's start and end."""

    def __init__(self, e4b, ev, names, n):
        self.e4b, self.ev, self.names, self.n = e4b, ev, list(names), n
        self.sets = []
        for _ in range(n):
            s = e4b.E4bKernelEvents()
            for name in self.names:
                kid = e4b._lib.KERNELS[name]
                s.start[kid] = self.ev.create()
                s.stop[kid] = self.ev.create()
            self.sets.append(s)

    def mean_ms(self):
        out = {}
        for name in self.names:
            kid = self.e4b._lib.KERNELS[name]
            ms = [self.ev.elapsed_ms(s.start[kid], s.stop[kid]) for s in self.sets]
            ms = [m for m in ms if m is not None]
            if ms:  # kernels this call does not launch are left out
                out[name] = sum(ms) / len(ms)
        return out

    def close(self):
        for s in self.sets:
            for name in self.names:
                kid = self.e4b._lib.KERNELS[name]
                self.ev.destroy(s.start[kid])
                self.ev.destroy(s.stop[kid])


def build_layer(e4b, torch, cfg, seed, kind="nf4", copies=1):
    from workloads import gen_weights

    stacks = []
    for which in ("gate_up", "down"):
        w = torch.from_numpy(gen_weights(cfg, seed, which)).to("cuda")
        stacks.append(e4b.quantize(w, kind))
        del w
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    layers = [e4b.MoELayer(*stacks)]
    for _ in range(copies - 1):
        gu, dn = stacks
        layers.append(e4b.MoELayer(
            e4b.QuantStack(gu.packed.clone(), gu.absmax.clone(), gu.E, gu.out, gu.inn, kind),
            e4b.QuantStack(dn.packed.clone(), dn.absmax.clone(), dn.E, dn.out, dn.inn, kind)))
    return layers


def vp(t):
    return ctypes.c_void_p(t.data_ptr())


def train_step_fn(e4b, torch, layer, x, lg, gy, k):
    """Raw-ABI closure of one forward (saving g|u) + dgrad with preallocated
    buffers; step(events) passes one e4b_kernel_events set (or None)."""
    lib = e4b.load()
    T = x.shape[0]
    dev = x.device
    idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    w = torch.empty(T, k, dtype=torch.float32, device=dev)
    y = torch.empty(T, layer.H, dtype=torch.bfloat16, device=dev)
    gx = torch.empty_like(y)
    gw = torch.empty(T, k, dtype=torch.float32, device=dev)
    # as the binding allocates it: uninitialised, the forward writes what the dgrad reads
    saved = torch.empty(e4b.saved_bytes(layer, T, k), dtype=torch.uint8, device=dev)
    ws = torch.empty(e4b.workspace_bytes(layer, T, k), dtype=torch.uint8, device=dev)
    L = layer.as_c()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    fwd_args = (ctypes.byref(L), T, k, vp(x), vp(lg), vp(idx), vp(w), vp(y), vp(saved), vp(ws),
                ws.numel(), 1, stream)
    bwd_args = (ctypes.byref(L), T, k, vp(idx), vp(w), vp(x), vp(saved), vp(gy), vp(gx), vp(gw),
                vp(ws), ws.numel(), stream)

    def step(events=None):
        ev = ctypes.byref(events) if events is not None else None
        s1 = lib.e4b_moe_forward_timed(*fwd_args, ev)
        s2 = lib.e4b_moe_dgrad_timed(*bwd_args, ev)
        if s1 or s2:
            raise RuntimeError(f"e4b status {s1} {s2}")

    keep = (idx, w, y, gx, gw, saved, ws, L)
    return step, keep


def timed_steps(torch, step, warmup, steps):
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def kernel_times(e4b, torch, ev, step, names, n):
    """Mean dispatch duration (ms) of each named kernel over n more steps."""
    kt = KernelTimer(e4b, ev, names, n)
    for i in range(n):
        step(kt.sets[i])
    torch.cuda.synchronize()
    out = kt.mean_ms()
    kt.close()
    return out


# Kernel sources whose text fixes the grouped GEMMs' memory traffic.
GEMM_SOURCES = ("gemm_wide.hip", "gemm_dev.h", "device.h", "kernels.h", "plan.h")


def gemm_source_digest():
    import hashlib

    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(ROOT, "bit_quantized_mixture_nf4_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the counter summary
    under profiles/ (FETCH_SIZE and WRITE_SIZE per dispatch from two
    rocprofv3 --pmc runs, each scaled by the same counter's reading for a
    plain copy of known size). The summary records the digest of the GEMM
    sources it was measured on; a stale or missing summary gives None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip()
    if fields.get("gemm_source_sha256") != gemm_source_digest():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def kernel_flops(cfg):
    P, H, I = cfg.P, cfg.H, cfg.I
    return {"gate_up_fwd": 4.0 * P * H * I, "down_fwd": 2.0 * P * H * I,
            "down_dgrad": 2.0 * P * H * I, "gate_up_dgrad": 4.0 * P * H * I}


def bench_workload(args, e4b, torch, ev, key):
    """Median over seeds of the training step on one workload."""
    from workloads import get_config, gen_x, gen_grad_y, gen_logits
    from workloads.gen import to_bf16_tensor

    name, kind, label = WORKLOADS[key]
    cfg = get_config(name)
    per_seed = []
    names = list(GEMMS) + ["route", "permute", "combine", "combine_dgrad"]
    for seed in args.seeds:
        log(f"{key}: building E={cfg.E} H={cfg.H} I={cfg.I} k={cfg.k} T={cfg.T} seed {seed}")
        layer = build_layer(e4b, torch, cfg, seed, kind)[0]
        x = to_bf16_tensor(gen_x(cfg, seed)).cuda()
        gy = to_bf16_tensor(gen_grad_y(cfg, seed)).cuda()
        lg = torch.from_numpy(gen_logits(cfg, seed)).cuda()
        step, keep = train_step_fn(e4b, torch, layer, x, lg, gy, cfg.k)
        dt = timed_steps(torch, step, args.warmup, args.steps)
        kms = kernel_times(e4b, torch, ev, step, names, args.steps)
        per_seed.append({"seed": seed, "ms_per_step": dt * 1e3, "kernels_ms": kms})
        log(f"{key} seed {seed}: step {dt * 1e3:.3f} ms -> {12.0 * cfg.P * cfg.H * cfg.I / dt / 1e12:.1f} "
            f"TFLOP/s; " + ", ".join(f"{n} {kms[n] * 1e3:.1f} us" for n in GEMMS))
        del keep, layer, x, gy, lg
        torch.cuda.empty_cache()
    med = statistics.median(r["ms_per_step"] for r in per_seed)
    kflops = kernel_flops(cfg)
    kmed = {n: statistics.median(r["kernels_ms"][n] for r in per_seed) for n in names}
    kernels = {n: {"ms": round(kmed[n], 4)} for n in names}
    for n in GEMMS:
        kernels[n]["tflops"] = round(kflops[n] / (kmed[n] * 1e-3) / 1e12, 1)
        kernels[n]["frac"] = round(kflops[n] / (kmed[n] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
    dom = max(GEMMS, key=lambda n: kmed[n])
    achieved = kflops[dom] / (kmed[dom] * 1e-3) / 1e12
    tflops = 12.0 * cfg.P * cfg.H * cfg.I / (med * 1e-3) / 1e12
    return {
        "config": {"workload": label, "E": cfg.E, "H": cfg.H, "I": cfg.I, "top_k": cfg.k,
                   "tokens": cfg.T, "routed_pairs": cfg.P, "codebook": kind, "router": cfg.routing,
                   "seeds": list(args.seeds)},
        "ms_per_step": round(med, 4),
        "tflops": round(tflops, 2),
        "frac_of_bf16_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "tokens_per_s": round(cfg.T / (med * 1e-3), 1),
        "per_seed_ms": [round(r["ms_per_step"], 4) for r in per_seed],
        "kernels": kernels,
        "roofline": {
            "bound": "mfma",
            "kernel": dom,
            "achieved": round(achieved, 1),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic(dom, key),
        },
    }


def olmoe_inputs(e4b, torch, seed=0):
    from workloads import get_config, gen_x, gen_grad_y, gen_logits
    from workloads.gen import to_bf16_tensor

    cfg = get_config("olmoe")
    x = to_bf16_tensor(gen_x(cfg, seed)).cuda()
    gy = to_bf16_tensor(gen_grad_y(cfg, seed)).cuda()
    lg = torch.from_numpy(gen_logits(cfg, seed)).cuda()
    return cfg, x, gy, lg


def bench_lora(args, e4b, torch, base_dt):
    """The OLMoE-shaped training step with per-expert LoRA adapters (r, alpha as on the pages)."""
    from workloads import gen_lora

    cfg, x, gy, lg = olmoe_inputs(e4b, torch)
    layer = build_layer(e4b, torch, cfg, 0, "nf4")[0]
    r, alpha = 8, 16.0
    lora = e4b.Lora(*(torch.from_numpy(m).cuda() for m in gen_lora(cfg, 0, r)), alpha=alpha)
    lib = e4b.load()
    T, k = cfg.T, cfg.k
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, dtype=torch.float32, device="cuda")
    y = torch.empty(T, cfg.H, dtype=torch.bfloat16, device="cuda")
    gx = torch.empty_like(y)
    gw = torch.empty(T, k, dtype=torch.float32, device="cuda")
    grads = [torch.empty_like(t) for t in (lora.A_gu, lora.B_gu, lora.A_dn, lora.B_dn)]
    saved = torch.empty(e4b.saved_bytes(layer, T, k), dtype=torch.uint8, device="cuda")
    ws = torch.empty(e4b.lora_workspace_bytes(layer, T, k), dtype=torch.uint8, device="cuda")
    L, LC = layer.as_c(), lora.as_c()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def step():
        s1 = lib.e4b_moe_lora_forward(ctypes.byref(L), ctypes.byref(LC), T, k, vp(x), vp(lg), vp(idx),
                                      vp(w), vp(y), vp(saved), vp(ws), ws.numel(), stream)
        s2 = lib.e4b_moe_lora_backward(ctypes.byref(L), ctypes.byref(LC), T, k, vp(idx), vp(w), vp(x),
                                       vp(saved), vp(gy), vp(gx), vp(gw), *(vp(g) for g in grads),
                                       vp(ws), ws.numel(), stream)
        if s1 or s2:
            raise RuntimeError(f"e4b status {s1} {s2}")

    dt = timed_steps(torch, step, args.warmup, args.steps)
    P, H, I = cfg.P, cfg.H, cfg.I
    # low-rank products: forward, dgrad slices, projections, adapter grads
    lora_flops = 2.0 * P * r * (H + 2 * I + I + H) * 3
    log(f"lora r={r}: step {dt * 1e3:.3f} ms ({dt / base_dt:.3f} x the frozen-base step)")
    del layer, lora, saved, ws
    torch.cuda.empty_cache()
    return {"workload": "olmoe_nf4", "r": r, "alpha": alpha, "ms_per_step": round(dt * 1e3, 4),
            "tflops_base_flops": round(12.0 * P * H * I / dt / 1e12, 1),
            "lora_flops_per_step": lora_flops, "vs_frozen_base_step": round(dt / base_dt, 4)}


def bench_lane(args, e4b, torch, base_dt, kind):
    """The OLMoE-shaped training step on another storage lane: bf16
    passthrough (weights stored bf16, no dequantization: the fidelity
    anchor), or the int8 / fp8 blockwise lanes (one code byte per weight,
    dequantized to bf16 in the workspace at each call, then the bf16-lane
    GEMMs)."""
    cfg, x, gy, lg = olmoe_inputs(e4b, torch)
    layer = build_layer(e4b, torch, cfg, 0, kind)[0]
    step, keep = train_step_fn(e4b, torch, layer, x, lg, gy, cfg.k)
    dt = timed_steps(torch, step, args.warmup, args.steps)
    tflops = 12.0 * cfg.P * cfg.H * cfg.I / dt / 1e12
    log(f"{kind} lane: step {dt * 1e3:.3f} ms -> {tflops:.1f} TFLOP/s ({base_dt / dt:.3f} x the nf4 "
        "step's speed)")
    del keep, layer
    torch.cuda.empty_cache()
    per_weight = {"bf16": 2.0, "int8": 1.0 + 4.0 / 64, "fp8": 1.0 + 4.0 / 64}[kind]
    return {"workload": f"olmoe_{kind}", "ms_per_step": round(dt * 1e3, 4), "tflops": round(tflops, 1),
            "weight_bytes": int(per_weight * cfg.E * 3 * cfg.H * cfg.I),
            f"nf4_step_over_{kind}_step": round(base_dt / dt, 4)}


def bench_mx8(args, e4b, torch, ev):
    """Forward only on an MXFP4 copy of the OLMoE-shaped layer: the MX path
    (activations as MXFP8 rows, both GEMMs on the block-scaled fp4 x fp8
    MFMA) against the grouped bf16 path on the same stored weights."""
    cfg, x, _, lg = olmoe_inputs(e4b, torch)
    layer = build_layer(e4b, torch, cfg, 0, "mxfp4")[0]
    lib = e4b.load()
    T, k = cfg.T, cfg.k
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, dtype=torch.float32, device="cuda")
    y = torch.empty(T, layer.H, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(e4b.workspace_bytes(layer, T, k), dtype=torch.uint8, device="cuda")
    L = layer.as_c()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P, H, I = cfg.P, cfg.H, cfg.I
    kflops = {"gate_up_fwd": 4.0 * P * H * I, "down_fwd": 2.0 * P * H * I}
    out = {}
    for name, path in (("mx8", e4b._lib.E4B_PATH_MX8), ("grouped", e4b._lib.E4B_PATH_GROUPED)):
        def step(events=None):
            s = lib.e4b_moe_forward_timed(ctypes.byref(L), T, k, vp(x), vp(lg), vp(idx), vp(w), vp(y),
                                          None, vp(ws), ws.numel(), path, stream,
                                          ctypes.byref(events) if events is not None else None)
            if s:
                raise RuntimeError(f"e4b status {s}")

        dt = timed_steps(torch, step, args.warmup, args.steps)
        kms = kernel_times(e4b, torch, ev, step, list(kflops), args.steps)
        out[name] = {
            "ms_per_forward": round(dt * 1e3, 4),
            "tflops": round(6.0 * P * H * I / dt / 1e12, 1),
            "kernels": {n: {"ms": round(kms[n], 4), "tflops": round(kflops[n] / (kms[n] * 1e-3) / 1e12, 1)}
                        for n in kflops},
        }
        log(f"mxfp4 layer, {name} forward: {dt * 1e3:.3f} ms -> {out[name]['tflops']} TFLOP/s "
            f"(gate_up {kms['gate_up_fwd']:.3f} ms, down {kms['down_fwd']:.3f} ms)")
    gu = out["mx8"]["kernels"]["gate_up_fwd"]["tflops"]
    out["workload"] = "olmoe_mxfp4"
    out["mx8"]["gate_up_fwd_frac_of_fp8_peak"] = round(gu / MFMA_FP8_PEAK_TFLOPS, 4)
    out["mx8_over_grouped_speed"] = round(out["grouped"]["ms_per_forward"] / out["mx8"]["ms_per_forward"], 4)
    del layer, ws
    torch.cuda.empty_cache()
    return out


def bench_decode(args, e4b, torch, ev):
    """Decode GEMV GB/s at T=1 and T=8 with 16 layer copies rotated (cold MALL/L2)."""
    import numpy as np
    from workloads import get_config, gen_x, gen_logits
    from workloads.gen import to_bf16_tensor

    copies = 16
    cfg0 = get_config("qwen3_decode")
    log(f"building {copies} copies of the qwen3 decode layer")
    layers = build_layer(e4b, torch, cfg0, 0, "nf4", copies=copies)
    lib = e4b.load()
    out = {}
    e_gu = 2 * cfg0.I * cfg0.H // 2 + 2 * cfg0.I * cfg0.H // 64 * 4  # packed + absmax per expert
    e_dn = cfg0.H * cfg0.I // 2 + cfg0.H * cfg0.I // 64 * 4
    names = ["decode_gate_up", "decode_down"]
    for T in (1, 8):
        cfg = get_config("qwen3_decode", T)
        x = to_bf16_tensor(gen_x(cfg, 0)).cuda()
        lg = torch.from_numpy(gen_logits(cfg, 0)).cuda()
        idx = torch.empty(T, cfg.k, dtype=torch.int32, device="cuda")
        w = torch.empty(T, cfg.k, dtype=torch.float32, device="cuda")
        y = torch.empty(T, cfg.H, dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(e4b.workspace_bytes(layers[0], T, cfg.k), dtype=torch.uint8, device="cuda")
        Ls = [l.as_c() for l in layers]
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        it = [0]

        def step(events=None, stream_c=stream, L=None):
            L = Ls[it[0] % copies] if L is None else L
            it[0] += 1
            s = lib.e4b_moe_forward_timed(ctypes.byref(L), T, cfg.k, vp(x), vp(lg), vp(idx), vp(w), vp(y),
                                          None, vp(ws), ws.numel(), e4b._lib.E4B_PATH_DECODE, stream_c,
                                          ctypes.byref(events) if events is not None else None)
            if s:
                raise RuntimeError(f"e4b status {s}")

        n = max(args.steps, 32)
        call_us = timed_steps(torch, step, args.warmup, n) * 1e6
        # the same calls captured in one HIP graph (one per layer copy) and replayed
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(stream_c=ctypes.c_void_p(side.cuda_stream))
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            sc = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for c in range(copies):
                step(stream_c=sc, L=Ls[c])
        graph.replay()
        torch.cuda.synchronize()
        reps = max(2, n // copies)
        t0 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        graph_us = (time.perf_counter() - t0) / (reps * copies) * 1e6
        del graph
        present = [nm for nm in names if nm in e4b._lib.KERNELS]
        kms = kernel_times(e4b, torch, ev, step, present, n)
        distinct = int(np.unique(idx.cpu().numpy()).size)
        b_gu = distinct * e_gu + T * cfg.H * 2 + T * cfg.k * cfg.I * 2
        b_dn = distinct * e_dn + T * cfg.k * cfg.I * 2 + T * cfg.H * 2
        us = (kms["decode_gate_up"] + kms["decode_down"]) * 1e3
        gbps = (b_gu + b_dn) / (us * 1e-6) / 1e9
        out[f"t{T}"] = {
            "distinct_experts": distinct,
            "bytes": b_gu + b_dn,
            "gemv_us": round(us, 2),
            "gbps": round(gbps, 1),
            "frac": round(gbps / HBM_PEAK_GBPS, 4),
            "timing": "kernel dispatch start/end events (hipExtLaunchKernelGGL)",
            "kernels_us": {nm: round(kms[nm] * 1e3, 2) for nm in present},
            "gate_up": {"us": round(kms["decode_gate_up"] * 1e3, 2),
                        "gbps": round(b_gu / (kms["decode_gate_up"] * 1e-3) / 1e9, 1)},
            "down": {"us": round(kms["decode_down"] * 1e3, 2),
                     "gbps": round(b_dn / (kms["decode_down"] * 1e-3) / 1e9, 1)},
            "forward_call_us": round(call_us, 2),
            "tokens_per_s": round(T / (call_us * 1e-6), 1),
            "graph_forward_call_us": round(graph_us, 2),
            "graph_tokens_per_s": round(T / (graph_us * 1e-6), 1),
            "cache": f"cold ({copies} layer copies rotated)",
        }
        log(f"decode T={T}: {distinct} experts, GEMV {us:.2f} us, {gbps:.0f} GB/s; forward call "
            f"{call_us:.1f} us eager, {graph_us:.1f} us from a HIP graph; kernels "
            + ", ".join(f"{nm} {kms[nm] * 1e3:.2f} us" for nm in present))
    if not args.no_stream:
        out["streamed"] = bench_decode_streamed(args, e4b, torch, layers[0])
    del layers
    torch.cuda.empty_cache()
    return out


def bench_decode_streamed(args, e4b, torch, layer, n_host=4, steps=8):
    """Decode with the layers kept in pinned host memory and streamed in with
    the layer-granular prefetch (two device slots, side-stream copies)."""
    from workloads import get_config, gen_x, gen_logits
    from workloads.gen import to_bf16_tensor

    host = []
    for _ in range(n_host):
        host.append(e4b.MoELayer(*[
            e4b.QuantStack(st.packed.cpu().pin_memory(), st.absmax.cpu().pin_memory(), st.E, st.out,
                           st.inn, st.codebook) for st in (layer.gate_up, layer.down)]))
    layer_bytes = sum(st.packed.numel() + st.absmax.numel() * 4 for st in (host[0].gate_up, host[0].down))
    pf = e4b.LayerPrefetcher(host)
    res = {"host_layers": n_host, "layer_bytes": layer_bytes}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        pf.prefetch(i % n_host)
        pf.acquire(i % n_host)
        pf.release(i % n_host)
    torch.cuda.synchronize()
    copy_s = (time.perf_counter() - t0) / steps
    res["h2d_gbps"] = round(layer_bytes / copy_s / 1e9, 1)
    for T in (1, 8):
        cfg = get_config("qwen3_decode", T)
        x = to_bf16_tensor(gen_x(cfg, 0)).cuda()
        lg = torch.from_numpy(gen_logits(cfg, 0)).cuda()

        def fwd(L):
            e4b.moe_forward(L, x, cfg.k, logits=lg, path="decode")

        for _ in range(2):
            fwd(layer)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fwd(layer)
        torch.cuda.synchronize()
        comp_s = (time.perf_counter() - t0) / steps
        t0 = time.perf_counter()
        pf.prefetch(0)
        for i in range(steps):
            if i + 1 < steps:
                pf.prefetch((i + 1) % n_host)
            L = pf.acquire(i % n_host)
            fwd(L)
            pf.release(i % n_host)
        torch.cuda.synchronize()
        step_s = (time.perf_counter() - t0) / steps
        res[f"t{T}"] = {"ms_per_layer": round(step_s * 1e3, 3), "copy_ms_per_layer": round(copy_s * 1e3, 3),
                        "compute_ms_per_layer": round(comp_s * 1e3, 4),
                        "tokens_per_s_per_layer": round(T / step_s, 1),
                        "overlap": round((copy_s + comp_s) / step_s, 3)}
        log(f"streamed decode T={T}: {step_s * 1e3:.2f} ms/layer (copy {copy_s * 1e3:.2f}, "
            f"compute {comp_s * 1e3:.3f}), H2D {res['h2d_gbps']} GB/s")
    del pf, host
    return res


def cpu_baseline(args, key):
    """The oracle (numpy fp64, as it stands) on the first S tokens of the headline workload."""
    from concurrent.futures import ThreadPoolExecutor
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info
    from workloads import get_config, gen_x, gen_grad_y, gen_logits, gen_expert_weight

    name, kind, _ = WORKLOADS[key]
    cfg = get_config(name)
    seed = args.seeds[0]
    S = min(args.cpu_tokens, cfg.T)
    x = gen_x(cfg, seed)[:S]
    gy = gen_grad_y(cfg, seed)[:S]
    idx, w = oracle.route(gen_logits(cfg, seed)[:S], cfg.k)
    experts = sorted(set(int(e) for e in idx.ravel()))
    log(f"cpu baseline: oracle weights for {len(experts)} experts")
    stacks = {}

    def prep(args_):
        which, e, r0, r1 = args_
        wt = gen_expert_weight(cfg, seed, which, e)[r0:r1]
        p, a = oracle.quantize_blockwise(wt[None], kind)
        return which, e, r0, oracle.dequantize(p, a, wt.shape[0], wt.shape[1], kind)[0]

    jobs = []
    for e in experts:
        for which, rows in (("gate_up", 2 * cfg.I), ("down", cfg.H)):
            stacks[(which, e)] = np.empty((rows, cfg.H if which == "gate_up" else cfg.I), np.float32)
            step = max(1, rows // 16)
            jobs += [(which, e, r0, min(rows, r0 + step)) for r0 in range(0, rows, step)]
    with ThreadPoolExecutor(max_workers=16) as ex:
        for which, e, r0, d in ex.map(prep, jobs):
            stacks[(which, e)][r0:r0 + d.shape[0]] = d
    remap = {e: i for i, e in enumerate(experts)}
    wgu = np.stack([stacks[("gate_up", e)] for e in experts])
    wdn = np.stack([stacks[("down", e)] for e in experts])
    del stacks
    idx_c = np.vectorize(remap.get)(idx).astype(np.int32)
    log(f"cpu baseline: oracle forward + dgrad on {S} tokens")
    reps, dt = 0, 0.0
    while reps < 8 and (reps == 0 or dt < args.cpu_min_seconds):
        t0 = time.perf_counter()
        oracle.moe_forward(x, idx_c, w, wgu, wdn)
        oracle.moe_dgrad(x, idx_c, w, wgu, wdn, gy)
        dt += time.perf_counter() - t0
        reps += 1
    flops = 12.0 * S * cfg.k * cfg.H * cfg.I * reps
    info = threadpool_info()
    blas = [d for d in info if d.get("user_api") == "blas"]
    threads = max([d.get("num_threads", 1) for d in blas] or [1])
    return {
        "value": round(flops / dt / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{key}: first {S} of {cfg.T} tokens ({S * cfg.k} routed pairs), seed {seed}, forward "
                  f"+ dgrad, {reps} pass(es) in {dt:.2f} s; weight generation/quantization excluded",
        "seconds": round(dt, 3),
        "host_cpu_count": os.cpu_count(),
        "blas": ", ".join(f"{d.get('internal_api')} {d.get('version')} ({d.get('num_threads')} threads)"
                          for d in blas),
    }


def host_info(torch):
    info = {"host_cpu_count": os.cpu_count(), "torch": torch.__version__, "torch_hip": torch.version.hip}
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        info["rocm"] = None
    try:
        info["gpu"] = torch.cuda.get_device_properties(0).gcnArchName
    except Exception:  # noqa: BLE001 - metadata only
        info["gpu"] = None
    return info


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workloads", default=",".join(WORKLOADS),
                    help="comma-separated subset of " + ", ".join(WORKLOADS) + "; the first is the headline")
    ap.add_argument("--seeds", default="0,1,2")
    ap.add_argument("--cpu-tokens", type=int, default=1024)
    ap.add_argument("--cpu-min-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="only run the decode measurement and print its JSON object")
    ap.add_argument("--no-lora", action="store_true")
    ap.add_argument("--no-bf16-lane", action="store_true")
    ap.add_argument("--no-8bit-lanes", action="store_true")
    ap.add_argument("--no-stream", action="store_true")
    ap.add_argument("--no-mx", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy 5 times (the reference "
                         "kernel for scaling FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "no multi-GPU path is built.", file=sys.stderr)
        sys.exit(2)
    args.seeds = [int(s) for s in args.seeds.split(",") if s != ""]
    keys = [k for k in args.workloads.split(",") if k]
    for k in keys:
        if k not in WORKLOADS:
            ap.error(f"unknown workload {k}")

    import torch
    import bit_quantized_mixture_nf4_amd as e4b

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5}), flush=True)
        return
    e4b.load()
    ev = HipEvents()
    if args.decode_only:
        print(json.dumps({"decode": bench_decode(args, e4b, torch, ev)}), flush=True)
        return
    results = {k: bench_workload(args, e4b, torch, ev, k) for k in keys}
    head = results[keys[0]]
    olmoe_ms = results["olmoe_nf4"]["ms_per_step"] * 1e-3 if "olmoe_nf4" in results else None
    lora = None if args.no_lora or olmoe_ms is None else bench_lora(args, e4b, torch, olmoe_ms)
    bf16 = None if args.no_bf16_lane or olmoe_ms is None else bench_lane(args, e4b, torch, olmoe_ms, "bf16")
    lanes8 = None if args.no_8bit_lanes or olmoe_ms is None else {
        kind: bench_lane(args, e4b, torch, olmoe_ms, kind) for kind in ("int8", "fp8")}
    mx = None if args.no_mx else bench_mx8(args, e4b, torch, ev)
    dec = None if args.no_decode else bench_decode(args, e4b, torch, ev)
    cpu = None if args.no_cpu_baseline else cpu_baseline(args, keys[0])
    line = {
        "metric": "grouped NF4 MoE fwd+dgrad TFLOP/s (% MFMA peak); decode GEMV HBM GB/s (% peak)",
        "value": head["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": dict(head["config"], key=keys[0]),
        "pct_mfma_peak": round(100 * head["tflops"] / MFMA_BF16_PEAK_TFLOPS, 2),
        "tokens_per_s": head["tokens_per_s"],
        "roofline": head["roofline"],
        "kernels": head["kernels"],
        "workloads": {k: v for k, v in results.items() if k != keys[0]},
        "decode": dec,
        "lora": lora,
        "bf16_lane": bf16,
        "lanes_8bit": lanes8,
        "mx8_forward": mx,
        "cpu_baseline": cpu,
        "host": host_info(torch),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

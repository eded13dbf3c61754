#!/usr/bin/env python3
"""Benchmark of the fused 4-bit MoE expert MLP on one MI355X.

One step = the whole hot path on one batch of the OLMoE-1B-7B-shaped layer
(E=64, H=2048, I=1024, top-8, T=4096, NF4, uniform router logits): route +
permute + grouped gate_up GEMM (SiLU*up) + grouped down GEMM + gather-combine
(forward, saving the gate/up projections) followed by the frozen-base dgrad
(permute + down^T GEMM with the SiLU-backward epilogue + gate_up^T GEMM +
combines). Throughput = 12*P*H*I algorithmic flops per step / wall time.

Also measured in the same run:
* per-kernel durations of the four grouped GEMMs with HIP events recorded on
  the launch stream (library timer hook), the largest gives `roofline`;
* the decode dequant-GEMV path on the Qwen3-30B-A3B-shaped layer (E=128,
  H=2048, I=768, top-8, Zipf routing) at T=1 and T=8, cold cache (16 layer
  copies rotated), as GB/s of the experts actually touched, and with the
  layers streamed from pinned host memory by the layer-granular prefetch;
* the same training step with per-expert LoRA adapters (r=8, alpha=16) over
  the frozen base (`lora`), and on the bf16 passthrough lane (`bf16_lane`);
* the CPU oracle (numpy float64) on a bounded sample of the same workload.

Prints ONE JSON line. `--gpus N` with N > 1 exits: the library runs on one GPU.
"""

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
MFMA_FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 MFMA (the rate of an fp4 x fp8 product)
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E


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

    def create(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(ev)) == 0
            arr[i] = ev
        return arr

    def elapsed_ms(self, start, stop):
        assert self.hip.hipEventSynchronize(stop) == 0
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), start, stop) == 0
        return ms.value

    def destroy(self, arr):
        for ev in arr:
            self.hip.hipEventDestroy(ev)


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


def train_step_fn(e4b, torch, layer, x, lg, gy, k):
    """Raw-ABI closures for one forward (saving g|u) + dgrad with preallocated buffers."""
    lib = e4b.load()
    T = x.shape[0]
    dev = x.device
    idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    w = torch.empty(T, k, dtype=torch.float32, device=dev)
    y = torch.empty(T, layer.H, dtype=torch.bfloat16, device=dev)
    gx = torch.empty_like(y)
    gw = torch.empty(T, k, dtype=torch.float32, device=dev)
    saved = torch.empty(e4b.saved_bytes(layer, T, k), dtype=torch.uint8, device=dev)
    ws = torch.empty(e4b.workspace_bytes(layer, T, k), dtype=torch.uint8, device=dev)
    L = layer.as_c()
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    fwd_args = (ctypes.byref(L), T, k, vp(x), vp(lg), vp(idx), vp(w), vp(y), vp(saved), vp(ws),
                ws.numel(), 1, stream)
    bwd_args = (ctypes.byref(L), T, k, vp(idx), vp(w), vp(x), vp(saved), vp(gy), vp(gx), vp(gw),
                vp(ws), ws.numel(), stream)

    def step():
        s1 = lib.e4b_moe_forward(*fwd_args)
        s2 = lib.e4b_moe_dgrad(*bwd_args)
        if s1 or s2:
            raise RuntimeError(f"e4b status {s1} {s2}")

    keep = (idx, w, y, gx, gw, saved, ws, L)
    return step, keep


def lora_step_fn(e4b, torch, layer, lora, x, lg, gy, k):
    """Raw-ABI closures for one LoRA forward (saving g|u) + backward with preallocated buffers."""
    lib = e4b.load()
    T = x.shape[0]
    dev = x.device
    idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    w = torch.empty(T, k, dtype=torch.float32, device=dev)
    y = torch.empty(T, layer.H, dtype=torch.bfloat16, device=dev)
    gx = torch.empty_like(y)
    gw = torch.empty(T, k, dtype=torch.float32, device=dev)
    grads = [torch.empty_like(t) for t in (lora.A_gu, lora.B_gu, lora.A_dn, lora.B_dn)]
    saved = torch.empty(e4b.saved_bytes(layer, T, k), dtype=torch.uint8, device=dev)
    ws = torch.empty(e4b.lora_workspace_bytes(layer, T, k), dtype=torch.uint8, device=dev)
    L, LC = layer.as_c(), lora.as_c()
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    fwd_args = (ctypes.byref(L), ctypes.byref(LC), T, k, vp(x), vp(lg), vp(idx), vp(w), vp(y),
                vp(saved), vp(ws), ws.numel(), stream)
    bwd_args = (ctypes.byref(L), ctypes.byref(LC), T, k, vp(idx), vp(w), vp(x), vp(saved), vp(gy),
                vp(gx), vp(gw), *(vp(g) for g in grads), vp(ws), ws.numel(), stream)

    def step():
        s1 = lib.e4b_moe_lora_forward(*fwd_args)
        s2 = lib.e4b_moe_lora_backward(*bwd_args)
        if s1 or s2:
            raise RuntimeError(f"e4b status {s1} {s2}")

    keep = (idx, w, y, gx, gw, grads, saved, ws, L, LC)
    return step, keep


def bench_lora(args, e4b, torch, cfg, layer, x, lg, gy, base_dt):
    """The same training step with per-expert LoRA adapters (r, alpha as on the pages)."""
    from workloads import gen_lora

    r, alpha = 8, 16.0
    lora = e4b.Lora(*(torch.from_numpy(m).cuda() for m in gen_lora(cfg, args.seed, r)), alpha=alpha)
    step, keep = lora_step_fn(e4b, torch, layer, lora, x, lg, gy, cfg.k)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    P, H, I = cfg.P, cfg.H, cfg.I
    # base GEMM flops plus the low-rank products (forward, dgrad slices, projections, adapter grads)
    lora_flops = 2.0 * P * r * (H + 2 * I + I + H) * 3
    log(f"lora r={r}: step {dt * 1e3:.3f} ms ({dt / base_dt:.3f} x the frozen-base step)")
    del keep
    return {
        "r": r, "alpha": alpha,
        "ms_per_step": round(dt * 1e3, 4),
        "tflops_base_flops": round(12.0 * P * H * I / dt / 1e12, 1),
        "lora_flops_per_step": lora_flops,
        "vs_frozen_base_step": round(dt / base_dt, 4),
    }


def bench_bf16_lane(args, e4b, torch, cfg, x, lg, gy, base_dt):
    """The same training step on the bf16 passthrough lane (weights stored bf16,
    no dequantization): the fidelity anchor, and the cost of the 4-bit decode."""
    layer = build_layer(e4b, torch, cfg, args.seed, "bf16")[0]
    step, keep = train_step_fn(e4b, torch, layer, x, lg, gy, cfg.k)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    tflops = 12.0 * cfg.P * cfg.H * cfg.I / dt / 1e12
    log(f"bf16 lane: step {dt * 1e3:.3f} ms -> {tflops:.1f} TFLOP/s ({base_dt / dt:.3f} x the "
        f"{args.codebook} step's speed)")
    del keep, layer
    torch.cuda.empty_cache()
    return {"ms_per_step": round(dt * 1e3, 4), "tflops": round(tflops, 1),
            "weight_bytes": 2 * cfg.E * 3 * cfg.H * cfg.I,
            "nf4_step_over_bf16_step": round(base_dt / dt, 4)}


def bench_mx8(args, e4b, torch, ev, cfg, x, lg):
    """Forward only on an MXFP4 copy of the layer: the MX path (activations
    converted to MXFP8 rows, both GEMMs on the block-scaled fp4 x fp8 MFMA)
    against the grouped bf16 path on the same stored weights."""
    layer = build_layer(e4b, torch, cfg, args.seed, "mxfp4")[0]
    lib = e4b.load()
    T, k = x.shape[0], cfg.k
    dev = x.device
    idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    w = torch.empty(T, k, dtype=torch.float32, device=dev)
    y = torch.empty(T, layer.H, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(e4b.workspace_bytes(layer, T, k), dtype=torch.uint8, device=dev)
    L = layer.as_c()
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P, H, I = cfg.P, cfg.H, cfg.I
    kflops = {"gate_up_fwd": 4.0 * P * H * I, "down_fwd": 2.0 * P * H * I}
    out = {}
    for name, path in (("mx8", e4b._lib.E4B_PATH_MX8), ("grouped", e4b._lib.E4B_PATH_GROUPED)):
        def step():
            s = lib.e4b_moe_forward(ctypes.byref(L), T, k, vp(x), vp(lg), vp(idx), vp(w), vp(y),
                                    None, vp(ws), ws.numel(), path, stream)
            if s:
                raise RuntimeError(f"e4b status {s}")

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        kms = time_kernels(e4b, torch, ev, step, list(kflops), args.steps)
        out[name] = {
            "ms_per_forward": round(dt * 1e3, 4),
            "tflops": round(6.0 * P * H * I / dt / 1e12, 1),
            "kernels": {n: {"ms": round(kms[n], 4),
                            "tflops": round(kflops[n] / (kms[n] * 1e-3) / 1e12, 1)}
                        for n in kflops},
        }
        log(f"mxfp4 layer, {name} forward: {dt * 1e3:.3f} ms -> {out[name]['tflops']} TFLOP/s "
            f"(gate_up {kms['gate_up_fwd']:.3f} ms, down {kms['down_fwd']:.3f} ms)")
    gu = out["mx8"]["kernels"]["gate_up_fwd"]["tflops"]
    out["mx8"]["gate_up_fwd_frac_of_fp8_peak"] = round(gu / MFMA_FP8_PEAK_TFLOPS, 4)
    out["mx8_over_grouped_speed"] = round(out["grouped"]["ms_per_forward"]
                                          / out["mx8"]["ms_per_forward"], 4)
    del layer, ws
    torch.cuda.empty_cache()
    return out


def time_kernels(e4b, torch, ev, step, names, n):
    """Average duration (ms) of each named kernel over n steps, events on its launch stream."""
    lib = e4b.load()
    out = {}
    for name in names:
        kid = e4b._lib.KERNELS[name]
        start, stop = ev.create(n), ev.create(n)
        assert lib.e4b_set_kernel_timer(kid, start, stop, n) == 0
        for _ in range(n):
            step()
        torch.cuda.synchronize()
        assert lib.e4b_set_kernel_timer(kid, None, None, 0) == 0
        ms = [ev.elapsed_ms(start[i], stop[i]) for i in range(n)]
        ev.destroy(start)
        ev.destroy(stop)
        out[name] = sum(ms) / n
    return out


# Kernel sources whose text fixes the grouped GEMMs' memory traffic.
GEMM_SOURCES = ("gemm.hip", "device.h", "kernels.h", "plan.h")


def gemm_source_digest():
    import hashlib

    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(ROOT, "bit_quantized_mixture_nf4_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the counter summary under profiles/.

    The summary (FETCH_SIZE and WRITE_SIZE per dispatch from two rocprofv3
    --pmc runs, each scaled by the same counter's reading for a plain copy of
    known size) records the digest of the GEMM sources it was measured on; a
    stale summary gives None.
    """
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


def bench_train(args, e4b, torch, ev):
    from workloads import get_config, gen_x, gen_grad_y, gen_logits
    from workloads.gen import to_bf16_tensor

    cfg = get_config(args.config)
    log(f"building {cfg.name} layer E={cfg.E} H={cfg.H} I={cfg.I} k={cfg.k} T={cfg.T}")
    layer = build_layer(e4b, torch, cfg, args.seed, args.codebook)[0]
    x = to_bf16_tensor(gen_x(cfg, args.seed)).cuda()
    gy = to_bf16_tensor(gen_grad_y(cfg, args.seed)).cuda()
    lg = torch.from_numpy(gen_logits(cfg, args.seed)).cuda()
    step, keep = train_step_fn(e4b, torch, layer, x, lg, gy, cfg.k)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    P, H, I = cfg.P, cfg.H, cfg.I
    flops = 12.0 * P * H * I
    tflops = flops / dt / 1e12
    log(f"step {dt * 1e3:.3f} ms -> {tflops:.1f} TFLOP/s")

    names = ["gate_up_fwd", "down_fwd", "down_dgrad", "gate_up_dgrad"]
    kms = time_kernels(e4b, torch, ev, step, names, args.steps)
    kflops = {"gate_up_fwd": 4.0 * P * H * I, "down_fwd": 2.0 * P * H * I,
              "down_dgrad": 2.0 * P * H * I, "gate_up_dgrad": 4.0 * P * H * I}
    kernels = {
        n: {"ms": round(kms[n], 4), "tflops": round(kflops[n] / (kms[n] * 1e-3) / 1e12, 1)}
        for n in names
    }
    dom = max(names, key=lambda n: kms[n])
    achieved = kflops[dom] / (kms[dom] * 1e-3) / 1e12
    roofline = {
        "bound": "mfma",
        "kernel": dom,
        "achieved": round(achieved, 1),
        "peak": MFMA_BF16_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
        "traffic": measured_traffic(dom, "olmoe"),
    }
    res = dict(cfg=cfg, dt=dt, tflops=tflops, kernels=kernels, roofline=roofline, x=x, lg=lg)
    res["lora"] = None if args.no_lora else bench_lora(args, e4b, torch, cfg, layer, x, lg, gy, dt)
    del keep, layer
    torch.cuda.empty_cache()
    res["bf16_lane"] = None if args.no_bf16_lane else bench_bf16_lane(args, e4b, torch, cfg, x, lg,
                                                                      gy, dt)
    torch.cuda.empty_cache()
    return res


def bench_decode(args, e4b, torch, ev):
    """Decode GEMV GB/s at T=1 and T=8 with 16 layer copies rotated (cold MALL/L2)."""
    import numpy as np
    from workloads import get_config, gen_x, gen_logits
    from workloads.gen import to_bf16_tensor

    copies = 16
    cfg0 = get_config("qwen3_decode")
    log(f"building {copies} copies of the qwen3 decode layer")
    layers = build_layer(e4b, torch, cfg0, args.seed, "nf4", copies=copies)
    lib = e4b.load()
    out = {}
    e_gu = 2 * cfg0.I * cfg0.H // 2 + 2 * cfg0.I * cfg0.H // 64 * 4  # packed + absmax per expert
    e_dn = cfg0.H * cfg0.I // 2 + cfg0.H * cfg0.I // 64 * 4
    for T in (1, 8):
        cfg = get_config("qwen3_decode", T)
        x = to_bf16_tensor(gen_x(cfg, args.seed)).cuda()
        lg = torch.from_numpy(gen_logits(cfg, args.seed)).cuda()
        idx = torch.empty(T, cfg.k, dtype=torch.int32, device="cuda")
        w = torch.empty(T, cfg.k, dtype=torch.float32, device="cuda")
        y = torch.empty(T, cfg.H, dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(e4b.workspace_bytes(layers[0], T, cfg.k), dtype=torch.uint8, device="cuda")
        Ls = [l.as_c() for l in layers]
        vp = lambda t: ctypes.c_void_p(t.data_ptr())
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        it = [0]

        def step():
            L = Ls[it[0] % copies]
            it[0] += 1
            s = lib.e4b_moe_forward(ctypes.byref(L), T, cfg.k, vp(x), vp(lg), vp(idx), vp(w), vp(y),
                                    None, vp(ws), ws.numel(), 2, stream)
            if s:
                raise RuntimeError(f"e4b status {s}")

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        n = max(args.steps, 32)
        t0 = time.perf_counter()
        for _ in range(n):
            step()
        torch.cuda.synchronize()
        call_us = (time.perf_counter() - t0) / n * 1e6
        # the same calls captured in one HIP graph (one per layer copy) and replayed
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            stream_c = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for c in range(copies):
                s_ = lib.e4b_moe_forward(ctypes.byref(Ls[c]), T, cfg.k, vp(x), vp(lg), vp(idx),
                                         vp(w), vp(y), None, vp(ws), ws.numel(), 2, stream_c)
                if s_:
                    raise RuntimeError(f"e4b status {s_}")
        graph.replay()
        torch.cuda.synchronize()
        reps = max(2, n // copies)
        t0 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        graph_us = (time.perf_counter() - t0) / (reps * copies) * 1e6
        del graph
        kms = time_kernels(e4b, torch, ev, step, ["decode_gate_up", "decode_down"], n)
        distinct = int(np.unique(idx.cpu().numpy()).size)
        b_gu = distinct * e_gu + T * cfg.H * 2 + T * cfg.k * cfg.I * 2
        b_dn = distinct * e_dn + T * cfg.k * cfg.I * 2 + T * cfg.k * cfg.H * 2
        us = (kms["decode_gate_up"] + kms["decode_down"]) * 1e3
        gbps = (b_gu + b_dn) / (us * 1e-6) / 1e9
        out[f"t{T}"] = {
            "distinct_experts": distinct,
            "bytes": b_gu + b_dn,
            "gemv_us": round(us, 2),
            "gbps": round(gbps, 1),
            "frac": round(gbps / HBM_PEAK_GBPS, 4),
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
            f"{call_us:.1f} us eager, {graph_us:.1f} us from a HIP graph")
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
    layer_bytes = sum(st.packed.numel() + st.absmax.numel() * 4
                      for st in (host[0].gate_up, host[0].down))
    pf = e4b.LayerPrefetcher(host)
    res = {"host_layers": n_host, "layer_bytes": layer_bytes}
    # copies alone (no compute)
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
        x = to_bf16_tensor(gen_x(cfg, args.seed)).cuda()
        lg = torch.from_numpy(gen_logits(cfg, args.seed)).cuda()

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
        res[f"t{T}"] = {"ms_per_layer": round(step_s * 1e3, 3),
                        "copy_ms_per_layer": round(copy_s * 1e3, 3),
                        "compute_ms_per_layer": round(comp_s * 1e3, 4),
                        "tokens_per_s_per_layer": round(T / step_s, 1),
                        "overlap": round((copy_s + comp_s) / step_s, 3)}
        log(f"streamed decode T={T}: {step_s * 1e3:.2f} ms/layer (copy {copy_s * 1e3:.2f}, "
            f"compute {comp_s * 1e3:.3f}), H2D {res['h2d_gbps']} GB/s")
    del pf, host
    return res


def cpu_baseline(args, cfg):
    """The oracle (numpy fp64) on the first S tokens of the same workload."""
    from concurrent.futures import ThreadPoolExecutor
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info
    from workloads import gen_x, gen_grad_y, gen_logits, gen_expert_weight

    S = args.cpu_tokens
    x = gen_x(cfg, args.seed)[:S]
    gy = gen_grad_y(cfg, args.seed)[:S]
    idx, w = oracle.route(gen_logits(cfg, args.seed)[:S], cfg.k)
    experts = sorted(set(int(e) for e in idx.ravel()))
    log(f"cpu baseline: oracle weights for {len(experts)} experts")
    stacks = {}

    def prep(args_):
        which, e = args_
        wt = gen_expert_weight(cfg, args.seed, which, e)
        p, a = oracle.quantize_blockwise(wt[None], args.codebook)
        return which, e, oracle.dequantize(p, a, wt.shape[0], wt.shape[1], args.codebook)[0]

    with ThreadPoolExecutor(max_workers=16) as ex:
        for which, e, d in ex.map(prep, [(wh, e) for e in experts for wh in ("gate_up", "down")]):
            stacks[(which, e)] = d
    remap = {e: i for i, e in enumerate(experts)}
    wgu = np.stack([stacks[("gate_up", e)] for e in experts])
    wdn = np.stack([stacks[("down", e)] for e in experts])
    del stacks
    idx_c = np.vectorize(remap.get)(idx).astype(np.int32)
    # forward + dgrad on the sample, repeated until at least min_seconds of
    # timed work (at most 8 passes)
    log(f"cpu baseline: oracle forward + dgrad on {S} tokens")
    reps, dt = 0, 0.0
    while reps < 8 and (reps == 0 or dt < args.cpu_min_seconds):
        t0 = time.perf_counter()
        oracle.moe_forward(x, idx_c, w, wgu, wdn)
        oracle.moe_dgrad(x, idx_c, w, wgu, wdn, gy)
        dt += time.perf_counter() - t0
        reps += 1
    flops = 12.0 * S * cfg.k * cfg.H * cfg.I * reps
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    return {
        "value": round(flops / dt / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {S} of {cfg.T} tokens ({S * cfg.k} routed pairs), forward + dgrad, "
                  f"{reps} pass(es) in {dt:.2f} s; weight generation/quantization excluded",
        "seconds": round(dt, 3),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="olmoe")
    ap.add_argument("--codebook", default="nf4")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-tokens", type=int, default=4096)
    ap.add_argument("--cpu-min-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-lora", action="store_true")
    ap.add_argument("--no-bf16-lane", action="store_true")
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
    tr = bench_train(args, e4b, torch, ev)
    mx = None if args.no_mx else bench_mx8(args, e4b, torch, ev, tr["cfg"], tr["x"], tr["lg"])
    dec = None if args.no_decode else bench_decode(args, e4b, torch, ev)
    cfg = tr["cfg"]
    cpu = None if args.no_cpu_baseline else cpu_baseline(args, cfg)
    line = {
        "metric": "grouped NF4 MoE fwd+dgrad TFLOP/s (% MFMA peak); decode GEMV HBM GB/s (% peak)",
        "value": round(tr["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(tr["dt"] * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "OLMoE-1B-7B-shaped MoE layer, forward + frozen-base dgrad",
            "E": cfg.E, "H": cfg.H, "I": cfg.I, "top_k": cfg.k, "tokens": cfg.T,
            "routed_pairs": cfg.P, "codebook": args.codebook, "router": cfg.routing,
            "seed": args.seed,
        },
        "pct_mfma_peak": round(100 * tr["tflops"] / MFMA_BF16_PEAK_TFLOPS, 2),
        "tokens_per_s": round(cfg.T / tr["dt"], 1),
        "roofline": tr["roofline"],
        "kernels": tr["kernels"],
        "decode": dec,
        "lora": tr["lora"],
        "bf16_lane": tr["bf16_lane"],
        "mx8_forward": mx,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

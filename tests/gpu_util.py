"""Helpers shared by the GPU parity tests (not collected by pytest)."""

import numpy as np
import torch

import oracle
import bit_quantized_mixture_nf4_amd as e4b
from workloads import gen_x, gen_grad_y, gen_logits, gen_weights

DEV = "cuda:0"


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)


def tol_check(got, ref, name, rel=1e-2):
    """max |got - ref| <= rel * max |ref| for one output tensor."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    assert np.all(np.isfinite(got)), name
    assert err <= rel * scale, f"{name}: max err {err:.3e} > {rel} * {scale:.3e}"
    return err, scale


def bf16_tensor(a_f32):
    return torch.from_numpy(np.ascontiguousarray(a_f32, np.float32)).to(torch.bfloat16).to(DEV)


def to_np(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


class Problem:
    """A synthetic layer + batch from the workload recipe, on the GPU and for the oracle."""

    def __init__(self, cfg, seed=0, codebook="nf4", with_grad=True):
        self.cfg, self.seed, self.codebook = cfg, seed, codebook
        self.x = gen_x(cfg, seed)
        self.logits = gen_logits(cfg, seed)
        self.grad_y = gen_grad_y(cfg, seed) if with_grad else None
        self.w_gu = gen_weights(cfg, seed, "gate_up")
        self.w_dn = gen_weights(cfg, seed, "down")
        gu = e4b.quantize(torch.from_numpy(self.w_gu).to(DEV), codebook)
        dn = e4b.quantize(torch.from_numpy(self.w_dn).to(DEV), codebook)
        self.layer = e4b.MoELayer(gu, dn)
        self.x_d = bf16_tensor(self.x)
        self.logits_d = torch.from_numpy(self.logits).to(DEV)
        self.grad_y_d = bf16_tensor(self.grad_y) if with_grad else None
        self._deq = None

    def oracle_weights(self, experts=None):
        """fp32 stored stacks from the oracle's own quantization (or bf16 rounding)."""
        if self._deq is None:
            self._deq = (
                oracle.stored_weights(self.w_gu, self.codebook),
                oracle.stored_weights(self.w_dn, self.codebook),
            )
        return self._deq


def oracle_expert_stacks(cfg, seed, experts, kind="nf4", threads=16):
    """Oracle-dequantized fp32 weights of only ``experts`` (regenerated per expert).

    Quantization runs on row slices in parallel threads; blocks never straddle a
    row, so quantizing row slices gives exactly the whole-stack result.
    """
    from concurrent.futures import ThreadPoolExecutor
    from workloads import gen_expert_weight

    out = {"gate_up": {}, "down": {}}
    jobs = []
    for e in experts:
        for which in ("gate_up", "down"):
            w = gen_expert_weight(cfg, seed, which, e)
            out[which][e] = np.empty_like(w)
            rows = w.shape[0]
            step = max(1, -(-rows // 64))
            for r0 in range(0, rows, step):
                jobs.append((w, out[which][e], r0, min(rows, r0 + step)))

    def one(job):
        w, dst, r0, r1 = job
        dst[r0:r1] = oracle.stored_weights(w[None, r0:r1], kind)[0]

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(one, jobs))
    return out


def oracle_store_expert(w, kind, threads=16):
    """The oracle's stored form of one expert's fp32 weight ``[out, in]``.

    Quantized on row slices in parallel threads (a block never straddles a
    row, so row slices give exactly the whole-expert result). Returns
    ``(stored bytes uint8 [nbytes], scale bytes uint8 [n] or None, dequantized
    fp32 [out, in])``: nf4 / fp4 -> packed codes and the absmax as its fp32
    bytes; int8 / fp8 -> one code byte per element and the absmax bytes;
    mxfp4 -> packed codes and the E8M0 bytes; bf16 -> the bf16 bit patterns as
    bytes and no scales.
    """
    from concurrent.futures import ThreadPoolExecutor

    rows, inn = w.shape
    step = max(1, -(-rows // (4 * threads)))
    slices = [(r0, min(rows, r0 + step)) for r0 in range(0, rows, step)]

    def one(sl):
        r0, r1 = sl
        ws = w[None, r0:r1]
        if kind == "bf16":
            bits = oracle.bf16_rne_bits(ws[0])
            return bits.view(np.uint8).reshape(-1), None, oracle.bf16_bits_to_f32(bits)
        if kind == "mxfp4":
            p, s = oracle.quantize_mx(ws)
            return p[0], s[0], oracle.dequantize_mx(p, s, r1 - r0, inn)[0]
        if kind in ("int8", "fp8"):
            from oracle import quant8

            c, a = quant8.quantize_blockwise8(ws, kind)
            return c[0], a[0].view(np.uint8), quant8.dequantize8(c, a, r1 - r0, inn, kind)[0]
        p, a = oracle.quantize_blockwise(ws, kind)
        return p[0], a[0].view(np.uint8), oracle.dequantize(p, a, r1 - r0, inn, kind)[0]

    with ThreadPoolExecutor(max_workers=threads) as ex:
        parts = list(ex.map(one, slices))
    codes = np.concatenate([p[0] for p in parts])
    scales = None if parts[0][1] is None else np.concatenate([p[1] for p in parts])
    deq = np.concatenate([p[2] for p in parts], axis=0)
    return codes, scales, deq


def stack_bytes(stack):
    """Host copies of a device stack as bytes per expert: (codes [E, n], scales [E, m] or None)."""
    codes = stack.packed.cpu().numpy()
    sc = stack.scales if stack.codebook == "mxfp4" else stack.absmax
    scales = None if sc is None else sc.cpu().numpy().view(np.uint8).reshape(stack.E, -1)
    return codes, scales


def expert_view(stack, e):
    """A one-expert QuantStack aliasing expert e of a device stack."""
    sl = slice(e, e + 1)
    return e4b.QuantStack(stack.packed[sl], None if stack.absmax is None else stack.absmax[sl], 1,
                          stack.out, stack.inn, stack.codebook,
                          None if stack.scales is None else stack.scales[sl])


def routed_pairs(idx, e):
    """(tokens, slots) of the pairs routed to expert e, in token order."""
    return np.nonzero(np.asarray(idx) == e)

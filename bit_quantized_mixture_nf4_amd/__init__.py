"""MI355X-native fused blockwise-4-bit (NF4 / FP4 / MXFP4) Mixture-of-Experts expert MLP.

Thin Python binding over ``libe4b.so`` (C ABI in ``include/e4b.h``). PyTorch is
used only for device memory and the current HIP stream: every computation runs
in the library's HIP kernels. The raw entry points are the ctypes functions of
``load()`` under their C names (``e4b_quantize_nf4``, ``e4b_dequantize_nf4``,
``e4b_moe_forward``, ``e4b_moe_dgrad``, ...); the functions below check torch
tensors (dtype, device, shape, contiguity, buffer sizes) and marshal them into
those entry points.

Layout (the fused-expert storage of the experts4bit-qlora 0.1.0 sdist,
``Experts4bit``): gate_up ``[E, 2I, H]`` (gate rows first), down
``[E, H, I]``; packed uint8 ``[E, out*in/2]`` (even element in the high
nibble) and fp32 absmax ``[E, out*in/64]`` (MXFP4: E8M0 scale bytes
``[E, out*in/32]``).
"""

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import (  # noqa: F401
    E4bError,
    E4bKernelEvents,
    E4bLayer,
    E4bLora,
    E4bPermLayout,
    E4bStack,
    check,
    load,
)

CODEBOOKS = {"nf4": _lib.E4B_CB_NF4, "fp4": _lib.E4B_CB_FP4, "bf16": _lib.E4B_CB_BF16,
             "mxfp4": _lib.E4B_CB_MXFP4, "int8": _lib.E4B_CB_INT8, "fp8": _lib.E4B_CB_FP8}
PATHS = {"auto": _lib.E4B_PATH_AUTO, "grouped": _lib.E4B_PATH_GROUPED, "decode": _lib.E4B_PATH_DECODE,
         "mx8": _lib.E4B_PATH_MX8}

__all__ = [
    "QuantStack",
    "MoELayer",
    "quantize",
    "dequantize",
    "mx8_rows",
    "moe_forward",
    "moe_dgrad",
    "Lora",
    "moe_lora_forward",
    "moe_lora_backward",
    "lora_workspace_bytes",
    "LayerPrefetcher",
    "workspace_bytes",
    "saved_bytes",
    "perm_layout",
    "check_expert_ids",
    "E4bError",
]


def _vp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t, name, dtype, device=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _need_buffer(t, name, nbytes, device):
    """A contiguous device byte buffer of at least ``nbytes`` bytes."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name} holds {have} bytes, the call needs {nbytes}")


def check_expert_ids(topk_idx, E):
    """Raise ValueError unless every id of ``topk_idx`` lies in [0, E).

    The kernels never index out of bounds with a bad id (they read it as
    expert 0), but the result is then meaningless; this check costs one
    device-to-host synchronization, so the calls below run it only when asked
    (``check_ids=True``).
    """
    if topk_idx.numel() and bool(((topk_idx < 0) | (topk_idx >= E)).any()):
        raise ValueError(f"topk_idx holds an expert id outside [0, {E})")


@dataclass
class QuantStack:
    """One stored fused stack of an [E, out, in] weight: packed 4-bit codes +
    fp32 absmax, packed E2M1 codes + E8M0 scales (codebook "mxfp4"), one code
    byte per element + fp32 absmax (codebooks "int8", "fp8"), or (codebook
    "bf16", the passthrough lane) the bf16 weight as bytes."""

    packed: torch.Tensor  # uint8 [E, out*in/2]; int8/fp8: [E, out*in]; bf16 lane: [E, out*in*2]
    absmax: torch.Tensor  # float32 [E, out*in/64]; bf16 / mxfp4: None
    E: int
    out: int
    inn: int
    codebook: str = "nf4"
    scales: torch.Tensor = None  # mxfp4: uint8 [E, out*in/32]

    def as_c(self):
        return E4bStack(
            self.packed.data_ptr(), None if self.absmax is None else self.absmax.data_ptr(),
            self.E, self.out, self.inn, 32 if self.codebook == "mxfp4" else 64,
            CODEBOOKS[self.codebook], None if self.scales is None else self.scales.data_ptr(),
        )

    @property
    def device(self):
        return self.packed.device


@dataclass
class MoELayer:
    """gate_up (out = 2I, in = H) and down (out = H, in = I) of one MoE layer."""

    gate_up: QuantStack
    down: QuantStack

    def as_c(self):
        return E4bLayer(self.gate_up.as_c(), self.down.as_c())

    @property
    def E(self):
        return self.gate_up.E

    @property
    def H(self):
        return self.gate_up.inn

    @property
    def I(self):  # noqa: E743
        return self.down.inn

    @property
    def device(self):
        return self.gate_up.device


def quantize(w, codebook="nf4"):
    """Blockwise (64) absmax quantization of a float32 [E, out, in] device stack: 4-bit
    (codebook "nf4" / "fp4") or 8-bit (codebook "int8": the dynamic tree map; "fp8": an
    E4M3 codebook), its MXFP4 conversion (codebook "mxfp4": E2M1 codes and an E8M0
    scale per 32 elements), or its bf16 passthrough storage (codebook "bf16")."""
    if w.dim() != 3:
        raise ValueError("w must be [E, out, in]")
    _need(w, "w", torch.float32)
    E, out, inn = w.shape
    if codebook not in CODEBOOKS:
        raise ValueError(f"codebook must be one of {sorted(CODEBOOKS)}")
    if codebook == "mxfp4":
        packed = torch.empty(E, out * inn // 2, dtype=torch.uint8, device=w.device)
        scales = torch.empty(E, out * inn // 32, dtype=torch.uint8, device=w.device)
        code = load().e4b_quantize_mxfp4(_vp(w), E, out, inn, _vp(packed), _vp(scales), _stream(w))
        check("e4b_quantize_mxfp4", code)
        return QuantStack(packed, None, E, out, inn, codebook, scales)
    bf16 = codebook == "bf16"
    nbytes = out * inn * 2 if bf16 else out * inn if codebook in ("int8", "fp8") else out * inn // 2
    packed = torch.empty(E, nbytes, dtype=torch.uint8, device=w.device)
    absmax = None if bf16 else torch.empty(E, out * inn // 64, dtype=torch.float32, device=w.device)
    code = load().e4b_quantize_nf4(
        _vp(w), E, out, inn, 64, CODEBOOKS[codebook], _vp(packed), _vp(absmax), _stream(w)
    )
    check("e4b_quantize_nf4", code)
    return QuantStack(packed, absmax, E, out, inn, codebook)


def mx8_rows(x):
    """MXFP8 conversion of bf16 rows [n, K] (K % 32 == 0) as the MX forward feeds
    them to the block-scaled MFMA: (codes uint8 [n, K] with the bytes of each
    element pair swapped, E8M0 scales uint8 [n, K/32])."""
    _need(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be [n, K]")
    n, K = x.shape
    codes = torch.empty(n, K, dtype=torch.uint8, device=x.device)
    scales = torch.empty(n, max(K // 32, 1), dtype=torch.uint8, device=x.device)
    check("e4b_mx8_rows", load().e4b_mx8_rows(_vp(x), n, K, _vp(codes), _vp(scales), _stream(x)))
    return codes, scales


def dequantize(stack, dtype=torch.float32):
    """[E, out, in] device tensor of fl32(code * absmax) (or its bf16 rounding)."""
    if dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("dtype must be float32 or bfloat16")
    out = torch.empty(stack.E, stack.out, stack.inn, dtype=dtype, device=stack.device)
    st = stack.as_c()
    code = load().e4b_dequantize_nf4(
        ctypes.byref(st), _lib.E4B_BF16 if dtype == torch.bfloat16 else _lib.E4B_F32, _vp(out),
        _stream(out),
    )
    check("e4b_dequantize_nf4", code)
    return out


def workspace_bytes(layer, T, top_k):
    c = layer.as_c()
    return int(load().e4b_moe_workspace_bytes(ctypes.byref(c), T, top_k))


def saved_bytes(layer, T, top_k):
    c = layer.as_c()
    return int(load().e4b_moe_saved_bytes(ctypes.byref(c), T, top_k))


def _workspace(layer, T, top_k, ws):
    need = workspace_bytes(layer, T, top_k)
    if ws is None:
        return torch.empty(max(need, 256), dtype=torch.uint8, device=layer.device)
    _need_buffer(ws, "workspace", need, layer.device)
    return ws


def _nbytes(t):
    return t.numel() * t.element_size()


def perm_layout(layer, T, top_k):
    """Byte offsets of the routing permutation that a grouped forward without
    saved state leaves in its workspace (``e4b_moe_perm_layout``): a dict with
    counts, offsets, tile_offsets, sorted_pair, pos_of_pair, tile_map and
    m_tiles_bound."""
    c, out = layer.as_c(), E4bPermLayout()
    check("e4b_moe_perm_layout", load().e4b_moe_perm_layout(ctypes.byref(c), T, top_k, ctypes.byref(out)))
    return {name: int(getattr(out, name)) for name, _ in E4bPermLayout._fields_}


def _check_x(x, name, layer, T=None):
    _need(x, name, torch.bfloat16, layer.device)
    if x.dim() != 2 or x.shape[1] != layer.H or (T is not None and x.shape[0] != T):
        want = f"({'T' if T is None else T}, {layer.H})"
        raise ValueError(f"{name} must have shape {want}, got {tuple(x.shape)}")


def _routing(layer, T, top_k, logits, topk_idx, topk_w, check_ids):
    dev = layer.device
    if logits is not None:
        _need(logits, "logits", torch.float32, dev, (T, layer.E))
        topk_idx = torch.empty(T, top_k, dtype=torch.int32, device=dev) if topk_idx is None else topk_idx
        topk_w = torch.empty(T, top_k, dtype=torch.float32, device=dev) if topk_w is None else topk_w
    if topk_idx is None or topk_w is None:
        raise ValueError("give logits, or both topk_idx and topk_w")
    _need(topk_idx, "topk_idx", torch.int32, dev, (T, top_k))
    _need(topk_w, "topk_w", torch.float32, dev, (T, top_k))
    if logits is None and check_ids:
        check_expert_ids(topk_idx, layer.E)
    return topk_idx, topk_w


def _saved_buffer(layer, T, top_k, save):
    # never cleared: the forward writes every byte the dgrad reads
    return torch.empty(max(saved_bytes(layer, T, top_k), 16), dtype=torch.uint8,
                       device=layer.device) if save else None


def moe_forward(layer, x, top_k, logits=None, topk_idx=None, topk_w=None, save=False,
                path="auto", workspace=None, out=None, check_ids=False):
    """Routed SwiGLU expert forward.

    Either ``logits`` (float32 [T, E]: routing computed on the device) or
    ``topk_idx`` (int32 [T, k]) and ``topk_w`` (float32 [T, k]) are given.
    ``check_ids`` checks given ids against [0, E) first (one host sync).
    Returns ``(y bf16 [T, H], topk_idx, topk_w, saved or None)``.
    """
    dev = layer.device
    _check_x(x, "x", layer)
    T = x.shape[0]
    if path not in PATHS:
        raise ValueError(f"path must be one of {sorted(PATHS)}")
    topk_idx, topk_w = _routing(layer, T, top_k, logits, topk_idx, topk_w, check_ids)
    if out is None:
        y = torch.empty(T, layer.H, dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", torch.bfloat16, dev, (T, layer.H))
        y = out
    saved = _saved_buffer(layer, T, top_k, save)
    ws = _workspace(layer, T, top_k, workspace)
    c = layer.as_c()
    code = load().e4b_moe_forward(
        ctypes.byref(c), T, top_k, _vp(x), _vp(logits), _vp(topk_idx), _vp(topk_w), _vp(y),
        _vp(saved), _vp(ws), _nbytes(ws), PATHS[path], _stream(x),
    )
    check("e4b_moe_forward", code)
    return y, topk_idx, topk_w, saved


def _check_saved(layer, T, top_k, saved):
    if saved is not None:
        _need_buffer(saved, "saved", saved_bytes(layer, T, top_k), layer.device)


def moe_dgrad(layer, topk_idx, topk_w, grad_y, x=None, saved=None, grad_w=True, workspace=None,
              check_ids=False):
    """Frozen-base input gradient. Returns ``(grad_x bf16 [T, H], grad_topk_w fp32 [T, k] or None)``."""
    dev = layer.device
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [T, k]")
    T, top_k = topk_idx.shape
    _check_x(grad_y, "grad_y", layer, T)
    _need(topk_idx, "topk_idx", torch.int32, dev, (T, top_k))
    _need(topk_w, "topk_w", torch.float32, dev, (T, top_k))
    if x is not None:
        _check_x(x, "x", layer, T)
    if x is None and saved is None:
        raise ValueError("give x (recompute) or the saved state of the forward")
    _check_saved(layer, T, top_k, saved)
    if check_ids:
        check_expert_ids(topk_idx, layer.E)
    gx = torch.empty(T, layer.H, dtype=torch.bfloat16, device=dev)
    gw = torch.empty(T, top_k, dtype=torch.float32, device=dev) if grad_w else None
    ws = _workspace(layer, T, top_k, workspace)
    c = layer.as_c()
    code = load().e4b_moe_dgrad(
        ctypes.byref(c), T, top_k, _vp(topk_idx), _vp(topk_w), _vp(x), _vp(saved), _vp(grad_y),
        _vp(gx), _vp(gw), _vp(ws), _nbytes(ws), _stream(grad_y),
    )
    check("e4b_moe_dgrad", code)
    return gx, gw


@dataclass
class Lora:
    """Per-expert LoRA adapters (fp32 device tensors): A_gu [E, r, H],
    B_gu [E, 2I, r], A_dn [E, r, I], B_dn [E, H, r]; scale alpha / r."""

    A_gu: torch.Tensor
    B_gu: torch.Tensor
    A_dn: torch.Tensor
    B_dn: torch.Tensor
    alpha: float

    @property
    def r(self):
        return self.A_gu.shape[1]

    def check(self, layer):
        E, H, I, r = layer.E, layer.H, layer.I, self.r
        for name, t, shape in (("A_gu", self.A_gu, (E, r, H)), ("B_gu", self.B_gu, (E, 2 * I, r)),
                               ("A_dn", self.A_dn, (E, r, I)), ("B_dn", self.B_dn, (E, H, r))):
            _need(t, name, torch.float32, layer.device, shape)

    def as_c(self):
        return E4bLora(self.A_gu.data_ptr(), self.B_gu.data_ptr(), self.A_dn.data_ptr(),
                       self.B_dn.data_ptr(), self.r, float(self.alpha))


def lora_workspace_bytes(layer, T, top_k):
    c = layer.as_c()
    return int(load().e4b_moe_lora_workspace_bytes(ctypes.byref(c), T, top_k))


def _lora_workspace(layer, T, top_k, ws):
    need = lora_workspace_bytes(layer, T, top_k)
    if ws is None:
        return torch.empty(max(need, 256), dtype=torch.uint8, device=layer.device)
    _need_buffer(ws, "workspace", need, layer.device)
    return ws


def moe_lora_forward(layer, lora, x, top_k, logits=None, topk_idx=None, topk_w=None, save=False,
                     workspace=None, check_ids=False):
    """Forward with per-expert LoRA adapters (grouped path).

    Returns ``(y bf16 [T, H], topk_idx, topk_w, saved or None)``.
    """
    dev = layer.device
    lora.check(layer)
    _check_x(x, "x", layer)
    T = x.shape[0]
    topk_idx, topk_w = _routing(layer, T, top_k, logits, topk_idx, topk_w, check_ids)
    y = torch.empty(T, layer.H, dtype=torch.bfloat16, device=dev)
    saved = _saved_buffer(layer, T, top_k, save)
    ws = _lora_workspace(layer, T, top_k, workspace)
    c, lc = layer.as_c(), lora.as_c()
    code = load().e4b_moe_lora_forward(
        ctypes.byref(c), ctypes.byref(lc), T, top_k, _vp(x), _vp(logits), _vp(topk_idx),
        _vp(topk_w), _vp(y), _vp(saved), _vp(ws), _nbytes(ws), _stream(x),
    )
    check("e4b_moe_lora_forward", code)
    return y, topk_idx, topk_w, saved


def moe_lora_backward(layer, lora, topk_idx, topk_w, x, grad_y, saved=None, grad_w=True,
                      workspace=None, check_ids=False):
    """Input gradient, routing-weight gradient and adapter gradients.

    Returns ``(grad_x bf16 [T, H], grad_topk_w fp32 or None, (dA_gu, dB_gu, dA_dn, dB_dn))``.
    """
    dev = layer.device
    lora.check(layer)
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [T, k]")
    T, top_k = topk_idx.shape
    _check_x(grad_y, "grad_y", layer, T)
    _need(topk_idx, "topk_idx", torch.int32, dev, (T, top_k))
    _need(topk_w, "topk_w", torch.float32, dev, (T, top_k))
    _check_x(x, "x", layer, T)
    _check_saved(layer, T, top_k, saved)
    if check_ids:
        check_expert_ids(topk_idx, layer.E)
    gx = torch.empty(T, layer.H, dtype=torch.bfloat16, device=dev)
    gw = torch.empty(T, top_k, dtype=torch.float32, device=dev) if grad_w else None
    grads = tuple(torch.empty_like(t) for t in (lora.A_gu, lora.B_gu, lora.A_dn, lora.B_dn))
    ws = _lora_workspace(layer, T, top_k, workspace)
    c, lc = layer.as_c(), lora.as_c()
    code = load().e4b_moe_lora_backward(
        ctypes.byref(c), ctypes.byref(lc), T, top_k, _vp(topk_idx), _vp(topk_w), _vp(x),
        _vp(saved), _vp(grad_y), _vp(gx), _vp(gw), *(_vp(g) for g in grads), _vp(ws), _nbytes(ws),
        _stream(grad_y),
    )
    check("e4b_moe_lora_backward", code)
    return gx, gw, grads


def _empty_like_on(t, device):
    return None if t is None else torch.empty(t.shape, dtype=t.dtype, device=device)


class LayerPrefetcher:
    """Layer-granular prefetch of stored layers kept in pinned host memory.

    Two device slots used in turn: ``prefetch(l)`` copies layer ``l`` into
    the next slot on a side stream (``e4b_stack_copy_async``) once the
    compute that last used that slot has finished; ``acquire(l)`` makes the
    current stream wait for the copy and returns the device layer;
    ``release(l)`` marks its slot free after the layer's kernels have been
    enqueued on the current stream. Layers are acquired in prefetch order and
    at most two are resident. (The 0.4.0 README's "Prefetched expert
    offload" bullet: layer L+1 copies on a side stream while layer L
    computes.)
    """

    def __init__(self, host_layers, device="cuda"):
        if not host_layers:
            raise ValueError("no layers")
        self.host = host_layers
        dev = torch.device(device)
        ref = host_layers[0]
        self.slots = []
        for _ in range(2):
            stacks = [QuantStack(_empty_like_on(st.packed, dev), _empty_like_on(st.absmax, dev),
                                 st.E, st.out, st.inn, st.codebook, _empty_like_on(st.scales, dev))
                      for st in (ref.gate_up, ref.down)]
            self.slots.append(MoELayer(*stacks))
        self.stream = torch.cuda.Stream(device=dev)  # default priority
        self.ready = [torch.cuda.Event() for _ in range(2)]
        self.free = [torch.cuda.Event() for _ in range(2)]
        for ev in self.free:
            ev.record(torch.cuda.current_stream(dev))
        self.next_slot = 0
        self.queue = []  # (layer, slot) in prefetch order

    def prefetch(self, l):
        if len(self.queue) == 2:
            raise RuntimeError("both slots are in use: release a layer first")
        s = self.next_slot
        self.next_slot ^= 1
        slot, src = self.slots[s], self.host[l]
        self.stream.wait_event(self.free[s])
        handle = ctypes.c_void_p(self.stream.cuda_stream)
        for dst, st in ((slot.gate_up, src.gate_up), (slot.down, src.down)):
            d, c = dst.as_c(), st.as_c()
            check("e4b_stack_copy_async",
                  load().e4b_stack_copy_async(ctypes.byref(d), ctypes.byref(c), handle))
        self.ready[s].record(self.stream)
        self.queue.append((l, s))

    def acquire(self, l):
        if not self.queue or self.queue[0][0] != l:
            raise RuntimeError(f"layer {l} is not the next prefetched layer")
        s = self.queue[0][1]
        torch.cuda.current_stream().wait_event(self.ready[s])
        return self.slots[s]

    def release(self, l):
        if not self.queue or self.queue[0][0] != l:
            raise RuntimeError(f"layer {l} is not the acquired layer")
        _, s = self.queue.pop(0)
        self.free[s].record(torch.cuda.current_stream())

"""C-ABI checks that need no GPU: the library loads, exports every symbol that
include/e4b.h declares, and every host-side validation error is reported
synchronously (no device pointer is touched on these paths)."""

import ctypes
import os
import re

import pytest

import bit_quantized_mixture_nf4_amd as e4b
from bit_quantized_mixture_nf4_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # a 16-byte-aligned non-null address; never dereferenced on these paths


def _declared():
    src = open(os.path.join(ROOT, "include", "e4b.h")).read()
    return sorted(set(re.findall(r"\b(e4b_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = e4b.load()
    names = _declared()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def _stack(E=4, out=128, inn=64, packed=FAKE, absmax=FAKE, bs=64, cb=0, scales=None):
    return _lib.E4bStack(packed, absmax, E, out, inn, bs, cb, scales)


def _layer(E=4, H=64, I=64, **kw):
    return _lib.E4bLayer(_stack(E, 2 * I, H, **kw), _stack(E, H, I, **kw))


def _fwd(L, T=4, k=2, x=FAKE, logits=None, idx=FAKE, w=FAKE, y=FAKE, saved=None, ws=FAKE,
         ws_bytes=1 << 40, path=0):
    return e4b.load().e4b_moe_forward(ctypes.byref(L), T, k, x, logits, idx, w, y, saved, ws,
                                      ws_bytes, path, None)


def _dgrad(L, T=4, k=2, idx=FAKE, w=FAKE, x=FAKE, saved=None, gy=FAKE, gx=FAKE, gw=FAKE,
           ws=FAKE, ws_bytes=1 << 40):
    return e4b.load().e4b_moe_dgrad(ctypes.byref(L), T, k, idx, w, x, saved, gy, gx, gw, ws,
                                    ws_bytes, None)


def test_quantize_validation():
    q = e4b.load().e4b_quantize_nf4
    assert q(None, 1, 64, 64, 64, 0, FAKE, FAKE, None) == _lib.E4B_ERR_NULL
    assert q(FAKE, 1, 64, 64, 64, 0, None, FAKE, None) == _lib.E4B_ERR_NULL
    assert q(FAKE, 1, 64, 96, 64, 0, FAKE, FAKE, None) == _lib.E4B_ERR_SHAPE
    assert q(FAKE, 0, 64, 64, 64, 0, FAKE, FAKE, None) == _lib.E4B_ERR_SHAPE
    assert q(FAKE, 1, 64, 64, 128, 0, FAKE, FAKE, None) == _lib.E4B_ERR_BLOCKSIZE
    assert q(FAKE, 1, 64, 64, 64, 6, FAKE, FAKE, None) == _lib.E4B_ERR_CODEBOOK
    assert q(FAKE, 1, 64, 64, 64, -1, FAKE, FAKE, None) == _lib.E4B_ERR_CODEBOOK
    # the 8-bit lanes need an absmax buffer like the 4-bit ones
    assert q(FAKE, 1, 64, 64, 64, _lib.E4B_CB_INT8, FAKE, None, None) == _lib.E4B_ERR_NULL
    assert q(FAKE, 1, 64, 64, 128, _lib.E4B_CB_FP8, FAKE, FAKE, None) == _lib.E4B_ERR_BLOCKSIZE
    # MXFP4 has its own entry point (E8M0 scale bytes, not fp32 absmax)
    assert q(FAKE, 1, 64, 64, 64, 3, FAKE, FAKE, None) == _lib.E4B_ERR_CODEBOOK
    # the bf16 lane needs no absmax buffer: NULL passes the pointer check and
    # the call stops at the next check (nothing is launched)
    assert q(FAKE, 1, 64, 64, 128, 2, FAKE, None, None) == _lib.E4B_ERR_BLOCKSIZE
    assert q(FAKE + 4, 1, 64, 64, 64, 0, FAKE, FAKE, None) == _lib.E4B_ERR_ALIGN


def test_dequantize_validation():
    d = e4b.load().e4b_dequantize_nf4
    st = _stack()
    assert d(ctypes.byref(st), 0, None, None) == _lib.E4B_ERR_NULL
    assert d(ctypes.byref(st), 7, FAKE, None) == _lib.E4B_ERR_DTYPE
    assert d(ctypes.byref(st), 0, FAKE + 8, None) == _lib.E4B_ERR_ALIGN
    assert d(ctypes.byref(_stack(bs=32)), 0, FAKE, None) == _lib.E4B_ERR_BLOCKSIZE
    assert d(ctypes.byref(_stack(cb=6)), 0, FAKE, None) == _lib.E4B_ERR_CODEBOOK
    assert d(ctypes.byref(_stack(inn=100)), 0, FAKE, None) == _lib.E4B_ERR_SHAPE
    assert d(ctypes.byref(_stack(packed=None)), 0, FAKE, None) == _lib.E4B_ERR_NULL
    assert d(None, 0, FAKE, None) == _lib.E4B_ERR_NULL


def test_layer_validation():
    L = _layer()
    bad_cb = _lib.E4bLayer(_stack(4, 128, 64, cb=0), _stack(4, 64, 64, cb=1))
    assert _fwd(bad_cb) == _lib.E4B_ERR_CODEBOOK
    bad_shape = _lib.E4bLayer(_stack(4, 130, 64), _stack(4, 64, 64))
    assert _fwd(bad_shape) == _lib.E4B_ERR_SHAPE
    bad_e = _lib.E4bLayer(_stack(4, 128, 64), _stack(5, 64, 64))
    assert _fwd(bad_e) == _lib.E4B_ERR_SHAPE
    big_e = _layer(E=2048)
    assert _fwd(big_e) == _lib.E4B_ERR_SHAPE
    assert _fwd(L, k=0) == _lib.E4B_ERR_SHAPE
    assert _fwd(L, k=5) == _lib.E4B_ERR_SHAPE  # top_k > E
    assert _fwd(L, T=-1) == _lib.E4B_ERR_SHAPE
    assert e4b.load().e4b_moe_forward(None, 4, 2, FAKE, None, FAKE, FAKE, FAKE, None, FAKE,
                                      1 << 40, 0, None) == _lib.E4B_ERR_NULL


def test_forward_and_dgrad_argument_errors():
    L = _layer()
    need = e4b.load().e4b_moe_workspace_bytes(ctypes.byref(L), 4, 2)
    assert need > 0
    assert _fwd(L, x=None) == _lib.E4B_ERR_NULL
    assert _fwd(L, y=None) == _lib.E4B_ERR_NULL
    assert _fwd(L, ws=None) == _lib.E4B_ERR_NULL
    assert _fwd(L, ws_bytes=need - 1) == _lib.E4B_ERR_WORKSPACE
    assert _fwd(L, x=FAKE + 2) == _lib.E4B_ERR_ALIGN
    assert _fwd(L, logits=FAKE + 4) == _lib.E4B_ERR_ALIGN
    assert _fwd(L, path=3) == _lib.E4B_ERR_PATH
    assert _fwd(L, T=9, path=2) == _lib.E4B_ERR_PATH  # decode path needs T <= 8
    assert _fwd(L, T=4, path=2, saved=FAKE) == _lib.E4B_ERR_PATH
    big = _layer(E=4, H=32768, I=64)
    assert _fwd(big, T=8, path=2) == _lib.E4B_ERR_PATH  # decode path needs max(H, I) <= 16384
    assert _dgrad(L, gy=None) == _lib.E4B_ERR_NULL
    assert _dgrad(L, x=None, saved=None) == _lib.E4B_ERR_NULL
    assert _dgrad(L, ws_bytes=need - 1) == _lib.E4B_ERR_WORKSPACE
    assert _dgrad(L, gw=FAKE + 4) == _lib.E4B_ERR_ALIGN


def test_zero_tokens_is_a_noop():
    L = _layer()
    assert _fwd(L, T=0, x=None, idx=None, w=None, y=None, ws=None, ws_bytes=0) == _lib.E4B_OK
    assert _dgrad(L, T=0, idx=None, w=None, x=None, gy=None, gx=None, gw=None, ws=None,
                  ws_bytes=0) == _lib.E4B_OK


@pytest.mark.parametrize("E,H,I,k,T", [(8, 256, 128, 2, 64), (64, 2048, 1024, 8, 4096),
                                       (128, 2048, 768, 8, 16384), (8, 4096, 14336, 2, 8192)])
def test_workspace_and_saved_sizes(E, H, I, k, T):
    L = _layer(E=E, H=H, I=I)
    lib = e4b.load()
    P = T * k
    saved = lib.e4b_moe_saved_bytes(ctypes.byref(L), T, k)
    # bf16 g|u in blocks of 256 rows x 128 pairs (g and u) per m-tile (at most
    # P / 256 + min(E, P) tiles of 256 pairs), then the permutation: an int4 per
    # m-tile, offsets and tile offsets over E + 1 experts, sorted pairs and
    # pair positions; then the LoRA forward's two fp32 [P, 16] rank projections
    m_tiles = (P + min(E, P) * 255) // 256
    gu = m_tiles * -(-I // 128) * 256 * 128 * 2 * 2
    perm_end = -(-gu // 256) * 256 + 16 * m_tiles + 8 * (E + 1) + 8 * P
    assert saved == -(-perm_end // 256) * 256 + 2 * P * 16 * 4
    ws = lib.e4b_moe_workspace_bytes(ctypes.byref(L), T, k)
    # at least the dgrad intermediates: g|u, dGU, grad_x rows
    assert ws >= P * (2 * I * 2 * 2 + H * 2)
    assert lib.e4b_moe_workspace_bytes(ctypes.byref(L), T, E + 1) == 0


def test_status_strings():
    for code in range(10):
        assert len(_lib.status_string(code)) > 0


def _lora(r=8, a=FAKE):
    return _lib.E4bLora(a, FAKE, FAKE, FAKE, r, 16.0)


def test_lora_argument_errors():
    L = _layer()
    lib = e4b.load()
    need = lib.e4b_moe_lora_workspace_bytes(ctypes.byref(L), 4, 2)
    assert need > lib.e4b_moe_workspace_bytes(ctypes.byref(L), 4, 2)

    def fwd(lo, ws_bytes=1 << 40, T=4, x=FAKE):
        return lib.e4b_moe_lora_forward(ctypes.byref(L), lo, T, 2, x, None, FAKE, FAKE, FAKE,
                                        None, FAKE, ws_bytes, None)

    def bwd(lo, ws_bytes=1 << 40, T=4, x=FAKE, dA=FAKE):
        return lib.e4b_moe_lora_backward(ctypes.byref(L), lo, T, 2, FAKE, FAKE, x, None, FAKE,
                                         FAKE, FAKE, dA, FAKE, FAKE, FAKE, FAKE, ws_bytes, None)

    for call in (fwd, bwd):
        assert call(None) == _lib.E4B_ERR_NULL
        assert call(ctypes.byref(_lora(a=None))) == _lib.E4B_ERR_NULL
        assert call(ctypes.byref(_lora(r=0))) == _lib.E4B_ERR_SHAPE
        assert call(ctypes.byref(_lora(r=17))) == _lib.E4B_ERR_SHAPE
        assert call(ctypes.byref(_lora(a=FAKE + 4))) == _lib.E4B_ERR_ALIGN
        assert call(ctypes.byref(_lora()), ws_bytes=need - 1) == _lib.E4B_ERR_WORKSPACE
        assert call(ctypes.byref(_lora()), T=0, x=None) == _lib.E4B_OK
    assert bwd(ctypes.byref(_lora()), x=None) == _lib.E4B_ERR_NULL
    assert bwd(ctypes.byref(_lora()), dA=None) == _lib.E4B_ERR_NULL
    assert bwd(ctypes.byref(_lora()), dA=FAKE + 4) == _lib.E4B_ERR_ALIGN


def test_bf16_lane_validation():
    bf = _lib.E4bLayer(_stack(4, 128, 64, absmax=None, cb=2), _stack(4, 64, 64, absmax=None, cb=2))
    # absmax may be NULL; the layer gets as far as the workspace check
    assert _fwd(bf, ws_bytes=0) == _lib.E4B_ERR_WORKSPACE
    # the decode GEMV reads 4-bit codes: a bf16 layer takes the grouped path only
    assert _fwd(bf, T=4, path=2) == _lib.E4B_ERR_PATH
    # a 4-bit stack still needs its absmax
    nf = _lib.E4bLayer(_stack(4, 128, 64, absmax=None), _stack(4, 64, 64))
    assert _fwd(nf) == _lib.E4B_ERR_NULL
    mixed = _lib.E4bLayer(_stack(4, 128, 64, cb=2), _stack(4, 64, 64, cb=0))
    assert _fwd(mixed) == _lib.E4B_ERR_CODEBOOK


def test_8bit_lane_validation():
    for cb in (_lib.E4B_CB_INT8, _lib.E4B_CB_FP8):
        L = _lib.E4bLayer(_stack(4, 128, 64, cb=cb), _stack(4, 64, 64, cb=cb))
        # the call reaches the workspace check; the GEMMs decode the code bytes
        # themselves, so the workspace is that of a 4-bit layer
        assert _fwd(L, ws_bytes=0) == _lib.E4B_ERR_WORKSPACE
        nf4 = _lib.E4bLayer(_stack(4, 128, 64), _stack(4, 64, 64))
        lib = e4b.load()
        w8 = lib.e4b_moe_workspace_bytes(ctypes.byref(L), 4, 2)
        w4 = lib.e4b_moe_workspace_bytes(ctypes.byref(nf4), 4, 2)
        assert w8 == w4
        # no GEMV for the 8-bit lanes: the decode path is refused
        assert _fwd(L, T=4, path=2) == _lib.E4B_ERR_PATH
        # the 8-bit stacks need their absmax
        bad = _lib.E4bLayer(_stack(4, 128, 64, absmax=None, cb=cb), _stack(4, 64, 64, cb=cb))
        assert _fwd(bad) == _lib.E4B_ERR_NULL


def test_ungated_layer_validation():
    ug = _lib.E4bLayer(_stack(4, 64, 64), _stack(4, 64, 64))  # gate_up out = I: has_gate=False
    assert _fwd(ug, ws_bytes=0) == _lib.E4B_ERR_WORKSPACE  # accepted up to the workspace check
    assert _fwd(ug, T=4, path=2) == _lib.E4B_ERR_PATH     # decode GEMV is for gated layers
    bad = _lib.E4bLayer(_stack(4, 96, 64), _stack(4, 64, 64))
    assert _fwd(bad) == _lib.E4B_ERR_SHAPE
    lib = e4b.load()
    lo = _lib.E4bLora(FAKE, FAKE, FAKE, FAKE, 8, 16.0)
    assert lib.e4b_moe_lora_forward(ctypes.byref(ug), ctypes.byref(lo), 4, 2, FAKE, None, FAKE,
                                    FAKE, FAKE, None, FAKE, 1 << 40, None) == _lib.E4B_ERR_SHAPE


def test_stack_copy_validation():
    cp = e4b.load().e4b_stack_copy_async
    a, b = _stack(4, 128, 64), _stack(4, 128, 128)
    assert cp(ctypes.byref(a), ctypes.byref(b), None) == _lib.E4B_ERR_SHAPE
    assert cp(ctypes.byref(a), ctypes.byref(_stack(4, 128, 64, cb=1)), None) == _lib.E4B_ERR_SHAPE
    assert cp(ctypes.byref(_stack(packed=None)), ctypes.byref(a), None) == _lib.E4B_ERR_NULL
    assert cp(None, ctypes.byref(a), None) == _lib.E4B_ERR_NULL


def test_mxfp4_validation():
    lib = e4b.load()
    q = lib.e4b_quantize_mxfp4
    assert q(None, 1, 64, 64, FAKE, FAKE, None) == _lib.E4B_ERR_NULL
    assert q(FAKE, 1, 64, 64, FAKE, None, None) == _lib.E4B_ERR_NULL
    assert q(FAKE, 1, 64, 48, FAKE, FAKE, None) == _lib.E4B_ERR_SHAPE  # in % 32
    assert q(FAKE, 0, 64, 64, FAKE, FAKE, None) == _lib.E4B_ERR_SHAPE
    assert q(FAKE, 1, 64, 64, FAKE, FAKE + 1, None) == _lib.E4B_ERR_ALIGN

    def mx(out, inn, bs=32, scales=FAKE, absmax=None):
        return _stack(4, out, inn, absmax=absmax, bs=bs, cb=3, scales=scales)

    d = lib.e4b_dequantize_nf4
    assert d(ctypes.byref(mx(128, 64, bs=64)), 0, FAKE, None) == _lib.E4B_ERR_BLOCKSIZE
    assert d(ctypes.byref(mx(128, 64, scales=None)), 0, FAKE, None) == _lib.E4B_ERR_NULL
    assert d(ctypes.byref(mx(128, 96)), 0, FAKE, None) == _lib.E4B_ERR_SHAPE  # rows of 64
    assert d(ctypes.byref(mx(128, 64, scales=FAKE + 8)), 0, FAKE, None) == _lib.E4B_ERR_ALIGN
    # a valid MXFP4 layer (absmax unused, NULL) gets as far as the workspace check
    L = _lib.E4bLayer(mx(128, 64), mx(64, 64))
    assert _fwd(L, ws_bytes=0) == _lib.E4B_ERR_WORKSPACE
    assert _dgrad(L, ws_bytes=0) == _lib.E4B_ERR_WORKSPACE
    mixed = _lib.E4bLayer(mx(128, 64), _stack(4, 64, 64))
    assert _fwd(mixed) == _lib.E4B_ERR_CODEBOOK
    # the MX forward (path 3): MXFP4 only, H and I multiples of 128, no saved state
    assert _fwd(_layer(), path=3) == _lib.E4B_ERR_PATH
    assert _fwd(L, path=3) == _lib.E4B_ERR_PATH  # H = I = 64
    L128 = _lib.E4bLayer(mx(256, 128), mx(128, 128))
    assert _fwd(L128, path=3, ws_bytes=0) == _lib.E4B_ERR_WORKSPACE
    assert _fwd(L128, path=3, saved=FAKE) == _lib.E4B_ERR_PATH
    r = lib.e4b_mx8_rows
    assert r(None, 4, 64, FAKE, FAKE, None) == _lib.E4B_ERR_NULL
    assert r(FAKE, 4, 48, FAKE, FAKE, None) == _lib.E4B_ERR_SHAPE
    assert r(FAKE + 2, 4, 64, FAKE, FAKE, None) == _lib.E4B_ERR_ALIGN
